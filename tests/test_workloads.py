"""The seeded input generators, on the CPU: the device-side draw of full
pools follows the same quantization recipes as the numpy generators, and
gives every expert its own bytes."""
import numpy as np
import torch

from expert_slot_cache_moe_amd import workloads as W


def _weights(seed, shape):
    g = np.random.default_rng(seed)
    w = g.standard_normal(shape).astype(np.float32) * np.float32(0.02)
    w[0, :32] = 0.0                       # an all-zero block (scale 0)
    w[1, 7] = 1e-30                       # a tiny value next to normal ones
    w[2, :16] = np.float32(0.02) * np.arange(16)   # exact ties between E2M1 neighbours
    return w


def test_torch_quantizers_follow_the_numpy_recipes():
    for seed in range(3):
        w = _weights(seed, (48, 256))
        for f_np, f_t in ((W._quantize_e2m1, W._quantize_e2m1_torch),
                          (W._quantize_mxfp4, W._quantize_mxfp4_torch)):
            a = f_np(w)
            b = f_t(torch.from_numpy(w))
            for x, y in zip(a, b):
                np.testing.assert_array_equal(x, y.numpy())


def test_device_pools_have_no_two_experts_alike():
    for fmt, nb in ((0, 2), (1, 6), (2, 4)):
        banks = W.device_expert_rows(fmt, 3, 24, 64, 64, device="cpu")
        assert len(banks) == nb
        rows = np.concatenate([b.numpy() for b in banks], 1)
        assert len({r.tobytes() for r in rows}) == 24
        again = W.device_expert_rows(fmt, 3, 24, 64, 64, device="cpu")
        assert all(torch.equal(a, b) for a, b in zip(banks, again))     # seeded
        if fmt == 1:
            for mat in (0, 1):
                glob = banks[3 * mat + 2].numpy().view(np.float32).reshape(-1)
                np.testing.assert_array_equal(glob, W.e2m1_global_scales(24, mat))
                assert len(set(glob.tolist())) == 24


def test_device_bf16_pool_is_normal_with_the_stated_spread():
    w13, w2 = W.device_expert_rows(0, 5, 4, 256, 128, device="cpu")
    v = w13.view(torch.bfloat16).float().numpy()
    assert abs(v.std() - 0.02) < 5e-4 and abs(v.mean()) < 5e-4
