"""moe_routed_decode_noalloc, the allocation-free routed decode: the same
results as moe_routed_decode, bit for bit, on two calls in a row whose
second is smaller (the library's scratch keeps the first call's contents),
for the single-token and the grouped paths in every weight format; sizes
beyond its scratch are refused on the host."""
import numpy as np
import pytest
import torch

import expert_slot_cache_moe_amd as m
from expert_slot_cache_moe_amd import workloads as W

pytestmark = pytest.mark.gpu


def _pool(fmt, rows, H, F, seed):
    banks = W.device_expert_rows(fmt, (seed, "noalloc"), rows, H, F)
    return banks, m.make_pool(fmt, H, F, rows, banks)


def _inputs(g, rows, H, T, K):
    x = torch.from_numpy(W.normal_bf16(g, (T, H)).view(np.int16)).cuda()
    idx = np.stack([g.choice(rows, K, replace=False) for _ in range(T)]).astype(np.int32)
    idx[g.random((T, K)) < 0.1] = -1
    w = torch.from_numpy(g.random((T, K)).astype(np.float32)).cuda()
    add = torch.from_numpy((g.standard_normal((T, H)) * 0.01).astype(np.float32)).cuda()
    return x, torch.from_numpy(idx).cuda(), w, add


@pytest.mark.parametrize("fmt", [0, 1, 2])
@pytest.mark.parametrize("H,F,rows,first,second", [
    (2048, 512, 24, (1, 8), (1, 4)),        # one token (the two stage launches), then fewer routes
    (1024, 256, 160, (600, 2), (150, 2)),   # a wide step (grouping + MFMA), then a smaller one
    (1024, 256, 160, (300, 2), (1, 2)),     # a wide step, then one token
])
def test_noalloc_equals_routed_decode_on_two_calls(fmt, H, F, rows, first, second):
    print(f"noalloc fmt {fmt} H {H} F {F} rows {rows} calls {first} then {second}", flush=True)
    g = W.rng(61, "noalloc", fmt, H, first)
    _, pool = _pool(fmt, rows, H, F, 61)
    for T, K in (first, second):
        x, idx, w, add = _inputs(g, rows, H, T, K)
        ref = torch.empty((T, H), dtype=torch.int16, device="cuda")
        ws = torch.empty(m.moe_routed_workspace_bytes(fmt, H, F, T, K), dtype=torch.uint8, device="cuda")
        m.moe_routed_decode(pool, x, idx, w, ref, ws, addend=add)
        out = torch.full((T, H), 0x7fc0, dtype=torch.int16, device="cuda")
        m.moe_routed_decode_noalloc(pool, x, idx, w, out, addend=add)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), (T, K)
        assert not torch.isnan(out.view(torch.bfloat16).float()).any()


def test_noalloc_refuses_steps_beyond_its_scratch():
    H, F, T, K = 4096, 1024, 1000, 8
    assert m.moe_routed_workspace_bytes(0, H, F, T, K) > m.MOE_NOALLOC_SCRATCH_BYTES
    banks = [torch.zeros((2, 4 * F * H), dtype=torch.uint8, device="cuda"),
             torch.zeros((2, 2 * H * F), dtype=torch.uint8, device="cuda")]
    pool = m.make_pool(0, H, F, 2, banks)
    x = torch.zeros((T, H), dtype=torch.int16, device="cuda")
    idx = torch.zeros((T, K), dtype=torch.int32, device="cuda")
    w = torch.zeros((T, K), dtype=torch.float32, device="cuda")
    out = torch.full((T, H), 7, dtype=torch.int16, device="cuda")
    with pytest.raises(m.MoeError) as e:
        m.moe_routed_decode_noalloc(pool, x, idx, w, out)
    assert e.value.status == m.MOE_INVALID_ARG and "workspace" in m.moe_last_error()
    torch.cuda.synchronize()
    assert (out == 7).all()                   # refused before any launch
