"""The single-token layer step against the non-cached streamed layer, bit
for bit.

FreeToken PR #680, section Tests: the GEMV over the cache's slots equals
the GEMV over the streamed layer exactly.  Here the whole layer step
(moe_layer_decode: top-k, admission, miss gather, shared expert, routed
experts, combine) runs over the slot cache in each of the four schedules,
on steps that fetch; its output must equal moe_routed_decode over the
layer's whole expert set in device memory (pool rows = expert ids), given
the same routes, weights and gated shared term, byte for byte.  In the
one-token schedules a fetched expert's gate/up dots are taken inside the
gather's workgroups, a different code path from the streamed pool's.

Every expert's bytes are drawn afresh (no two experts alike, E2M1 global
scales distinct per expert), so a read of the wrong slot cannot pass."""
import numpy as np
import pytest
import torch

import expert_slot_cache_moe_amd as m
from expert_slot_cache_moe_amd import workloads as W
from expert_slot_cache_moe_amd.layer import SlotCacheLayers
import oracle
from parity import check_close

pytestmark = pytest.mark.gpu

# (name, layers, experts, slots, hidden, ffn, top-k, tokens): the Tiny decode
# config (+ a shared expert of the routed width) and the shared-expert decode
# shape over fewer experts and a small cache, so that most steps fetch.
SHAPES = {
    "tiny": (1, 8, 4, 64, 128, 2, 24),
    "c3": (2, 48, 20, 2048, 512, 8, 5),
}


def _stack(fmt, shape, overlap, seed):
    L, E, S, H, F, K, _ = SHAPES[shape]
    host = []
    for l in range(L):
        dev = W.device_expert_rows(fmt, (seed, l), E, H, F)
        host.append([W.pinned_copy(b) for b in dev])
        del dev
    g = W.rng(seed, "streamed", "shared", shape)
    sh = [(W.normal_bf16(g, 2 * F * H, 0.02), W.normal_bf16(g, H * F, 0.02), W.normal_bf16(g, H, 0.02))
          for _ in range(L)]
    lay = SlotCacheLayers(layers=L, experts=E, slots=S, hidden=H, ffn=F, fmt=fmt, host_rows=host,
                          shared=sh, max_tokens=1, max_top_k=K, overlap=overlap)
    return lay, sh


@pytest.mark.parametrize("overlap", [0, 1, 2, 3])
@pytest.mark.parametrize("fmt", [0, 1, 2])
@pytest.mark.parametrize("shape", ["tiny", "c3"])
def test_single_token_layer_step_equals_the_streamed_layer(shape, fmt, overlap):
    L, E, S, H, F, K, tokens = SHAPES[shape]
    seed = 40 + fmt
    print(f"shape {shape} fmt {fmt} overlap {overlap}", flush=True)
    lay, sh = _stack(fmt, shape, overlap, seed)
    g = W.rng(seed, "streamed", "steps", shape)
    streamed = [lay.streamed_pool(l) for l in range(L)]
    out = torch.empty((1, H), dtype=torch.int16, device="cuda")
    ref_out = torch.empty_like(out)
    ids = torch.empty((1, K), dtype=torch.int32, device="cuda")
    w = torch.empty((1, K), dtype=torch.float32, device="cuda")
    add = torch.empty((1, H), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(m.moe_routed_workspace_bytes(fmt, H, F, 1, K),
                         m.moe_routed_workspace_bytes(0, H, F, 1, 1)), dtype=torch.uint8, device="cuda")
    oc = oracle.OracleCache(L, E, S)
    fetching_steps = 0
    try:
        for t in range(tokens):
            for l in range(L):
                x = torch.from_numpy(W.normal_bf16(g, (1, H)).view(np.int16)).cuda()
                lg = W.zipf_logits(g, 1, E, 0.6)
                before = m.moe_cache_stats(lay.cache, l)
                lay.decode(l, x, torch.from_numpy(lg).cuda(), K, out, ids_out=ids, w_out=w)
                torch.cuda.synchronize()
                fetched = int(m.moe_cache_stats(lay.cache, l)[2] - before[2])
                fetching_steps += fetched > 0
                own = m.moe_cache_read_state(lay.cache)["own"]
                slots = ids.cpu().numpy()
                assert (slots >= 0).all()                      # no cap: every route is resident
                experts = (own[slots] - l * E).astype(np.int32)
                # the non-cached layer: the same kernels over the layer's experts,
                # rows = expert ids, with the gated shared term as the addend
                m.moe_shared_expert(lay.shared[l], H, x, add, ws)
                m.moe_routed_decode(streamed[l], x, torch.from_numpy(experts).cuda(), w, ref_out, ws,
                                    addend=add)
                torch.cuda.synchronize()
                assert torch.equal(out, ref_out), f"token {t} layer {l} (fetched {fetched})"
                # and the oracle: admission exact, output within tolerance
                e_ids, wts = oracle.topk(lg, K)
                np.testing.assert_array_equal(oc.admit(l, e_ids.reshape(-1)).reshape(1, K), slots)
                np.testing.assert_array_equal(np.sort(experts, 1), np.sort(e_ids, 1))
                if t < 2:
                    _, o_add = oracle.shared(H, F, *sh[l], x.cpu().numpy().view(np.uint16))
                    pool = oracle.Pool(fmt, H, F, [b.numpy() for b in lay.host[l]])
                    ref = oracle.routed(pool, e_ids, wts, x.cpu().numpy().view(np.uint16), addend=o_add)
                    check_close(out.view(torch.bfloat16).double().cpu().numpy(), ref, f"token {t} layer {l}")
        assert fetching_steps >= L * tokens // 3, fetching_steps
    finally:
        lay.close()
