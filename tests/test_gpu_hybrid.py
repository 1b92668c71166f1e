"""The hybrid decode step (FreeToken PR #491, sections 4-5) vs the oracle:
routes the capped admission leaves at -1 run on host cores, the rest on
the GPU, and the partials are added.

Slot ids (with -1 for the CPU routes), the slot map and the statistics must
match the oracle exactly; outputs must match the oracle's full layer (every
route, plus the gated shared term) within max |gpu - oracle| <= 2e-2 * max
|oracle|.  With no CPU route the step must equal moe_layer_decode bit for
bit."""
import numpy as np
import pytest
import torch

import expert_slot_cache_moe_amd as m
from expert_slot_cache_moe_amd import workloads as W
from expert_slot_cache_moe_amd.layer import SlotCacheLayers
import oracle
from parity import check_close

pytestmark = pytest.mark.gpu



def _dev_u16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def _layers(seed, L, E, S, H, F, T, K, overlap, shared=True, fmt=0):
    g = W.rng(seed, "hybrid", L, E, H, T, fmt)
    host = [W.expert_rows(fmt, g, E, H, F) for _ in range(L)]
    sh = None
    if shared:
        sh = [(W.normal_bf16(g, 2 * F * H, 0.02), W.normal_bf16(g, H * F, 0.02), W.normal_bf16(g, H, 0.02))
              for _ in range(L)]
    lay = SlotCacheLayers(layers=L, experts=E, slots=S, hidden=H, ffn=F, fmt=fmt, host_rows=host, shared=sh,
                          max_tokens=T, max_top_k=K, overlap=overlap)
    return lay, host, sh, g


@pytest.mark.parametrize("overlap,T,max_fetch,shared,fmt", [
    (2, 1, 0, True, 0),       # every miss on the CPU, overlapped
    (0, 1, 0, True, 0),       # the serial debug order
    (1, 1, 1, True, 0),       # one fetch per step, the rest on the CPU
    (2, 5, 1, True, 0),       # a small batch (grouped GPU path)
    (2, 3, 0, False, 0),      # no shared expert: the CPU partial alone is the added term
    (3, 1, 1, True, 0),       # schedule 3 (the hybrid step overlaps the CPU half)
    (2, 1, 0, True, 1),       # E2M1 experts (E4M3 per-16 scales) on both halves
    (2, 5, 1, True, 2),       # MXFP4 experts, a small batch
])
def test_hybrid_steps_match_the_oracle(overlap, T, max_fetch, shared, fmt):
    L, E, S, H, F, K = 2, 16, 6, 64, 128, 2
    lay, host, sh, g = _layers(51, L, E, S, H, F, T, K, overlap, shared, fmt)
    m.moe_cache_set_cpu_threads(lay.cache, 4)
    oc = oracle.OracleCache(L, E, S)
    out = torch.empty((T, H), dtype=torch.int16, device="cuda")
    ids = torch.empty((T, K), dtype=torch.int32, device="cuda")
    cpu_routes = 0
    try:
        for step in range(14):
            for l in range(L):
                x = W.normal_bf16(g, (T, H))
                lg = W.zipf_logits(g, T, E, 0.6)
                lay.decode_hybrid(l, _dev_u16(x), torch.from_numpy(lg).cuda(), K, out, ids_out=ids,
                                  max_fetch=max_fetch)
                ids_e, w = oracle.topk(lg, K)
                slots = oc.admit(l, ids_e.reshape(-1), max_fetch).reshape(T, K)
                add = None
                if shared:
                    _, add = oracle.shared(H, F, sh[l][0], sh[l][1], sh[l][2], x)
                ref = oracle.routed(oracle.Pool(fmt, H, F, host[l]), ids_e, w, x, addend=add)
                torch.cuda.synchronize()
                np.testing.assert_array_equal(ids.cpu().numpy(), slots, err_msg=f"step {step} layer {l}")
                got = out.view(torch.bfloat16).double().cpu().numpy()
                check_close(got, ref, f"step {step} layer {l}")
                cpu_routes += int((slots < 0).sum())
        st = m.moe_cache_read_state(lay.cache)
        o = oc.state()
        for k in ("res", "own", "stamp", "stats", "freq", "dlast"):
            np.testing.assert_array_equal(st[k].reshape(o[k].shape), o[k], err_msg=k)
        assert cpu_routes > 5        # the steps did send routes to the CPU
    finally:
        lay.close()


def test_hybrid_with_no_cpu_route_equals_the_layer_step():
    L, E, S, H, F, K, T = 2, 16, 16, 64, 128, 2, 1
    a, host, sh, g = _layers(52, L, E, S, H, F, T, K, 0)
    b = SlotCacheLayers(layers=L, experts=E, slots=S, hidden=H, ffn=F, host_rows=host, shared=sh,
                        max_tokens=T, max_top_k=K, overlap=0)
    m.moe_cache_set_cpu_threads(a.cache, 3)
    outs = [torch.empty((T, H), dtype=torch.int16, device="cuda") for _ in range(2)]
    try:
        for step in range(10):
            for l in range(L):
                x = _dev_u16(W.normal_bf16(g, (T, H)))
                lg = torch.from_numpy(W.zipf_logits(g, T, E, 0.6)).cuda()
                a.decode_hybrid(l, x, lg, K, outs[0])
                b.decode(l, x, lg, K, outs[1])
                torch.cuda.synchronize()
                assert torch.equal(outs[0], outs[1]), (step, l)
    finally:
        a.close()
        b.close()


def test_hybrid_needs_threads_and_refuses_capture():
    L, E, S, H, F, K, T = 1, 8, 4, 64, 128, 2, 1
    lay, host, sh, g = _layers(53, L, E, S, H, F, T, K, 2)
    out = torch.empty((T, H), dtype=torch.int16, device="cuda")
    x = _dev_u16(W.normal_bf16(g, (T, H)))
    lg = torch.from_numpy(W.zipf_logits(g, T, E, 0.6)).cuda()
    try:
        with pytest.raises(m.MoeError):
            lay.decode_hybrid(0, x, lg, K, out)
        m.moe_cache_set_cpu_threads(lay.cache, 2)
        s = torch.cuda.Stream()
        graph = torch.cuda.CUDAGraph()
        with pytest.raises(m.MoeError):
            with torch.cuda.graph(graph, stream=s):
                lay.decode_hybrid(0, x, lg, K, out, stream=s)
        torch.cuda.synchronize()
        st = m.moe_cache_read_state(lay.cache)
        assert st["clock"] == 0          # neither call launched anything
        m.moe_cache_set_cpu_threads(lay.cache, 0)
        with pytest.raises(m.MoeError):
            lay.decode_hybrid(0, x, lg, K, out)
    finally:
        lay.close()
