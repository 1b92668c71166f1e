"""The shared-expert decode workload at full size, in the launch
configuration bench.py times: 40 layers x 256 experts, top-8 + gated
shared expert, H 2048, F 512, 3164 slots, bf16 experts in a 64.4 GB
pinned host store, the staged schedule captured as one hipGraph per token.
After 64 warm-up tokens, the next 3 tokens' slot ids (all 40 layers) must
equal the oracle's admission bit for bit, their router weights match, and
their outputs match the oracle within the tolerance, the oracle reading
each routed expert's own host rows (so the gathered slot bytes are checked
too).  Every expert of the store is drawn afresh, so no two slots hold
the same bytes."""
import gc

import numpy as np
import pytest
import torch

import bench
import expert_slot_cache_moe_amd as m
from expert_slot_cache_moe_amd import workloads as W
import oracle
from parity import check_close

pytestmark = pytest.mark.gpu


def test_full_size_decode_matches_oracle():
    L, E, K, H, F, S = bench.L, bench.E, bench.K, bench.H, bench.F, bench.S
    warm, check = bench.CACHE_WARM_TOKENS, 3
    lay = bench.build_stack(torch, m, W, overlap=2)
    try:
        lg_all, x_all = bench.make_trace(torch, W, warm + check)
        x_st = torch.empty((L, 1, H), dtype=torch.int16, device="cuda")
        lg_st = torch.empty((L, 1, E), dtype=torch.float32, device="cuda")
        out = torch.empty((L, 1, H), dtype=torch.int16, device="cuda")
        ids = torch.empty((L, 1, K), dtype=torch.int32, device="cuda")
        w = torch.empty((L, 1, K), dtype=torch.float32, device="cuda")
        # the bench's token graph: token t's inputs staged by the device-side
        # step counter (replay t reads token t)
        tok = torch.zeros(1, dtype=torch.int64, device="cuda")
        graph = bench.capture(torch, lay, x_st, lg_st, out, (x_all, lg_all, tok), ids, w)
        for t in range(warm):
            graph.replay()
        torch.cuda.synchronize()

        lg_np = lg_all.cpu().numpy()
        x_np = x_all.cpu().numpy().view(np.uint16)
        oc = oracle.OracleCache(L, E, S)
        for t in range(warm):
            for l in range(L):
                e_ids, _ = oracle.topk(lg_np[t, l], K)
                oc.admit(l, e_ids.reshape(-1))
        # the oracle reads each expert's own host rows (every expert drawn afresh)
        pools = [oracle.Pool(0, H, F, [b.numpy() for b in lay.host[l]]) for l in range(L)]
        gs = W.rng(0, "bench", "shared")
        shared = [(W.normal_bf16(gs, 2 * F * H, 0.02), W.normal_bf16(gs, H * F, 0.02),
                   W.normal_bf16(gs, H, 0.02)) for _ in range(L)]

        misses = 0
        for t in range(warm, warm + check):
            graph.replay()
            torch.cuda.synchronize()
            got_ids = ids.cpu().numpy()
            got_w = w.cpu().numpy()
            got = out.view(torch.bfloat16).double().cpu().numpy()
            for l in range(L):
                e_ids, wts = oracle.topk(lg_np[t, l], K)
                slots = oc.admit(l, e_ids.reshape(-1)).reshape(1, K)
                misses += len(oc.plan_slot)
                np.testing.assert_array_equal(got_ids[l], slots, err_msg=f"token {t} layer {l}")
                np.testing.assert_allclose(got_w[l], wts, rtol=1e-5)
                idx = np.where(slots >= 0, e_ids, -1).astype(np.int32)
                _, add = oracle.shared(H, F, *shared[l], x_np[t, l])
                ref = oracle.routed(pools[l], idx, wts, x_np[t, l], addend=add)
                check_close(got[l], ref, f"token {t} layer {l}")
        assert misses > 0                    # the checked tokens do fetch
    finally:
        lay.close()
        # hand the 60 GB of pinned host memory back, so later tests can pin
        del lay
        gc.collect()
        torch.cuda.synchronize()
        if hasattr(torch._C, "_host_emptyCache"):
            torch._C._host_emptyCache()
