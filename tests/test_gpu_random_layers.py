"""Seeded random layer steps against the oracle: formats, widths, expert
and slot counts, batch sizes, top-k, fetch caps, schedules and shared
experts drawn at random, so that the paths between them (fused and separate
top-k, one-token stages, grouped MFMA and vector kernels, capped admission,
the four schedules) are crossed in combinations no hand-written case
names.

Per step: slot ids exact, outputs within max |gpu - oracle| <= 2e-2 * max
|oracle|, and after the steps the slot map, owners, stamps, statistics,
histogram and demand recency exact."""
import numpy as np
import pytest
import torch

import expert_slot_cache_moe_amd as m
from expert_slot_cache_moe_amd import workloads as W
from expert_slot_cache_moe_amd.layer import SlotCacheLayers
import oracle
from parity import check_close

pytestmark = pytest.mark.gpu

CASES = 36


def _draw(i):
    g = np.random.default_rng([77, i])
    fmt = int(g.choice([0, 0, 1, 2]))
    H = int(g.choice([64, 128, 256, 1024]))
    F = int(g.choice([64, 128, 256]))
    E = int(g.integers(4, 65))
    S = int(g.integers(1, E + 5))
    K = int(g.integers(1, min(8, E) + 1))
    T = int(g.choice([1, 1, 2, 5, 17, 33, 40]))
    overlap = int(g.integers(0, 4))
    shared = bool(g.random() < 0.6)
    L = int(g.integers(1, 4))
    caps = [int(c) for c in g.choice([-1, -1, 0, 1, 3], 4)]
    return dict(fmt=fmt, H=H, F=F, E=E, S=S, K=K, T=T, overlap=overlap, shared=shared, L=L,
                caps=caps)


@pytest.mark.parametrize("i", range(CASES))
def test_random_layer_steps_match_the_oracle(i):
    c = _draw(i)
    fmt, H, F, E, S, K, T, L = c["fmt"], c["H"], c["F"], c["E"], c["S"], c["K"], c["T"], c["L"]
    g = W.rng(78, "random-layers", i)
    host = [W.expert_rows(fmt, g, E, H, F) for _ in range(L)]
    sh = None
    if c["shared"]:
        sh = [(W.normal_bf16(g, 2 * F * H, 0.02), W.normal_bf16(g, H * F, 0.02), W.normal_bf16(g, H, 0.02))
              for _ in range(L)]
    print(f"case {i}: {c}", flush=True)
    lay = SlotCacheLayers(layers=L, experts=E, slots=S, hidden=H, ffn=F, fmt=fmt, host_rows=host,
                          shared=sh, max_tokens=T, max_top_k=K, overlap=c["overlap"])
    oc = oracle.OracleCache(L, E, S)
    out = torch.empty((T, H), dtype=torch.int16, device="cuda")
    ids = torch.empty((T, K), dtype=torch.int32, device="cuda")
    try:
        for step, cap in enumerate(c["caps"]):
            layer = step % L
            x = W.normal_bf16(g, (T, H))
            lg = W.zipf_logits(g, T, E, 0.8)
            lay.decode(layer, torch.from_numpy(x.view(np.int16)).cuda(), torch.from_numpy(lg).cuda(), K,
                       out, ids_out=ids, max_fetch=cap)
            ids_e, w = oracle.topk(lg, K)
            slots = oc.admit(layer, ids_e.reshape(-1), cap).reshape(T, K)
            add = None
            if sh is not None:
                _, add = oracle.shared(H, F, sh[layer][0], sh[layer][1], sh[layer][2], x)
            ref = oracle.routed(oracle.Pool(fmt, H, F, host[layer]), np.where(slots >= 0, ids_e, -1), w,
                                x, addend=add)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(ids.cpu().numpy(), slots, err_msg=f"step {step}")
            got = out.view(torch.bfloat16).double().cpu().numpy()
            scale = np.abs(ref).max()
            if scale == 0:
                assert (got == 0).all(), f"step {step}"
            else:
                check_close(got, ref, f"step {step}")
        st = m.moe_cache_read_state(lay.cache)
        o = oc.state()
        for k in ("res", "own", "stamp", "stats", "freq", "dlast"):
            np.testing.assert_array_equal(st[k].reshape(o[k].shape), o[k], err_msg=k)
    finally:
        lay.close()


@pytest.mark.parametrize("i", range(12))
def test_random_hybrid_steps_match_the_oracle(i):
    """The hybrid step (routes left at -1 run on host threads) at random
    weight formats, widths, batch sizes, caps, schedules and thread
    counts."""
    g0 = np.random.default_rng([79, i])
    H = int(g0.choice([64, 128, 256, 1024]))
    F = int(g0.choice([64, 128, 256]))
    E = int(g0.integers(4, 49))
    S = int(g0.integers(1, E + 3))
    K = int(g0.integers(1, min(8, E) + 1))
    T = int(g0.choice([1, 2, 5, 17, 40]))
    L = int(g0.integers(1, 3))
    overlap = int(g0.integers(0, 4))
    shared = bool(g0.random() < 0.6)
    threads = int(g0.choice([1, 2, 5]))
    caps = [int(c) for c in g0.choice([0, 0, 1, 3, -1], 4)]
    fmt = int(g0.choice([0, 1, 2]))
    print(f"hybrid case {i}: fmt {fmt} H {H} F {F} E {E} S {S} K {K} T {T} L {L} overlap {overlap} "
          f"shared {shared} threads {threads} caps {caps}", flush=True)
    g = W.rng(80, "random-hybrid", i)
    host = [W.expert_rows(fmt, g, E, H, F) for _ in range(L)]
    sh = None
    if shared:
        sh = [(W.normal_bf16(g, 2 * F * H, 0.02), W.normal_bf16(g, H * F, 0.02), W.normal_bf16(g, H, 0.02))
              for _ in range(L)]
    lay = SlotCacheLayers(layers=L, experts=E, slots=S, hidden=H, ffn=F, fmt=fmt, host_rows=host, shared=sh,
                          max_tokens=T, max_top_k=K, overlap=overlap)
    m.moe_cache_set_cpu_threads(lay.cache, threads)
    oc = oracle.OracleCache(L, E, S)
    out = torch.empty((T, H), dtype=torch.int16, device="cuda")
    ids = torch.empty((T, K), dtype=torch.int32, device="cuda")
    try:
        for step, cap in enumerate(caps):
            layer = step % L
            x = W.normal_bf16(g, (T, H))
            lg = W.zipf_logits(g, T, E, 0.8)
            lay.decode_hybrid(layer, torch.from_numpy(x.view(np.int16)).cuda(), torch.from_numpy(lg).cuda(),
                              K, out, ids_out=ids, max_fetch=cap)
            ids_e, w = oracle.topk(lg, K)
            slots = oc.admit(layer, ids_e.reshape(-1), cap).reshape(T, K)
            add = None
            if sh is not None:
                _, add = oracle.shared(H, F, sh[layer][0], sh[layer][1], sh[layer][2], x)
            ref = oracle.routed(oracle.Pool(fmt, H, F, host[layer]), ids_e, w, x, addend=add)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(ids.cpu().numpy(), slots, err_msg=f"step {step}")
            got = out.view(torch.bfloat16).double().cpu().numpy()
            check_close(got, ref, f"step {step}")
        st = m.moe_cache_read_state(lay.cache)
        o = oc.state()
        for k in ("res", "own", "stamp", "stats", "freq", "dlast"):
            np.testing.assert_array_equal(st[k].reshape(o[k].shape), o[k], err_msg=k)
    finally:
        lay.close()
