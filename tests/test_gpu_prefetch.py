"""GPU look-ahead prefetch with the LFRU eviction guard vs the oracle
(llama.cpp fork PR #126, sections Consumer and Eviction guard).

The slot map, owners, stamps, LRU order, statistics, demand heat and fill
plans must match the oracle bit for bit after every call; prefetched slots
must hold their experts' bytes; layer steps after a prefetch must match the
oracle within the layer tolerance (max |gpu - oracle| <= 2e-2 * max
|oracle|), and a captured token with prefetches must replay like the same
calls run eagerly."""
import json
import os

import numpy as np
import pytest
import torch

import expert_slot_cache_moe_amd as m
from expert_slot_cache_moe_amd import workloads as W
from expert_slot_cache_moe_amd.layer import SlotCacheLayers
import oracle
from parity import check_close

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    with open(os.path.join(GOLDEN, "prefetch_guard.json")) as f:
        return json.load(f)


def _dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()


def _dev_u16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def _same(gc, oc, what=""):
    st = m.moe_cache_read_state(gc)
    o = oc.state()
    for k in ("res", "own", "stamp", "stats", "freq", "dlast"):
        np.testing.assert_array_equal(st[k].reshape(o[k].shape), o[k], err_msg=f"{what}: {k}")
    assert st["clock"] == o["clock"], what
    assert st["last_demand"] == o["last_demand"], what
    expect_order = np.lexsort((np.arange(oc.S), o["stamp"]))
    np.testing.assert_array_equal(st["order"], expect_order, err_msg=f"{what}: order")


def _same_fills(gc, oc, what=""):
    ps, pe = m.moe_cache_read_fills(gc)
    np.testing.assert_array_equal(ps, oc.fill_slot, err_msg=f"{what}: fill slots")
    np.testing.assert_array_equal(pe, oc.fill_expert, err_msg=f"{what}: fill experts")


@pytest.mark.parametrize("case", _golden()["pool_case"]["cases"], ids=["warm-survives", "once-evicted"])
def test_three_slot_guard_case(case):
    g = _golden()["pool_case"]
    L, E, S = g["layers"], g["experts"], g["slots"]
    gc = m.moe_cache_create(num_layers=L, num_experts=E, num_slots=S, max_routes=8)
    oc = oracle.OracleCache(L, E, S)
    try:
        for ids in case["demand_steps"]:
            m.moe_admit(gc, 0, _dev_i32(ids))
            oc.admit(0, ids)
        m.moe_prefetch(gc, 0, _dev_i32(case["predict"]))
        oc.prefetch(0, case["predict"])
        _same(gc, oc, "after prefetch")
        _same_fills(gc, oc)
        st = m.moe_cache_read_state(gc)
        assert st["stats"][0][m.MOE_STAT_PF_FILLED] == case["fills"]
        assert st["stats"][0][m.MOE_STAT_PF_DROPPED] == case["dropped"]
        for e, resident in case["resident_after_prefetch"].items():
            assert (st["res"][int(e)] >= 0) == resident
        t = _dev_i32(case["then_demand"])
        m.moe_admit(gc, 0, t)
        oc.admit(0, case["then_demand"])
        assert (t.cpu().numpy() >= 0).all()
        d = m.moe_cache_read_state(gc)["stats"][0][m.MOE_STAT_MISSED] - st["stats"][0][m.MOE_STAT_MISSED]
        assert d == case["then_missed"]
        _same(gc, oc, "after demand")
    finally:
        m.moe_cache_destroy(gc)


@pytest.mark.parametrize("case", _golden()["threshold_cases"]["cases"],
                         ids=lambda c: f"{c['score_res']}-vs-{c['score_pred']}")
def test_guard_threshold_cases(case):
    g = _golden()["threshold_cases"]
    E, S = 4, 1
    gc = m.moe_cache_create(num_layers=1, num_experts=E, num_slots=S, max_routes=4)
    oc = oracle.OracleCache(1, E, S)
    try:
        oc.res[0], oc.own[0], oc.stamp[0] = 0, 0, g["slot_stamp"]
        oc.clock[0], oc.last_demand[0] = g["clock"], g["last_demand"]
        oc.freq[0], oc.dlast[0] = case["freq_res"], case["dlast_res"]
        oc.freq[1], oc.dlast[1] = case["freq_pred"], case["dlast_pred"]
        m.moe_cache_write_state(gc, oc.res, oc.own, oc.stamp, int(oc.clock[0]), freq=oc.freq,
                                dlast=oc.dlast, last_demand=int(oc.last_demand[0]))
        m.moe_prefetch(gc, 0, _dev_i32([1]))
        oc.prefetch(0, [1])
        _same(gc, oc)
        _same_fills(gc, oc)
        st = m.moe_cache_read_state(gc)
        assert (st["res"][0] == 0) == case["protected"]
    finally:
        m.moe_cache_destroy(gc)


def _mixed(L, E, S, one, qw, ops, max_routes):
    gc = m.moe_cache_create(num_layers=L, num_experts=E, num_slots=S, one_call_width=one,
                            query_width=qw, max_routes=max_routes)
    oc = oracle.OracleCache(L, E, S, one, qw)
    try:
        for i, (kind, layer, ids, cap) in enumerate(ops):
            t = _dev_i32(ids)
            if kind == "d":
                m.moe_admit(gc, layer, t, cap)
                exp = oc.admit(layer, ids, cap)
                np.testing.assert_array_equal(t.cpu().numpy(), exp, err_msg=f"op {i}: ids")
            else:
                m.moe_prefetch(gc, layer, t)
                oc.prefetch(layer, ids)
                if len(ids):
                    _same_fills(gc, oc, f"op {i}")
            _same(gc, oc, f"op {i} ({kind})")
        return m.moe_cache_read_state(gc)["stats"]
    finally:
        m.moe_cache_destroy(gc)


def _ops(g, L, E, n_ops, max_r, hot_frac, cap_choices=(-1,)):
    ops = []
    for _ in range(n_ops):
        layer = int(g.integers(0, L))
        R = int(g.integers(0, max_r + 1))
        hot = g.random(R) < hot_frac
        ids = np.where(hot, g.integers(0, max(2, E // 8), R), g.integers(-2, E + 2, R)).astype(np.int32)
        kind = "p" if g.random() < 0.45 else "d"
        ops.append((kind, layer, ids, int(g.choice(cap_choices))))
    return ops


@pytest.mark.parametrize("L,E,S,one,qw,max_r", [
    (2, 16, 6, 256, 128, 8),         # narrow demand steps, tight cache: the guard decides often
    (3, 64, 40, 256, 128, 64),       # narrow steps up to one wave
    (2, 96, 70, 40, 16, 300),        # wide chunked steps
    (1, 300, 500, 256, 128, 250),    # many predictions per call
    (2, 64, 6000, 256, 128, 64),     # (slot, owner) order longer than the entries a thread holds
])
def test_mixed_traces_match_the_oracle(L, E, S, one, qw, max_r):
    g = np.random.default_rng(100 + E)
    ops = _ops(g, L, E, 160, max_r, 0.5, (-1, -1, 0, 5))
    stats = _mixed(L, E, S, one, qw, ops, max_r)
    assert stats[:, m.MOE_STAT_PF_FILLED].sum() > 0
    if S < E:       # the guard (or a cache full of pinned slots) has dropped some
        assert stats[:, m.MOE_STAT_PF_DROPPED].sum() > 0


def test_mixed_trace_on_the_global_memory_order():
    """More than 16384 slots: the order holds plain slot ids and demand steps
    use the global-memory admission kernel."""
    g = np.random.default_rng(7)
    L, E, S = 2, 64, 16400
    ops = _ops(g, L, E, 40, 100, 0.5)
    # demand steps over every expert first, so the guard has heat to compare
    warm = [("d", l, np.arange(E, dtype=np.int32), -1) for l in range(L)]
    _mixed(L, E, S, 256, 128, warm + ops, 128)


def test_width_zero_and_invalid_ids():
    gc = m.moe_cache_create(num_layers=2, num_experts=8, num_slots=4, max_routes=8)
    oc = oracle.OracleCache(2, 8, 4)
    try:
        m.moe_admit(gc, 0, _dev_i32([1, 2]))
        oc.admit(0, [1, 2])
        before = m.moe_cache_read_state(gc)
        m.moe_prefetch(gc, 1, _dev_i32([]), n=0)
        after = m.moe_cache_read_state(gc)
        for k in before:
            np.testing.assert_array_equal(np.asarray(after[k]), np.asarray(before[k]), err_msg=k)
        m.moe_prefetch(gc, 1, _dev_i32([-1, 8, 99]))
        oc.prefetch(1, [-1, 8, 99])
        _same(gc, oc)
        assert m.moe_cache_read_state(gc)["stats"][1][m.MOE_STAT_PF_CALLS] == 1
    finally:
        m.moe_cache_destroy(gc)


def test_bad_arguments_launch_nothing():
    gc = m.moe_cache_create(num_layers=2, num_experts=8, num_slots=4, max_routes=4)
    try:
        ids = _dev_i32(np.zeros(8))
        with pytest.raises(m.MoeError):
            m.moe_prefetch(gc, 2, ids[:2])
        with pytest.raises(m.MoeError):
            m.moe_prefetch(gc, -1, ids[:2])
        with pytest.raises(m.MoeError):
            m.moe_prefetch(gc, 0, ids)            # 8 ids > max_routes 4
        st = m.moe_cache_read_state(gc)
        assert st["clock"] == 0 and (st["stats"] == 0).all()
    finally:
        m.moe_cache_destroy(gc)


@pytest.mark.parametrize("fmt", [0, 1, 2])
def test_prefetched_slots_hold_their_experts_bytes(fmt):
    L, E, S, H, F = 2, 16, 6, 64, 128
    g = W.rng(41, "prefetch-bytes", fmt)
    host = [W.expert_rows(fmt, g, E, H, F) for _ in range(L)]
    lay = SlotCacheLayers(layers=L, experts=E, slots=S, hidden=H, ffn=F, fmt=fmt, host_rows=host,
                          max_tokens=1, max_top_k=4)
    oc = oracle.OracleCache(L, E, S)
    try:
        for step in range(12):
            layer = step % L
            d = g.choice(E, 2, replace=False).astype(np.int32)
            m.moe_admit(lay.cache, layer, _dev_i32(d))
            oc.admit(layer, d)
            m.moe_gather_misses(lay.cache)
            p = g.choice(E, 3, replace=False).astype(np.int32)
            m.moe_prefetch(lay.cache, 1 - layer, _dev_i32(p))
            oc.prefetch(1 - layer, p)
            m.moe_prefetch_join(lay.cache)
            torch.cuda.synchronize()
            _same(lay.cache, oc, f"step {step}")
            for s, e in zip(oc.fill_slot.tolist(), oc.fill_expert.tolist()):
                for b, bank in enumerate(lay.slot_banks):
                    np.testing.assert_array_equal(bank[s].cpu().numpy(), host[1 - layer][b][e],
                                                  err_msg=f"step {step} slot {s} bank {b}")
    finally:
        lay.close()


def _predict(g, true_ids, E, accuracy):
    """Each true expert kept with probability `accuracy`, else replaced by a
    random expert."""
    keep = g.random(true_ids.size) < accuracy
    return np.where(keep, true_ids, g.integers(0, E, true_ids.size)).astype(np.int32)


def _oracle_layer(oc, host, sh, layer, x, lg, K, fmt, H, F):
    ids_e, w = oracle.topk(lg, K)
    slots = oc.admit(layer, ids_e.reshape(-1)).reshape(ids_e.shape)
    _, add = oracle.shared(H, F, sh[layer][0], sh[layer][1], sh[layer][2], x)
    idx = np.where(slots >= 0, ids_e, -1)
    return oracle.routed(oracle.Pool(fmt, H, F, host[layer]), idx, w, x, addend=add), slots


@pytest.mark.parametrize("overlap,fmt", [(0, 0), (1, 0), (2, 0), (2, 1)])
def test_layer_steps_with_lookahead_match_the_oracle(overlap, fmt):
    """Each layer step is followed by a prefetch of the next layer's
    predicted experts; the next step's hits include the prefetched ones."""
    L, E, S, H, F, K = 3, 16, 10, 64, 128, 2
    g = W.rng(43, "lookahead", overlap, fmt)
    host = [W.expert_rows(fmt, g, E, H, F) for _ in range(L)]
    sh = [(W.normal_bf16(g, 2 * F * H, 0.02), W.normal_bf16(g, H * F, 0.02), W.normal_bf16(g, H, 0.02))
          for _ in range(L)]
    lay = SlotCacheLayers(layers=L, experts=E, slots=S, hidden=H, ffn=F, fmt=fmt, host_rows=host,
                          shared=sh, max_tokens=1, max_top_k=K, overlap=overlap)
    oc = oracle.OracleCache(L, E, S)
    out = torch.empty((1, H), dtype=torch.int16, device="cuda")
    ids = torch.empty((1, K), dtype=torch.int32, device="cuda")
    try:
        for t in range(12):
            lgs = W.zipf_logits(g, L, E, 0.7)
            for l in range(L):
                x = W.normal_bf16(g, (1, H))
                lay.decode(l, _dev_u16(x), torch.from_numpy(lgs[l:l + 1]).cuda(), K, out, ids_out=ids)
                ref, slots = _oracle_layer(oc, host, sh, l, x, lgs[l:l + 1], K, fmt, H, F)
                nxt = (l + 1) % L
                true_next, _ = oracle.topk(lgs[nxt:nxt + 1], K)
                pred = _predict(g, true_next.reshape(-1), E, 0.7)
                m.moe_prefetch(lay.cache, nxt, _dev_i32(pred))
                oc.prefetch(nxt, pred)
                torch.cuda.synchronize()
                np.testing.assert_array_equal(ids.cpu().numpy(), slots, err_msg=f"token {t} layer {l}")
                got = out.view(torch.bfloat16).double().cpu().numpy()
                check_close(got, ref, f"token {t} layer {l}")
        m.moe_prefetch_join(lay.cache)
        _same(lay.cache, oc)
        st = m.moe_cache_read_state(lay.cache)["stats"]
        assert st[:, m.MOE_STAT_PF_FILLED].sum() > 5
    finally:
        lay.close()


def test_captured_token_with_prefetches_replays_like_eager():
    """A token of 3 layer steps, each followed by a prefetch of the next
    layer, captured as one graph (the prefetch copies fork to the cache's
    prefetch stream and join at the next admission) and replayed over 30
    tokens, equals the same calls run eagerly."""
    L, E, S, H, F, K = 3, 16, 10, 64, 128, 2
    mk = lambda: SlotCacheLayers(layers=L, experts=E, slots=S, hidden=H, ffn=F,
                                 host_rows=host, shared=sh, max_tokens=1, max_top_k=K, overlap=2)
    g = W.rng(44, "lookahead-graph")
    host = [W.expert_rows(0, g, E, H, F) for _ in range(L)]
    sh = [(W.normal_bf16(g, 2 * F * H, 0.02), W.normal_bf16(g, H * F, 0.02), W.normal_bf16(g, H, 0.02))
          for _ in range(L)]
    graph_l, eager_l = mk(), mk()
    x_st = torch.empty((L, 1, H), dtype=torch.int16, device="cuda")
    lg_st = torch.empty((L, 1, E), dtype=torch.float32, device="cuda")
    pr_st = torch.empty((L, K), dtype=torch.int32, device="cuda")
    out_g = torch.empty((L, 1, H), dtype=torch.int16, device="cuda")
    out_e = torch.empty_like(out_g)

    def token(lay, out, stream=None):
        for l in range(L):
            lay.decode(l, x_st[l], lg_st[l], K, out[l], stream=stream)
            m.moe_prefetch(lay.cache, (l + 1) % L, pr_st[(l + 1) % L], stream=stream)
        m.moe_prefetch_join(lay.cache, stream=stream)

    def load(t):
        lgs = W.zipf_logits(g, L, E, 0.7)
        true_ids, _ = oracle.topk(lgs, K)
        x_st.copy_(_dev_u16(W.normal_bf16(g, (L, 1, H))))
        lg_st.copy_(torch.from_numpy(lgs.reshape(L, 1, E)))
        pr_st.copy_(_dev_i32(_predict(g, true_ids.reshape(-1), E, 0.6).reshape(L, K)))

    try:
        s = torch.cuda.Stream()
        load(0)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=s):
            token(graph_l, out_g, stream=s)
        for t in range(30):
            load(t)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            token(eager_l, out_e)
            torch.cuda.synchronize()
            assert torch.equal(out_g, out_e), f"token {t}"
        a = m.moe_cache_read_state(graph_l.cache)
        b = m.moe_cache_read_state(eager_l.cache)
        for k in ("res", "own", "stamp", "stats", "freq", "dlast", "order"):
            np.testing.assert_array_equal(a[k], b[k], err_msg=k)
        assert a["stats"][:, m.MOE_STAT_PF_CALLS].tolist() == [30] * L
        assert a["stats"][:, m.MOE_STAT_PF_FILLED].sum() > 0
    finally:
        graph_l.close()
        eager_l.close()


def test_many_experts_prefetch_is_sized_by_the_prediction_count():
    """The prefetch kernel's LDS grows with the predictions a call may hold
    (min(max_routes, E)), not with E alone: 3400 experts with calls of up to
    300 ids work; a cache whose full-width prefetch would not fit the LDS is
    still created, and only its prefetch is refused."""
    g = np.random.default_rng(21)
    L, E, S = 2, 3400, 3500
    ops = [("d", l, g.choice(E, 200, replace=False).astype(np.int32), -1) for l in range(L)]
    for _ in range(30):
        kind = "p" if g.random() < 0.5 else "d"
        ids = np.minimum(g.zipf(1.2, int(g.integers(1, 300))) - 1, E + 1).astype(np.int32)
        ops.append((kind, int(g.integers(0, L)), ids, -1))
    _mixed(L, E, S, 256, 128, ops, 300)

    E2, S2 = 3300, 3400
    gc = m.moe_cache_create(num_layers=1, num_experts=E2, num_slots=S2, max_routes=E2)
    try:
        m.moe_admit(gc, 0, _dev_i32(np.arange(100)))
        with pytest.raises(m.MoeError) as e:
            m.moe_prefetch(gc, 0, _dev_i32([5, 500]))
        assert e.value.status == m.MOE_UNSUPPORTED
        assert m.moe_cache_read_state(gc)["clock"] == 1
    finally:
        m.moe_cache_destroy(gc)


def test_eager_prefetch_must_be_joined_before_a_capture():
    """A prefetch issued eagerly and still pending when a capture begins
    cannot be waited for inside the capture: the layer step refuses (it would
    otherwise race with the copy); after moe_prefetch_join it captures."""
    L, E, S, H, F, K = 2, 16, 10, 64, 128, 2
    g = W.rng(45, "eager-then-capture")
    host = [W.expert_rows(0, g, E, H, F) for _ in range(L)]
    lay = SlotCacheLayers(layers=L, experts=E, slots=S, hidden=H, ffn=F, host_rows=host,
                          max_tokens=1, max_top_k=K, overlap=2)
    x = _dev_u16(W.normal_bf16(g, (1, H)))
    lg = torch.from_numpy(W.zipf_logits(g, 1, E, 0.7)).cuda()
    out = torch.empty((1, H), dtype=torch.int16, device="cuda")
    try:
        lay.decode(0, x, lg, K, out)
        m.moe_prefetch(lay.cache, 1, _dev_i32([3, 4]))
        torch.cuda.synchronize()
        s = torch.cuda.Stream()
        graph = torch.cuda.CUDAGraph()
        with pytest.raises(m.MoeError):
            with torch.cuda.graph(graph, stream=s):
                lay.decode(1, x, lg, K, out, stream=s)
        torch.cuda.synchronize()
        m.moe_prefetch_join(lay.cache)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=s):
            lay.decode(1, x, lg, K, out, stream=s)
        graph.replay()
        torch.cuda.synchronize()
        assert m.moe_cache_read_state(lay.cache)["stats"][1][m.MOE_STAT_CALLS] == 1
    finally:
        lay.close()
