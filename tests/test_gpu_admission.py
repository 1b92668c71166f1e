"""GPU admission vs the oracle: rewritten ids, miss plans, slot maps,
stamps, clock, statistics and histograms must match bit for bit after
every step, on each configuration's admission shape."""
import numpy as np
import pytest
import torch

import expert_slot_cache_moe_amd as m
from expert_slot_cache_moe_amd import workloads as W
import oracle

pytestmark = pytest.mark.gpu


def _same(gc, oc, check_plan=True):
    st = m.moe_cache_read_state(gc)
    o = oc.state()
    for k in ("res", "own", "stamp", "stats", "freq", "dlast"):
        np.testing.assert_array_equal(st[k].reshape(o[k].shape), o[k], err_msg=k)
    assert st["clock"] == o["clock"] and st["last_demand"] == o["last_demand"]
    # the LRU order array is the slots sorted by (stamp, slot)
    expect_order = np.lexsort((np.arange(oc.S), o["stamp"]))
    np.testing.assert_array_equal(st["order"], expect_order, err_msg="order")
    if check_plan:
        ps, pe = m.moe_cache_read_plan(gc)
        np.testing.assert_array_equal(ps, oc.plan_slot, err_msg="plan slots")
        np.testing.assert_array_equal(pe, oc.plan_expert, err_msg="plan experts")


def _run(L, E, S, steps, one=256, qw=128, check_every=1):
    max_routes = max([len(s[1]) for s in steps] + [1])
    gc = m.moe_cache_create(num_layers=L, num_experts=E, num_slots=S, one_call_width=one,
                            query_width=qw, max_routes=max_routes)
    oc = oracle.OracleCache(L, E, S, one, qw)
    try:
        for i, (layer, ids, cap) in enumerate(steps):
            ids = np.asarray(ids, np.int32)
            t = torch.from_numpy(ids.copy()).cuda()
            m.moe_admit(gc, layer, t, cap)
            exp = oc.admit(layer, ids, cap)
            np.testing.assert_array_equal(t.cpu().numpy(), exp, err_msg=f"step {i}")
            if (i + 1) % check_every == 0 or i == len(steps) - 1:
                _same(gc, oc)
    finally:
        m.moe_cache_destroy(gc)


def test_tiny_trace():
    lg = W.tiny_logits(0, 32)[:, 0, :]
    ids, _ = oracle.topk(lg, 2)
    _run(1, 8, 4, [(0, ids[t], -1) for t in range(32)])


@pytest.mark.parametrize("requests", W.ADMISSION_BATCHES)
def test_admission_only_all_hits(requests):
    """512 experts pre-filled into 2100 slots, then steps of `requests` x 10
    uniform ids: every step is all hits."""
    steps = [(0, np.arange(512), -1)]
    for k in range(4):
        steps.append((0, W.admission_ids(k, requests), -1))
    _run(1, 512, 2100, steps)


def test_admission_only_crossover_widths():
    """One-call width forced down to 128 (re-measuring the crossover):
    130..240-route steps then take the chunked path."""
    steps = [(0, np.arange(512), -1)] + [(0, W.admission_ids(9, r), -1) for r in (13, 16, 24)]
    _run(1, 512, 2100, steps, one=128, qw=128)


@pytest.mark.parametrize("R", [255, 256, 257, 384])
def test_one_call_width_boundary(R):
    """At most 256 routes are one query over the raw route list; 257 and
    more go through the distinct list in 128-expert chunks; with misses and
    evictions (600 experts over 500 slots), states bit-exact each step."""
    g = np.random.default_rng(30 + R)
    steps = [(0, g.integers(0, 600, R), -1) for _ in range(12)]
    _run(1, 600, 500, steps)


def test_wide_step_counts_printed_on_the_pages():
    E = 160
    g = W.rng(0, "test", "wide")
    resident = g.choice(E, 7, replace=False)
    routes = W.wide_bf16_routes(0).reshape(-1)
    assert len(set(routes.tolist())) == E
    gc = m.moe_cache_create(num_layers=1, num_experts=E, num_slots=E, max_routes=300)
    try:
        m.moe_admit(gc, 0, torch.from_numpy(resident.astype(np.int32)).cuda())
        before = m.moe_cache_stats(gc, 0)
        t = torch.from_numpy(routes.astype(np.int32)).cuda()
        m.moe_admit(gc, 0, t)
        d = m.moe_cache_stats(gc, 0) - before
        assert d.tolist() == [1, 160, 153, 0, 0, 0, 0, 0]
        st = m.moe_cache_read_state(gc)
        np.testing.assert_array_equal(st["own"][t.cpu().numpy()], routes)
        assert int(st["freq"].sum()) == 7 + 300
    finally:
        m.moe_cache_destroy(gc)


@pytest.mark.parametrize("E,R,widths", [(640, 300, (256, 128)), (640, 300, (3, 3)),
                                        (256, 252, (256, 128)), (256, 252, (3, 3))])
def test_prefill_chunk_cold_cache(E, R, widths):
    g = W.rng(1, "prefill", E)
    T = R // 6
    steps = []
    for k in range(3):
        ids = np.stack([g.choice(E, 6, replace=False) for _ in range(T)]).reshape(-1)
        steps.append((0, ids, -1))
    _run(1, E, E, steps, one=widths[0], qw=widths[1])


@pytest.mark.parametrize("S,widths", [(1100, (256, 128)), (160, (3, 3)), (160, (256, 128))])
def test_wide_e2m1_step(S, widths):
    g = W.rng(2, "wide-e2m1")
    steps = [(0, np.stack([g.choice(160, 2, replace=False) for _ in range(600)]).reshape(-1), -1)
             for _ in range(3)]
    _run(1, 160, S, steps, one=widths[0], qw=widths[1])


def test_random_steps_with_caps_invalid_ids_and_cross_layer_eviction():
    g = np.random.default_rng(11)
    L, E, S = 4, 96, 70
    steps = []
    for _ in range(200):
        R = int(g.integers(0, 400))
        steps.append((int(g.integers(0, L)), g.integers(-5, E + 5, R), int(g.choice([-1, -1, 0, 7]))))
    _run(L, E, S, steps, one=40, qw=16)


def test_odd_widths_and_tiny_slot_counts():
    g = np.random.default_rng(12)
    for (L, E, S, one, qw) in [(2, 5, 1, 1, 1), (1, 3, 2, 2, 1), (3, 17, 9, 5, 3), (1, 2000, 3000, 256, 128)]:
        steps = [(int(g.integers(0, L)), g.integers(-1, E + 1, int(g.integers(0, 3 * E // 2 + 2))),
                  int(g.choice([-1, 0, 1, 4]))) for _ in range(40)]
        _run(L, E, S, steps, one=one, qw=qw)


def test_shared_expert_decode_trace_shape():
    """40 layers x 256 experts, top-8, 3164 slots: 48 tokens of the decode
    trace, compared after every token."""
    tr = W.DecodeTrace(0, 40, 256, 8)
    steps = []
    for _ in range(48):
        sets = tr.step_sets()
        steps += [(l, sets[l], -1) for l in range(40)]
    _run(40, 256, 3164, steps, check_every=40)


def test_empty_step_ticks_the_clock():
    _run(2, 8, 4, [(0, [], -1), (1, [3], -1), (1, [], -1), (0, [3, 3], -1)])


def test_bad_arguments_launch_nothing():
    gc = m.moe_cache_create(num_layers=2, num_experts=8, num_slots=4, max_routes=4)
    try:
        ids = torch.zeros(8, dtype=torch.int32, device="cuda")
        with pytest.raises(m.MoeError):
            m.moe_admit(gc, 2, ids[:2])
        with pytest.raises(m.MoeError):
            m.moe_admit(gc, 0, ids)          # 8 routes > max_routes 4
        assert m.moe_cache_read_state(gc)["clock"] == 0
    finally:
        m.moe_cache_destroy(gc)


def test_large_cache_uses_the_general_kernel():
    """More than 16384 slots: the global-memory admission kernel."""
    g = np.random.default_rng(13)
    L, E, S = 40, 640, 20000
    steps = [(int(g.integers(0, L)), g.integers(-1, E, int(g.integers(1, 700))), int(g.choice([-1, 5])))
             for _ in range(60)]
    _run(L, E, S, steps, check_every=10)


@pytest.mark.parametrize("S", [5000, 12000])
def test_register_order_of_8_and_16_slots_per_thread(S):
    """Caches of 4097-16384 slots keep 8 or 16 (slot, owner) order entries
    per thread of the register-resident kernel; wide and narrow steps with
    evictions across layers (20 x 640 experts > S)."""
    g = np.random.default_rng(S)
    L, E = 20, 640
    steps = []
    for i in range(80):
        R = int(g.integers(1, 64)) if i % 2 else int(g.integers(64, 1300))
        steps.append((int(g.integers(0, L)), g.integers(-1, E + 1, R), int(g.choice([-1, -1, 3]))))
    _run(L, E, S, steps, check_every=4)


@pytest.mark.parametrize("one,qw", [(256, 128), (20, 8), (1, 1)])
def test_narrow_steps_with_caps_and_invalid_ids(one, qw):
    """Steps of at most 64 routes (one route per lane of a wave), over a
    cache larger than 256 slots, with fetch caps, ids outside [0, E) and
    evictions across layers, at one-call and chunked widths."""
    g = np.random.default_rng(14 + one)
    L, E, S = 3, 200, 300
    steps = []
    for _ in range(300):
        R = int(g.integers(0, 65))
        steps.append((int(g.integers(0, L)), g.integers(-3, E + 3, R), int(g.choice([-1, -1, 0, 2, 9]))))
    _run(L, E, S, steps, one=one, qw=qw)
