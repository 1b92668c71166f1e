"""Pins for the oracle's look-ahead prefetch and its LFRU eviction guard
(CPU only).

The guard case and the score threshold come from llama.cpp fork PR #126
(sections Eviction guard and Verification), stored in
tests/golden/prefetch_guard.json with the reading they rest on.  Mixed
demand/prefetch traces are brute-forced against the recency-list model in
tests/spec_lru.py, and invariants the page fixes are checked after every
call of random traces.
"""
import json
import os

import numpy as np
import pytest

import oracle
from spec_lru import SpecCache

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

# column of the per-layer statistics
CALLS, MET, MISSED, OVERFLOW, INVALID, PF_CALLS, PF_FILLED, PF_DROPPED = range(8)


def _golden():
    with open(os.path.join(GOLDEN, "prefetch_guard.json")) as f:
        return json.load(f)


# ---------------------------------------------------------------- pins from the page

@pytest.mark.parametrize("case", _golden()["pool_case"]["cases"], ids=lambda c: c["what"][:40])
def test_three_slot_guard_case(case):
    g = _golden()["pool_case"]
    oc = oracle.OracleCache(g["layers"], g["experts"], g["slots"])
    for ids in case["demand_steps"]:
        oc.admit(0, ids)
    before = oc.state()
    oc.prefetch(0, case["predict"])
    after = oc.state()
    d = after["stats"][0] - before["stats"][0]
    assert d[PF_CALLS] == 1
    assert d[PF_FILLED] == case["fills"] == oc.fill_slot.size
    assert d[PF_DROPPED] == case["dropped"]
    for e, resident in case["resident_after_prefetch"].items():
        assert (after["res"][int(e)] >= 0) == resident, e
    if case["fills"] == 0:
        # no copy and no eviction: the slot map is untouched
        np.testing.assert_array_equal(after["res"], before["res"])
        np.testing.assert_array_equal(after["own"], before["own"])
    # prefetch never counts as demand
    np.testing.assert_array_equal(after["freq"], before["freq"])
    np.testing.assert_array_equal(after["dlast"], before["dlast"])
    assert after["last_demand"] == before["last_demand"]
    assert d[:PF_CALLS].tolist() == [0] * PF_CALLS
    out = oc.admit(0, case["then_demand"])
    assert (out >= 0).all()
    assert oc.state()["stats"][0][MISSED] - after["stats"][0][MISSED] == case["then_missed"]


@pytest.mark.parametrize("case", _golden()["threshold_cases"]["cases"],
                         ids=lambda c: f"{c['score_res']}-vs-{c['score_pred']}")
def test_guard_threshold_hand_worked(case):
    g = _golden()["threshold_cases"]
    oc = oracle.OracleCache(1, 4, 1)
    oc.res[0] = 0
    oc.own[0] = 0
    oc.stamp[0] = g["slot_stamp"]
    oc.clock[0] = g["clock"]
    oc.last_demand[0] = g["last_demand"]
    oc.freq[0], oc.dlast[0] = case["freq_res"], case["dlast_res"]
    oc.freq[1], oc.dlast[1] = case["freq_pred"], case["dlast_pred"]
    oc.prefetch(0, [1])
    st = oc.state()
    if case["protected"]:
        assert st["stats"][0][PF_DROPPED] == 1 and oc.fill_slot.size == 0
        assert st["res"][0] == 0 and st["res"][1] == -1
    else:
        assert st["stats"][0][PF_FILLED] == 1
        assert oc.fill_slot.tolist() == [0] and oc.fill_expert.tolist() == [1]
        assert st["res"][0] == -1 and st["res"][1] == 0 and st["own"][0] == 1
        assert st["stamp"][0] == g["clock"] + 1


def test_width_zero_is_a_no_op():
    oc = oracle.OracleCache(2, 16, 8)
    oc.admit(0, [1, 2, 3])
    before = oc.state()
    oc.prefetch(1, [])
    after = oc.state()
    for k in before:
        np.testing.assert_array_equal(np.asarray(after[k]), np.asarray(before[k]), err_msg=k)


def test_ids_outside_the_expert_range_are_ignored():
    oc = oracle.OracleCache(1, 16, 8)
    oc.prefetch(0, [-1, 16, 99, -7])
    st = oc.state()
    assert st["stats"][0][PF_CALLS] == 1
    assert st["stats"][0][PF_FILLED] == 0 and st["stats"][0][PF_DROPPED] == 0
    assert (st["res"] == -1).all()


def test_slots_of_the_latest_demand_step_are_never_chosen():
    # every slot was used by the latest demand step: the prediction is dropped
    oc = oracle.OracleCache(1, 16, 4)
    oc.admit(0, [0, 1, 2, 3])
    oc.prefetch(0, [9])
    st = oc.state()
    assert st["stats"][0][PF_DROPPED] == 1 and st["res"][9] == -1
    # fills made since then are pinned too: a second prefetch cannot evict them
    oc = oracle.OracleCache(1, 16, 4)
    oc.admit(0, [0, 1])
    oc.prefetch(0, [5, 6])
    assert sorted(oc.fill_expert.tolist()) == [5, 6]
    oc.prefetch(0, [7])
    st = oc.state()
    assert st["stats"][0][PF_DROPPED] == 1
    assert (st["res"][[0, 1, 5, 6]] >= 0).all()


def test_heat_counts_demand_only():
    # a prediction never makes itself warm: predicting an expert many times
    # leaves its frequency at 0, so it never protects its slot
    oc = oracle.OracleCache(1, 16, 2)
    for _ in range(5):
        oc.admit(0, [0])          # expert 0 warm in slot 0; slot 1 free
        oc.prefetch(0, [3])       # fills slot 1 the first time, then a hit
    assert oc.state()["freq"][3] == 0
    oc.admit(0, [0])
    oc.admit(0, [4])              # evicts 3 by plain LRU on the demand path
    st = oc.state()
    assert st["res"][3] == -1 and st["res"][4] >= 0


# ---------------------------------------------------------------- brute force

def _same_state(oc, sp):
    a, b = oc.state(), sp.arrays()
    for k in ("res", "own", "stamp", "stats", "freq", "dlast"):
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)
    assert a["clock"] == b["clock"] and a["last_demand"] == b["last_demand"]


def _run_mixed(L, E, S, one, qw, ops):
    oc = oracle.OracleCache(L, E, S, one, qw)
    sp = SpecCache(L, E, S, one, qw)
    for kind, layer, ids, cap in ops:
        if kind == "d":
            a = oc.admit(layer, ids, cap)
            b = sp.step(layer, list(ids), cap)
            assert a.tolist() == b
        else:
            oc.prefetch(layer, ids)
            sp.prefetch(layer, list(ids))
            assert list(zip(oc.fill_slot.tolist(), oc.fill_expert.tolist())) == sp.fills, ops
        _same_state(oc, sp)


def test_brute_force_mixed_traces_tiny_caches():
    rng = np.random.default_rng(11)
    for _ in range(3000):
        L = int(rng.integers(1, 3))
        E = int(rng.integers(1, 6))
        S = int(rng.integers(1, 4))
        one = int(rng.integers(1, 4))
        qw = int(rng.integers(1, 4))
        ops = []
        for _ in range(int(rng.integers(1, 9))):
            R = int(rng.integers(0, 5))
            ids = rng.integers(-1, E + 1, R).astype(np.int32).tolist()
            kind = "p" if rng.random() < 0.4 else "d"
            ops.append((kind, int(rng.integers(0, L)), ids, int(rng.choice([-1, -1, 0, 1]))))
        _run_mixed(L, E, S, one, qw, ops)


def test_brute_force_mixed_traces_with_warm_experts():
    """Longer traces over few experts, so that frequencies pass 2 and the
    guard both protects and gives way."""
    rng = np.random.default_rng(12)
    for _ in range(300):
        L = int(rng.integers(1, 3))
        E = int(rng.integers(3, 12))
        S = int(rng.integers(2, 8))
        ops = []
        for _ in range(40):
            R = int(rng.integers(0, 6))
            hot = rng.random(R) < 0.6
            ids = np.where(hot, rng.integers(0, 2, R), rng.integers(-1, E + 1, R)).astype(np.int32).tolist()
            kind = "p" if rng.random() < 0.5 else "d"
            ops.append((kind, int(rng.integers(0, L)), ids, -1))
        _run_mixed(L, E, S, 256, 128, ops)


# ---------------------------------------------------------------- invariants

def test_prefetch_invariants_on_random_traces():
    rng = np.random.default_rng(13)
    L, E, S = 3, 64, 40
    oc = oracle.OracleCache(L, E, S)
    dropped_seen = filled_seen = 0
    for step in range(600):
        layer = int(rng.integers(0, L))
        if rng.random() < 0.5:
            R = int(rng.integers(0, 12))
            ids = np.minimum(rng.zipf(1.3, R) - 1, E + 2).astype(np.int32)
            oc.admit(layer, ids)
            continue
        n = int(rng.integers(0, 10))
        ids = rng.integers(-2, E + 2, n).astype(np.int32)
        before = oc.state()
        oc.prefetch(layer, ids)
        st = oc.state()
        if n == 0:
            continue
        assert st["clock"] == before["clock"] + 1
        now, ld = st["clock"], before["last_demand"]
        for k in ("freq", "dlast"):
            np.testing.assert_array_equal(st[k], before[k])
        assert st["last_demand"] == ld
        d = st["stats"][layer] - before["stats"][layer]
        want = sorted({int(e) for e in ids if 0 <= e < E})
        missing = [e for e in want if before["res"][layer * E + e] < 0]
        assert d[PF_CALLS] == 1 and d[PF_FILLED] + d[PF_DROPPED] == len(missing)
        assert oc.fill_expert.tolist() == [e for e in missing if st["res"][layer * E + e] >= 0]
        # fills: slots that were neither pinned nor predicted hits, now owned
        # by the prediction and stamped with this call's clock
        hits = {int(before["res"][layer * E + e]) for e in want if e not in missing}
        for s, e in zip(oc.fill_slot.tolist(), oc.fill_expert.tolist()):
            old_stamp = before["stamp"][s]
            assert not (old_stamp != 0 and old_stamp >= ld), "pinned slot chosen"
            assert s not in hits
            assert st["own"][s] == layer * E + e and st["stamp"][s] == now
        # pinned slots keep their owners
        pinned = (before["stamp"] != 0) & (before["stamp"] >= ld)
        np.testing.assert_array_equal(st["own"][pinned], before["own"][pinned])
        # res/own stay inverse maps
        for s in range(S):
            if st["own"][s] >= 0:
                assert st["res"][st["own"][s]] == s
        assert int((st["res"] >= 0).sum()) == int((st["own"] >= 0).sum())
        dropped_seen += int(d[PF_DROPPED])
        filled_seen += int(d[PF_FILLED])
    assert dropped_seen > 0 and filled_seen > 0
