"""Pins for the oracle's slot-cache admission (CPU only).

Each test ties the C oracle to something other than itself: counts and
widths the pages print (tests/golden), an independently written
recency-list model (tests/spec_lru.py) run exhaustively on tiny caches,
and invariants the pages fix, checked after every step of random traces.
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle
from spec_lru import SpecCache

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _same_state(oc: oracle.OracleCache, spec: SpecCache):
    a, b = oc.state(), spec.arrays()
    for k in ("res", "own", "stamp", "stats", "freq"):
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)
    assert a["clock"] == b["clock"]


# ---------------------------------------------------------------- pins from the pages

def test_query_widths_printed_on_the_pages():
    g = _golden("wide_step_admission.json")
    for case in g["cases"]:
        got = oracle.query_widths(case["routes"], case["experts"], g["one_call_width"], g["query_width"])
        assert got == case["query_widths"], case["what"]


def test_query_widths_one_call_boundary_is_inclusive():
    assert oracle.query_widths(256, 512) == [256]
    assert oracle.query_widths(257, 512) == [128, 128, 1]
    # The distinct list has the fixed length min(R, E): 480 and 1280 routes
    # over 512 experts give 4 queries each.
    assert oracle.query_widths(480, 512) == [128, 128, 128, 96]
    assert oracle.query_widths(1280, 512) == [128] * 4


def _wide_step_routes(rng, rows, experts):
    """rows x top-2 routes that together name every expert at least once."""
    ids = np.empty((rows, 2), np.int32)
    perm = rng.permutation(experts)
    for r in range(rows):
        if 2 * r + 1 < experts:
            ids[r] = perm[2 * r], perm[2 * r + 1]
        else:
            ids[r] = rng.choice(experts, 2, replace=False)
    return ids.reshape(-1)


def test_wide_step_statistics_printed_on_the_pages():
    g = _golden("wide_step_admission.json")
    case = g["cases"][0]
    E, R = case["experts"], case["routes"]
    rng = np.random.default_rng(1)
    oc = oracle.OracleCache(1, E, E, g["one_call_width"], g["query_width"])
    resident = rng.choice(E, case["resident_before"], replace=False).astype(np.int32)
    oc.admit(0, resident)
    before = oc.state()
    ids = _wide_step_routes(rng, case["rows"], E)
    assert ids.size == R and len(set(ids.tolist())) == E
    out = oc.admit(0, ids)
    after = oc.state()
    d = after["stats"][0] - before["stats"][0]
    assert d[1] == case["stats"]["met"]
    assert d[2] == case["stats"]["missed"]
    assert d[0] == case["stats"]["calls"]
    assert d[3] == 0 and d[4] == 0
    assert int((after["freq"] - before["freq"]).sum()) == case["histogram_total"]
    np.testing.assert_array_equal(after["freq"] - before["freq"], np.bincount(ids, minlength=E))
    # every route decodes at its expert's slot
    assert (out >= 0).all()
    np.testing.assert_array_equal(after["own"][out], ids)
    # queries of 128 then 32: the plan lists the first 128 distinct experts'
    # misses before the remaining 32's, each part ascending
    D = np.arange(E)
    first = set(D[:128].tolist()) - set(resident.tolist())
    pe = oc.plan_expert.tolist()
    assert len(pe) == case["stats"]["missed"]
    assert set(pe[: len(first)]) == first and pe == sorted(pe)


def test_eight_route_step_is_one_admission_in_place():
    rng = np.random.default_rng(2)
    oc = oracle.OracleCache(1, 160, 160)
    ids = rng.choice(160, 8, replace=False).astype(np.int32)
    out = oc.admit(0, ids)
    st = oc.state()
    assert st["stats"][0][0] == 1
    np.testing.assert_array_equal(out, st["res"][ids])
    assert oracle.query_widths(8, 160) == [8]


def test_route_split_worked_example():
    g = _golden("route_split_example.json")
    oc = oracle.OracleCache(1, 64, 4)
    oc.admit(0, [0, 1, 2])       # slots 0, 1, 2
    oc.admit(0, [11])            # expert 11 -> slot 3
    out = oc.admit(0, g["original_expert_ids"], max_fetch=0)   # 42 gets no slot
    assert out.tolist() == g["cache_result"]
    cpu_ids = [e if s < 0 else -1 for e, s in zip(g["original_expert_ids"], out)]
    assert cpu_ids == g["cpu_expert_ids"]


# ---------------------------------------------------------------- brute force

def _run_both(L, E, S, one, qw, steps):
    oc = oracle.OracleCache(L, E, S, one, qw)
    sp = SpecCache(L, E, S, one, qw)
    for layer, ids, cap in steps:
        a = oc.admit(layer, ids, cap)
        b = sp.step(layer, list(ids), cap)
        assert a.tolist() == b, (steps, layer, ids, cap)
        assert list(zip(oc.plan_slot.tolist(), oc.plan_expert.tolist())) == sp.plan
        _same_state(oc, sp)


def test_brute_force_every_short_sequence():
    """Every 2-step sequence of 0..2 routes over ids {-1,0,1,2} (E=3, S=2,
    one layer) at every width pair in {1,2,3}^2 and caps {-1,0,1}; then
    every 3-route second step after a few first steps."""
    alphabet = [-1, 0, 1, 2]
    short = [list(p) for n in range(0, 3) for p in itertools.product(alphabet, repeat=n)]
    three = [list(p) for p in itertools.product(alphabet, repeat=3)]
    for one, qw in itertools.product([1, 2, 3], repeat=2):
        for a in short:
            for b in short:
                for cap in (-1, 0, 1):
                    _run_both(1, 3, 2, one, qw, [(0, a, -1), (0, b, cap)])
    for one, qw in [(1, 1), (2, 1), (3, 2)]:
        for a in ([], [0], [2, 1], [0, 0], [-1, 2]):
            for b in three:
                for cap in (-1, 0, 1):
                    _run_both(1, 3, 2, one, qw, [(0, a, -1), (0, b, cap)])


def test_brute_force_random_tiny_caches():
    rng = np.random.default_rng(3)
    for _ in range(4000):
        L = int(rng.integers(1, 3))
        E = int(rng.integers(1, 5))
        S = int(rng.integers(1, 4))
        one = int(rng.integers(1, 4))
        qw = int(rng.integers(1, 4))
        steps = []
        for _ in range(int(rng.integers(1, 4))):
            R = int(rng.integers(0, 5))
            ids = rng.integers(-1, E + 1, R).astype(np.int32).tolist()
            steps.append((int(rng.integers(0, L)), ids, int(rng.choice([-1, 0, 1]))))
        _run_both(L, E, S, one, qw, steps)


def test_brute_force_random_medium_caches():
    rng = np.random.default_rng(4)
    for _ in range(200):
        L = int(rng.integers(1, 4))
        E = int(rng.integers(4, 40))
        S = int(rng.integers(2, 50))
        one = int(rng.integers(1, 20))
        qw = int(rng.integers(1, 12))
        steps = []
        for _ in range(8):
            R = int(rng.integers(0, 60))
            ids = rng.integers(-2, E + 2, R).astype(np.int32).tolist()
            steps.append((int(rng.integers(0, L)), ids, int(rng.choice([-1, -1, 0, 3]))))
        _run_both(L, E, S, one, qw, steps)


# ---------------------------------------------------------------- invariants

def _check_invariants(oc, before, layer, ids_in, out, cap):
    st = oc.state()
    E, S = oc.E, oc.S
    res, own = st["res"], st["own"]
    # res/own are inverse maps on resident entries
    for s in range(S):
        if own[s] >= 0:
            assert res[own[s]] == s
    for le in np.nonzero(res >= 0)[0]:
        assert own[res[le]] == le
    valid = (ids_in >= 0) & (ids_in < E)
    # a hit maps to a slot holding that expert
    ok = out >= 0
    assert (own[out[ok]] == layer * E + ids_in[ok]).all()
    assert (~valid <= (out < 0)).all()
    # -1 only for invalid ids or overflowed misses
    dstats = st["stats"][layer] - before["stats"][layer]
    overflowed = set(ids_in[valid & (out < 0)].tolist())
    assert len(overflowed) == dstats[3]
    if cap < 0 and len(set(ids_in[valid].tolist())) <= S:
        assert dstats[3] == 0 and (out[valid] >= 0).all()
    # one call; met = distinct valid; histogram = every valid route
    assert dstats[0] == 1
    assert dstats[1] == len(set(ids_in[valid].tolist()))
    assert dstats[4] == int((~valid).sum())
    assert int((st["freq"] - before["freq"]).sum()) == int(valid.sum())
    # every used slot carries this step's stamp; plan rows are distinct
    now = st["clock"]
    assert now == before["clock"] + 1
    assert (st["stamp"][out[ok]] == now).all()
    ps, pe = oc.plan_slot, oc.plan_expert
    assert len(set(ps.tolist())) == ps.size and len(set(pe.tolist())) == pe.size
    assert (own[ps] == layer * E + pe).all()
    assert ps.size <= min(ids_in.size, E)
    if cap >= 0:
        assert ps.size <= cap


@pytest.mark.parametrize("one,qw", [(256, 128), (3, 3), (1, 1), (40, 16)])
def test_invariants_on_random_traces(one, qw):
    rng = np.random.default_rng(5 + one + qw)
    L, E, S = 3, 96, 120
    oc = oracle.OracleCache(L, E, S, one, qw)
    for step in range(300):
        layer = int(rng.integers(0, L))
        R = int(rng.integers(0, 200))
        ids = rng.integers(-3, E + 3, R).astype(np.int32)
        cap = int(rng.choice([-1, -1, -1, 0, 5]))
        before = oc.state()
        out = oc.admit(layer, ids, cap)
        _check_invariants(oc, before, layer, ids, out, cap)
