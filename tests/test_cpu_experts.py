"""The hybrid decode step's CPU half (routes left at -1 computed on host
cores; FreeToken PR #491, sections 4-5) against the oracle, on the CPU.

moe_cpu_experts runs the library's host-thread expert pool on host arrays;
no device call is made.  Tolerance as for the GPU layer outputs: max |cpu -
oracle| <= 2e-2 * max |oracle| (fp32 sums, bf16 activation, against double
precision).  The result must not depend on the thread count."""
import numpy as np
import pytest

import expert_slot_cache_moe_amd as m
from expert_slot_cache_moe_amd import workloads as W
import oracle
from parity import check_close



def _case(seed, E, H, F, T, K, cpu_frac, fmt=0):
    g = W.rng(seed, "cpu-experts", E, H, T, fmt)
    banks = W.expert_rows(fmt, g, E, H, F)
    x = W.normal_bf16(g, (T, H))
    ids = np.stack([g.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
    cpu = np.where(g.random((T, K)) < cpu_frac, ids, -1).astype(np.int32)
    w = g.random((T, K)).astype(np.float32)
    return banks, x, cpu, w


@pytest.mark.parametrize("fmt", [0, 1, 2])
@pytest.mark.parametrize("E,H,F,T,K,frac", [
    (8, 64, 128, 1, 2, 1.0),          # the tiny layer, every route on the CPU
    (8, 64, 128, 5, 2, 0.5),          # ragged: some tokens have no CPU route
    (16, 256, 64, 7, 4, 0.4),
    (32, 2048, 512, 1, 8, 0.3),       # the shared-expert decode shape, one token
])
def test_cpu_routes_match_the_oracle(E, H, F, T, K, frac, fmt):
    banks, x, cpu, w = _case(1, E, H, F, T, K, frac, fmt)
    got = m.moe_cpu_experts(4, cpu, w, x, banks, H, F, fmt)
    ref = oracle.routed(oracle.Pool(fmt, H, F, banks), cpu, w.astype(np.float64), x)
    assert (got[(cpu < 0).all(axis=1)] == 0).all()       # tokens with no CPU route add nothing
    check_close(got, ref, "CPU experts")


def test_e2m1_rows_of_an_odd_number_of_scale_blocks():
    """E2M1 rows need only whole 16-element blocks: widths of 80 and 48
    leave an odd block after the pairs the vector loop takes."""
    E, H, F, T, K = 8, 80, 48, 3, 2
    banks, x, cpu, w = _case(5, E, H, F, T, K, 0.7, fmt=1)
    got = m.moe_cpu_experts(3, cpu, w, x, banks, H, F, 1)
    ref = oracle.routed(oracle.Pool(1, H, F, banks), cpu, w.astype(np.float64), x)
    check_close(got, ref, "CPU experts, E2M1, odd blocks")


@pytest.mark.parametrize("fmt", [0, 1, 2])
def test_result_does_not_depend_on_the_thread_count(fmt):
    banks, x, cpu, w = _case(2, 16, 256, 128, 6, 4, 0.7, fmt)
    outs = [m.moe_cpu_experts(n, cpu, w, x, banks, 256, 128, fmt) for n in (1, 2, 3, 8)]
    for o in outs[1:]:
        np.testing.assert_array_equal(o, outs[0])


def test_no_cpu_route_gives_zeros():
    banks, x, cpu, w = _case(3, 8, 64, 128, 3, 2, 0.0)
    assert (cpu < 0).all()
    got = m.moe_cpu_experts(2, cpu, w, x, banks, 64, 128)
    assert (got == 0).all()


def test_bad_sizes_are_rejected():
    banks, x, cpu, w = _case(4, 8, 64, 128, 1, 2, 1.0)
    with pytest.raises(m.MoeError):
        m.moe_cpu_experts(0, cpu, w, x, banks, 64, 128)
    with pytest.raises(m.MoeError):
        m.moe_cpu_experts(2, cpu, w, x[:, :40], banks, 40, 128)     # H % 16
    with pytest.raises(m.MoeError):
        m.moe_cpu_experts(2, cpu, w, x[:, :48], banks, 48, 128, m.MOE_FMT_MXFP4)   # H % 32
    with pytest.raises(m.MoeError):
        m.moe_cpu_experts(2, cpu, w, x, banks, 64, 128, 7)          # no such format
