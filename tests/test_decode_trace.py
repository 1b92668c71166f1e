"""The synthetic decode trace's temporal locality, on the CPU.

The shared-expert decode page reports about 28 expert misses per token for
its setup: 40 MoE layers x 256 experts, top-8, a 3164-slot cache, batch 1
(FreeToken issue #753, section Setup).  The trace's `stay` probability is
set so that the oracle's admission, after the bench's 64-token cache
warm-up, lands there."""
import numpy as np

import oracle
from expert_slot_cache_moe_amd.workloads import DecodeTrace


def _misses_per_token(stay, warm=64, measure=128, seed=0):
    tr = DecodeTrace(seed, 40, 256, 8, stay=stay)
    oc = oracle.OracleCache(40, 256, 3164)
    counts = []
    for _ in range(warm + measure):
        sets = tr.step_sets()
        before = oc.stats[:, 2].sum()
        for l in range(40):
            oc.admit(l, sets[l])
        counts.append(oc.stats[:, 2].sum() - before)
    return float(np.mean(counts[warm:]))


def test_default_trace_gives_about_28_misses_per_token():
    assert abs(_misses_per_token(0.73) - 28.0) <= 2.0


def test_more_locality_gives_fewer_misses():
    # the calibration knob moves the figure the right way
    assert _misses_per_token(0.85, measure=48) < _misses_per_token(0.73, measure=48) - 5
