"""The CPU oracle for one offloaded MoE decode layer step.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this package; the product path never does.
It shares no code with the HIP library.  The arithmetic lives in
``moe_ref.c`` (plain C, double precision); this module only builds it and
marshals numpy arrays into it.
"""
from .ref import (  # noqa: F401
    build,
    lib,
    bf16_to_f64,
    e4m3_to_f64,
    e2m1_to_f64,
    e8m0_to_f64,
    query_widths,
    OracleCache,
    topk,
    expert_ffn,
    routed,
    shared,
    gather,
    Pool,
)
