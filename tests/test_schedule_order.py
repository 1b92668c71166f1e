"""The ordering of the layer-step schedules, on the CPU, with no device.

FreeToken issue #753 (section "Correctness evidence") backs its fork/join
with a CPU test over fake streams that fails when either the producer wait
or the consumer wait is removed.  Here the library itself records, instead
of issuing, every launch, event record and stream wait of a run of layer
steps (moe_trace_layer_steps: placeholder buffers, no GPU), with the
buffers each kernel reads and writes.  A vector-clock model of HIP streams
(in-order per stream; a wait orders its stream after everything before the
event's latest record) gives happens-before, and:

  - no two launches that touch the same buffer, one of them writing, are
    unordered (the slots a step's plan fills and the slots that already held
    their expert are disjoint within one step, so only those two parts may
    overlap in time);
  - every reader of slot bytes follows the step's writer of fresh slots
    (the gather, or stage 1's gather role); the next admission follows the
    previous gather and the previous prefetch copy; the launch that writes
    the output follows the writer of the shared term;
  - deleting any wait -- every instance of it, or just one in the middle of
    the run -- makes the check find a race.

All four schedules, one token and five-row steps, the three weight formats,
with and without a shared expert, with and without look-ahead prefetch."""
import itertools

import pytest

import expert_slot_cache_moe_amd as m

LAYERS, TOKENS = 3, 3


def _trace(overlap, T, fmt, shared, prefetch):
    H, F = 64, 128          # a shape with staged kernels in every format
    return m.moe_trace_layer_steps(num_layers=LAYERS, num_experts=16, num_slots=8, hidden=H, ffn=F,
                                   T=T, K=2, overlap=overlap, weight_format=fmt, with_shared=shared,
                                   prefetch_width=4 if prefetch else 0, tokens=TOKENS)


def _parse(lines):
    ops, step = [], None
    for ln in lines:
        f = ln.split()
        if f[0] in ("S", "P"):
            step = (f[0], int(f[1]), int(f[2]))
        elif f[0] == "J":
            step = ("J",)
        elif f[0] == "L":
            ops.append(dict(kind="L", stream=f[1], name=f[2], step=step,
                            reads=set(f[3].split(",")) - {"-"}, writes=set(f[4].split(",")) - {"-"}))
        else:
            ops.append(dict(kind=f[0], stream=f[1], event=f[2], step=step))
    return ops


def _clocks(ops):
    """Vector clocks: op b happens after op a iff b's clock has seen a's
    position on a's stream."""
    last, seq, recorded = {}, {}, {}
    for op in ops:
        s = op["stream"]
        vc = dict(last.get(s, {}))
        if op["kind"] == "W" and op["event"] in recorded:
            for k, v in recorded[op["event"]].items():
                vc[k] = max(vc.get(k, -1), v)
        seq[s] = seq.get(s, -1) + 1
        vc[s] = seq[s]
        op["seq"], op["vc"] = seq[s], vc
        last[s] = vc
        if op["kind"] == "E":
            recorded[op["event"]] = vc
    return ops


def _hb(a, b):
    return b["vc"].get(a["stream"], -1) >= a["seq"]


def _clash(x, y, same_step):
    if x == y:
        return True
    bx, by = x.split(":")[0], y.split(":")[0]
    if bx != by:
        return False
    if x == bx or y == by:          # all slots against a part of them
        return True
    return not same_step            # fresh against resident: disjoint within one step


def _conflict(a, b):
    same = a["step"] == b["step"]
    for xs, ys in ((a["writes"], b["writes"]), (a["writes"], b["reads"]), (a["reads"], b["writes"])):
        for x in xs:
            for y in ys:
                if _clash(x, y, same):
                    return (x, y)
    return None


def _races(ops):
    launches = [op for op in _clocks(ops) if op["kind"] == "L"]
    found = []
    for i, a in enumerate(launches):
        for b in launches[i + 1:]:
            c = _conflict(a, b)
            if c and not _hb(a, b):
                found.append((a["name"], a["stream"], a["step"], b["name"], b["stream"], b["step"], c))
    return found


CASES = list(itertools.product((0, 1, 2, 3), (1, 5), (0, 1, 2), (True, False), (False, True)))


@pytest.mark.parametrize("overlap,T,fmt,shared,prefetch", CASES)
def test_schedule_has_no_race_and_every_wait_is_needed(overlap, T, fmt, shared, prefetch):
    lines = _trace(overlap, T, fmt, shared, prefetch)
    ops = _parse(lines)
    assert not any("unknown" in op.get("reads", set()) | op.get("writes", set()) for op in ops)
    assert _races(ops) == []

    launches = [op for op in ops if op["kind"] == "L"]
    steps = sorted({op["step"] for op in launches if op["step"][0] == "S"})
    assert len(steps) == LAYERS * TOKENS
    for st in steps:
        mine = [op for op in launches if op["step"] == st]
        fills = [op for op in mine if any(w.startswith("slots") for w in op["writes"])]
        assert len(fills) == 1                      # one writer of the step's fresh slots
        readers = [op for op in mine if op is not fills[0] and any(r in ("slots", "slots:fresh")
                                                                    for r in op["reads"])]
        assert readers and all(_hb(fills[0], r) for r in readers)
        admit = [op for op in mine if op["name"] == "admit_kernel"]
        assert len(admit) == 1
        first = launches.index(mine[0])
        earlier = [op for op in launches[:first] if op["name"] in ("gather_kernel", "stage1_kernel")]
        assert all(_hb(op, admit[0]) for op in earlier)     # after every earlier gather and copy
        writers_out = [op for op in mine if "out" in op["writes"]]
        assert len(writers_out) == 1
        for op in mine:
            if "addend" in op["writes"]:
                assert _hb(op, writers_out[0])                # the shared term joins before the combine

    # every wait is load-bearing: without it the check finds a race
    waits = sorted({(op["stream"], op["event"]) for op in ops if op["kind"] == "W"})
    if overlap in (1, 3) and (shared or overlap == 1):
        assert ("side", "ready") in waits and ("compute", "done") in waits
    if prefetch:
        assert ("prefetch", "pf_ready") in waits and ("compute", "pf_done") in waits
    if overlap in (0, 2) and not prefetch:
        assert waits == []                          # one stream: nothing to join
    for site in waits:
        kept = [op for op in _parse(lines) if not (op["kind"] == "W" and (op["stream"], op["event"]) == site)]
        assert _races(kept), f"removing every wait {site} goes unnoticed"
        idx = [i for i, op in enumerate(_parse(lines))
               if op["kind"] == "W" and (op["stream"], op["event"]) == site and op["step"][1:] == (1, 1)]
        for i in idx:
            one = _parse(lines)
            del one[i]
            assert _races(one), f"removing the wait {site} of token 1, layer 1 goes unnoticed"


def test_the_checker_sees_an_unordered_pair():
    # two streams touching one buffer with no event between them
    ops = _parse(["S 0 0", "L compute a - buf", "L side b buf -"])
    assert _races(ops)
    ops = _parse(["S 0 0", "L compute a - buf", "E compute done", "W side done", "L side b buf -"])
    assert not _races(ops)
    # a wait before the record does not order anything
    ops = _parse(["S 0 0", "W side done", "L compute a - buf", "E compute done", "L side b buf -"])
    assert _races(ops)
    # fresh and resident slots of one step may overlap in time; of two steps, not
    ops = _parse(["S 0 0", "L side g - slots:fresh", "L compute r slots:resident -"])
    assert not _races(ops)
    ops = _parse(["S 0 0", "L side g - slots:fresh", "S 0 1", "L compute r slots:resident -"])
    assert _races(ops)


def test_trace_rejects_bad_arguments():
    with pytest.raises(m.MoeError):
        m.moe_trace_layer_steps(num_layers=1, num_experts=8, num_slots=4, hidden=64, ffn=128, T=1, K=2,
                                overlap=4)
    with pytest.raises(m.MoeError):
        m.moe_trace_layer_steps(num_layers=1, num_experts=8, num_slots=4, hidden=64, ffn=128, T=1, K=9,
                                overlap=0)


@pytest.mark.parametrize("fmt", [0, 1, 2])
def test_staged_schedule_covers_single_token_steps_of_every_format(fmt):
    """Schedule 2 runs a one-token step as admission + two stage launches
    in bf16, E2M1 and MXFP4 alike; wider steps and other schedules keep the
    separate gather."""
    for H, F in ((64, 128), (2048, 512), (1024, 256)):
        ops = _parse(m.moe_trace_layer_steps(num_layers=1, num_experts=32, num_slots=12, hidden=H, ffn=F,
                                             T=1, K=8, overlap=2, weight_format=fmt, tokens=1))
        assert [op["name"] for op in ops if op["kind"] == "L"] == ["admit_kernel", "stage1_kernel",
                                                                  "stage2_kernel"]
    ops = _parse(m.moe_trace_layer_steps(num_layers=1, num_experts=32, num_slots=12, hidden=64, ffn=128,
                                         T=3, K=2, overlap=2, weight_format=fmt, tokens=1))
    assert "gather_kernel" in [op["name"] for op in ops]

