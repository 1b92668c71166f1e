"""Host-side logic of bench.py, on the CPU: the in-graph input staging and
the counter summary (no device call)."""
import csv

import torch

import bench


def test_stage_inputs_copies_the_counters_row_and_advances_it():
    x_all = torch.arange(5 * 3 * 2, dtype=torch.int16).view(5, 3, 1, 2)
    lg_all = torch.randn(5, 3, 1, 4)
    x_st = torch.empty((3, 1, 2), dtype=torch.int16)
    lg_st = torch.empty((3, 1, 4))
    step = torch.tensor([2], dtype=torch.int64)
    for t in (2, 3, 4):
        bench.stage_inputs(torch, ((x_all, x_st), (lg_all, lg_st)), step)
        assert torch.equal(x_st, x_all[t]) and torch.equal(lg_st, lg_all[t])
        assert int(step) == t + 1


def test_counter_summary_keeps_template_arguments_and_derives_per_wave_figures(tmp_path, capsys):
    name = "void moe::mfma_detail::up_mfma_kernel<1, 1, 3>(moe::PoolView, moe::Items, unsigned short const*, unsigned short*)"
    rows = [("SQ_WAVES", 100.0), ("SQ_WAVE_CYCLES", 1000.0), ("SQ_WAIT_INST_ANY", 400.0),
            ("SQ_ACTIVE_INST_VALU", 200.0), ("SQ_INSTS_VALU", 5000.0), ("SQ_INSTS_MFMA", 800.0)]
    path = tmp_path / "c.csv"
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Counter_Name", "Counter_Value"])
        for c, v in rows:
            w.writerow([name, c, v])
            w.writerow([name, c, v])            # two dispatches, the same values
    bench.summarize_counters([str(path)])
    out = capsys.readouterr().out
    assert "up_mfma_kernel<1, 1, 3>  (dispatches 2)" in out
    assert ("up_mfma_kernel<1, 1, 3>: 100 waves a dispatch; stalled on outstanding loads 40% of wave "
            "cycles, VALU issuing 20%; 50 VALU and 8 MFMA instructions per wave") in out


def test_token_plan_warms_the_cache_whatever_warmup_is_given():
    # the driver's short run: 5 warm-up tokens asked for, 20 timed
    n_warm, n_tok, first = bench.token_plan(5, 20)
    assert n_warm == bench.CACHE_WARM_TOKENS == 64
    assert (n_tok, first) == (84, 64)
    # a longer warm-up than the cache needs is kept
    assert bench.token_plan(100, 7) == (100, 107, 100)


def test_replay_legs_never_index_past_the_trace():
    for warmup, steps in ((5, 20), (0, 1), (64, 256), (3, 40)):
        n_warm, n_tok, first = bench.token_plan(warmup, steps)
        timed = bench.leg_tokens(first, n_tok)
        assert list(timed) == list(range(first, first + steps))
        hyb = bench.leg_tokens(first, n_tok, bench.HYBRID_TOKENS)
        assert len(hyb) == min(steps, bench.HYBRID_TOKENS)
        assert all(0 <= t < n_tok for t in hyb)


def test_a_failing_side_leg_becomes_an_error_field():
    def broken():
        raise IndexError("index 25 is out of bounds")

    assert bench.run_leg("x", broken) == {"error": "IndexError: index 25 is out of bounds"}
    assert bench.run_leg("y", lambda a, b=0: a + b, 2, b=3) == 5
