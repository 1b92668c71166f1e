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
