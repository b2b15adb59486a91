"""Host logic of bench.py's profile summary: a synthetic rocprofv3 kernel
trace is split per kernel into the dispatches that follow the abs-max
pre-pass and those that do not (the bench's roofline averages the latter)."""
import csv
import importlib.util
import json
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def write_csv(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_summary_splits_launches_by_the_pre_pass(tmp_path, monkeypatch):
    bench = load_bench()
    out_dir = tmp_path / "profiles"
    monkeypatch.setattr(bench, "PROFILES", str(out_dir))
    run = tmp_path / "run"
    run.mkdir()
    amax, bf = "void k_amax<float, 0>(AmaxArgs)", "void k_quant_bf<float, 4, 0, 1>(QuantArgs)"
    # dispatch order (start time, name, duration in ns); listed out of order on purpose
    trace = [(5000, bf, 300), (0, bf, 100), (1000, amax, 10), (2000, bf, 200), (3000, bf, 120), (4000, amax, 12)]
    write_csv(run / "x_kernel_trace.csv", ["Kernel_Name", "Start_Timestamp", "End_Timestamp"],
              [(n, t, t + d) for t, n, d in trace])
    write_csv(run / "x_kernel_stats.csv",
              ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs"],
              [(bf, 4, 720, 180, 97.0, 100, 300), (amax, 2, 22, 11, 3.0, 10, 12)])
    bench.summarize([str(run)], "unit_label", "synthetic")
    d = json.load(open(out_dir / "unit_label.json"))
    split = d["split"][bf]
    # without the pre-pass: t=0 (first) and t=3000 (after a bf launch)
    assert split["without_amax"] == {"dispatches": 2, "avg_us": (0.100 + 0.120) / 2}
    # right after k_amax: t=2000 and t=5000
    assert split["after_amax"] == {"dispatches": 2, "avg_us": (0.200 + 0.300) / 2}
    assert d["split"][amax]["without_amax"]["dispatches"] == 2
    md = open(out_dir / "unit_label.md").read()
    assert "| 2 | 0.11 | 2 | 0.25 |" in md
