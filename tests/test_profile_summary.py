"""The rocprofv3 CSV summaries behind the files in profiles/ (host logic only)."""

import os

from memory_bound_transformer_decode_amd import profile_summary as ps


def _write(tmp_path, name, header, rows):
    d = tmp_path / "run" / "host"
    d.mkdir(parents=True, exist_ok=True)
    with open(d / name, "w") as f:
        f.write(",".join(header) + "\n")
        for r in rows:
            f.write(",".join(str(x) for x in r) + "\n")
    return str(tmp_path / "run")


def test_stats_match_keeps_only_matching_kernels(tmp_path, capsys):
    d = _write(tmp_path, "run_kernel_stats.csv",
               ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs"],
               [["setup_fill", 10, 9000, 900, 60.0, 800, 1000],
                ["dec::k_attn", 4, 4000, 1000, 26.7, 900, 1100],
                ["dec::k_gemv", 2, 2000, 1000, 13.3, 950, 1050]])
    ps.main(["stats", d, "--command", "cmd", "--match", "dec::"])
    out = capsys.readouterr().out
    assert "setup_fill" not in out
    rows = [l for l in out.splitlines() if l.startswith("| `")]
    assert [r.split("`")[1] for r in rows] == ["dec::k_attn", "dec::k_gemv"]  # by total time


def test_counters_mean_per_dispatch(tmp_path, capsys):
    d = _write(tmp_path, "run_counter_collection.csv",
               ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"],
               [[1, "dec::k_attn", "SQ_WAVES", 10], [1, "dec::k_attn", "SQ_BUSY", 4],
                [2, "dec::k_attn", "SQ_WAVES", 30], [2, "dec::k_attn", "SQ_BUSY", 8],
                [3, "other", "SQ_WAVES", 1000]])
    ps.main(["counters", d, "--command", "cmd", "--match", "dec::"])
    out = capsys.readouterr().out
    assert "other" not in out
    header = [l for l in out.splitlines() if l.startswith("| kernel")][0]
    assert header.split("|")[3].strip() == "SQ_BUSY"
    row = [l for l in out.splitlines() if l.startswith("| `dec::k_attn")][0]
    cells = [c.strip() for c in row.split("|")]
    assert cells[2] == "2" and cells[3] == "6" and cells[4] == "20"


def test_markers_per_range_without_the_first_calls(tmp_path, capsys):
    d = _write(tmp_path, "run_marker_api_trace.csv",
               ["Domain", "Function", "Process_Id", "Thread_Id", "Correlation_Id", "Start_Timestamp",
                "End_Timestamp"],
               [["MARKER_CORE_RANGE_API", "dec_step", 1, 1, 1, 0, 50000000],  # capture: left out
                ["MARKER_CORE_RANGE_API", "dec_step", 1, 1, 2, 60000000, 60002000],
                ["MARKER_CORE_RANGE_API", "dec_step", 1, 1, 3, 70000000, 70004000],
                ["MARKER_CORE_RANGE_API", "dec_step", 1, 1, 4, 80000000, 80003000],
                ["MARKER_CORE_RANGE_API", "dec_prefill", 1, 1, 5, 0, 1000]])
    ps.main(["markers", d, "--command", "cmd"])
    out = capsys.readouterr().out
    assert "dec_prefill" not in out  # its only call is the left-out first one
    row = [l for l in out.splitlines() if l.startswith("| `dec_step")][0]
    cells = [c.strip() for c in row.split("|")]
    assert cells[2] == "3" and cells[3] == "3.0" and cells[4] == "3.0" and cells[5] == "2.0" and cells[6] == "4.0"
