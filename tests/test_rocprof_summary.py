"""Host logic of the profile summaries (rocprof_summary): counter tables, byte
scaling against the copy probe, the traffic record the bench reads, and the
per-grid launch table of a kernel trace.  Synthetic CSVs in the rocprofv3
column layout; no GPU."""

import csv
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from lossless_speculative_drafting_amd import rocprof_summary as rs  # noqa: E402

COUNTER_FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def _counter_csv(path, dispatches):
    """dispatches: [(id, kernel name, duration ns, {counter: value or [values per dimension]})]"""
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=COUNTER_FIELDS)
        w.writeheader()
        for d, name, dur, ctrs in dispatches:
            for cn, v in ctrs.items():
                for part in (v if isinstance(v, list) else [v]):
                    w.writerow({"Dispatch_Id": d, "Kernel_Name": name, "Counter_Name": cn, "Counter_Value": part,
                                "Start_Timestamp": 1000, "End_Timestamp": 1000 + dur})
    return path


def test_counters_scale_bytes_by_the_copy_probe_and_derive_clock_and_mfma(tmp_path, capsys):
    # copy probe: 1 MiB copied, FETCH reads half (512 KiB), WRITE reads it exactly
    cf = _counter_csv(str(tmp_path / "cf" / "p.csv"), [(1, "__amd_rocclr_copyBuffer", 1000, {"FETCH_SIZE": 512.0})])
    cw = _counter_csv(str(tmp_path / "cw" / "p.csv"), [(1, "__amd_rocclr_copyBuffer", 1000, {"WRITE_SIZE": 1024.0})])
    # two dispatches of one kernel, 10 us each, a 2 GHz clock on 8 XCDs (GRBM adds them up),
    # MFMA busy 40% of 256 CUs x 4 SIMDs; FETCH given per dimension (summed)
    cyc = 20000.0
    ctr = {"FETCH_SIZE": [100.0, 100.0], "WRITE_SIZE": 50.0, "GRBM_GUI_ACTIVE": 8 * cyc,
           "SQ_VALU_MFMA_BUSY_CYCLES": 0.4 * cyc * 256 * 4, "TCC_HIT_sum": 75.0, "TCC_MISS_sum": 25.0,
           "SQ_INSTS_VALU_MFMA_MOPS_BF16": 1e6}
    run = _counter_csv(str(tmp_path / "run1" / "p.csv"),
                       [(7, "void gated_gemm_kernel<128, 128>(x)", 10000, ctr),
                        (8, "void gated_gemm_kernel<128, 128>(x)", 10000, ctr),
                        (9, "void other_kernel()", 5000, {"FETCH_SIZE": 1.0})])
    rs.main(["counters", run, "--group", "gemm=gated_gemm_kernel", "--copy-fetch", cf, "--copy-write", cw,
             "--copy-mib", "1"])
    out = capsys.readouterr().out
    row = next(ln for ln in out.splitlines() if ln.startswith("| gemm"))
    assert "| 2 | 10.00 |" in row                    # two dispatches, 10 us each
    assert "FETCH_SIZE 0.41 MB (scaled)" in row      # 200 KiB x 2 (the probe's scale) = 409600 B
    assert "WRITE_SIZE 0.05 MB (scaled)" in row      # 50 KiB x 1
    assert "2000 MHz" in row                         # 8 x 20000 cycles / 8 XCDs / 10 us
    assert "MFMA busy 40.0%" in row
    assert "L2 hit 75.0%" in row
    assert "512.0 GFLOP" not in row and "0.5 GFLOP" in row  # 1e6 MOPs x 512 flop


def test_traffic_record_sums_the_reduction_into_its_launch(tmp_path, capsys):
    cf = _counter_csv(str(tmp_path / "cf" / "p.csv"), [(1, "copy", 1000, {"FETCH_SIZE": 512.0})])
    cw = _counter_csv(str(tmp_path / "cw" / "p.csv"), [(1, "copy", 1000, {"WRITE_SIZE": 1024.0})])
    main, red = "gated_gemm_kernel<256, 256, 2, 4, 64, false, false, 0, 3, 1>", "splitk_reduce_kernel<false>"
    seq = [(1, main, 1, 100.0), (2, red, 1, 10.0), (3, main, 1, 300.0), (4, "row_stats_kernel", 1, 999.0)]
    fe = _counter_csv(str(tmp_path / "fe" / "p.csv"), [(d, n, t, {"FETCH_SIZE": v}) for d, n, t, v in seq])
    wr = _counter_csv(str(tmp_path / "wr" / "p.csv"), [(d, n, t, {"WRITE_SIZE": v / 10}) for d, n, t, v in seq])
    out_json = str(tmp_path / "traffic.json")
    rs.main(["traffic", "--fetch", fe, "--write", wr, "--copy-fetch", cf, "--copy-write", cw, "--copy-mib", "1",
             "--key", "gated_gemm", "--launch", ", false, false,", "--also", red, "--source", "gemm.hip",
             "--out", out_json])
    rec = json.load(open(out_json))["gated_gemm"]
    # launches: (100 + 10) and 300 KiB fetched -> mean 205 KiB x 2; writes (10 + 1) and 30 -> 20.5 KiB x 1
    assert rec["launches"] == [2, 2]
    assert rec["fetch_kib_per_launch_raw"] == pytest.approx(205.0)
    assert rec["bytes_per_launch"] == round(205.0 * 1024 * 2 + 20.5 * 1024 * 1)
    assert rec["source_digest"] == rs.source_digest(["gemm.hip"])


def test_bench_reads_traffic_only_for_the_code_it_was_taken_on():
    import bench
    path = os.path.join(ROOT, "profiles", "traffic.json")
    rec = json.load(open(path))["gated_gemm"]
    assert bench.committed_traffic("gated_gemm", rec["source_digest"]) == rec["bytes_per_launch"]
    assert bench.committed_traffic("gated_gemm", "0" * 16) is None
    assert bench.committed_traffic("no_such_kernel", rec["source_digest"]) is None
    # the bench's digest and the summary tool's digest are the same function of the sources
    assert bench.source_digest("gemm.hip") == rs.source_digest(["gemm.hip"])


def test_trace_table_groups_launches_by_kernel_and_grid(tmp_path, capsys):
    fields = ["Kind", "Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X", "Grid_Size_Y",
              "Grid_Size_Z", "Workgroup_Size_X"]
    path = str(tmp_path / "kt.csv")
    rows = [(1, "void k<1>(int)", 0, 4000, 512), (2, "void k<1>(int)", 0, 2000, 512), (3, "void k<1>(int)", 0, 9000, 1024),
            (4, "void other()", 0, 1000, 64)]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for d, n, s, e, g in rows:
            w.writerow({"Kind": "KERNEL_DISPATCH", "Dispatch_Id": d, "Kernel_Name": n, "Start_Timestamp": s,
                        "End_Timestamp": e, "Grid_Size_X": g, "Grid_Size_Y": 1, "Grid_Size_Z": 1,
                        "Workgroup_Size_X": 256})
    rs.main(["trace", path, "--match", "k<1>", "--calls"])
    lines = capsys.readouterr().out.splitlines()
    g512 = next(ln for ln in lines if "| 512 |" in ln)
    assert "| 2 | 3.00 |" in g512                    # two launches of 4 and 2 us
    assert any("calls in order: 4.0 2.0" in ln for ln in lines)
    assert any("| 1024 |" in ln and "| 1 | 9.00 |" in ln for ln in lines)
    assert not any("other" in ln for ln in lines)
