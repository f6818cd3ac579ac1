"""Host logic of the benchmark's counter bookkeeping (CPU only): the per-launch
traffic of a kernel from two rocprofv3 counter files, each scaled by what it
reads for the run's first eight 256 MiB copies, and the source hash that keys a
summary to the kernels' code (comments do not count)."""
import csv
import json
import os

import pytest

import bench

FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size", "Kernel_Id",
          "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count",
          "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def _write(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, value) in enumerate(rows, 1):
            w.writerow({k: 0 for k in FIELDS} | dict(Dispatch_Id=i, Kernel_Name=name, Counter_Name=counter,
                                                     Counter_Value=value))


def test_summarize_counters_scales_by_the_first_copies(tmp_path, monkeypatch):
    copy = "__amd_rocclr_copyBuffer"
    kern = "void sv::k_row_stats<sv::BF16, true>(void const*, long)"
    # FETCH reads half of a copy's 262144 KiB; a later, larger copy must not
    # count as calibration
    fetch = [(copy, 131072.0)] * 8 + [(kern, 1000.0), (kern, 1002.0), (copy, 999999.0)]
    write = [(copy, 262144.0)] * 8 + [(kern, 4.0), (kern, 6.0), ("void sv::k_chain_draw<x>(y)", 77.0)]
    f, w = tmp_path / "f.csv", tmp_path / "w.csv"
    _write(f, "FETCH_SIZE", fetch)
    _write(w, "WRITE_SIZE", write)
    monkeypatch.setattr(bench, "traffic_file", lambda kernel, workload: str(tmp_path / "out.json"))
    bench.summarize_counters("c3", "k_row_stats", str(f), str(w))
    res = json.load(open(tmp_path / "out.json"))
    assert res["FETCH_SIZE"]["scale"] == pytest.approx(0.5)
    assert res["WRITE_SIZE"]["scale"] == pytest.approx(1.0)
    assert res["FETCH_SIZE"]["bytes_per_launch"] == pytest.approx(1001.0 / 0.5 * 1024)
    assert res["WRITE_SIZE"]["bytes_per_launch"] == pytest.approx(5.0 * 1024)
    assert res["bytes_per_launch"] == int(1001.0 / 0.5 * 1024 + 5.0 * 1024)
    assert res["kernel_source_sha1"] == bench.source_hash("k_row_stats")


def test_code_hash_ignores_comments_and_layout():
    a = "int f(int x) {  // the first\n  return x + 1; /* two\n lines */ }\n"
    b = "int f(int x) {\n\n  return x + 1;   }  // other words\n"
    c = "int f(int x) { return x + 2; }"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(c)


def test_every_committed_summary_names_its_kernel_and_workload():
    prof = os.path.join(bench.ROOT, "profiles")
    for name in os.listdir(prof):
        if name.endswith("_traffic.json"):
            d = json.load(open(os.path.join(prof, name)))
            assert name == os.path.basename(bench.traffic_file(d["kernel"], d["workload"]))
            assert d["bytes_per_launch"] > 0
