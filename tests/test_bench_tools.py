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


# ---- in-kernel time lines (records built by hand: 100 ticks per us) ----

def _tick(us):
    return int(round(1_000_000 + us * 100))


def test_timeline_walk_phases_from_records():
    import numpy as np
    B, G = 2, 2
    A = np.zeros((16384, 64), dtype=np.int64)
    for b in range(B):
        for g in range(G):
            r = A[b * G + g]
            r[0], r[1] = _tick(0.5 * g), _tick(1.0 + 0.5 * g)
            t = 2.0
            nx = 2 + b  # request 0: two exchanges, request 1: three
            for x in range(nx):
                s = 2 + 6 * x
                for j, d in enumerate((0.0, 1.0, 0.25, 0.5, 0.1, 0.3)):
                    t += d
                    r[s + j] = _tick(t + g * 0.1)
                t += 0.7  # the next child's test
            r[61], r[62], r[63] = _tick(t), _tick(t + 0.4), _tick(t + 2.9)
    out = bench.timeline_walk(A, B)
    assert out["workgroups_per_request"] == G and out["rounds"] == dict(mean=2.5, max=3)
    ph = out["phases_us"]
    assert ph["pass"]["n"] == 5 and ph["pass"]["p50"] == pytest.approx(1.0)
    # the slowest workgroup stores its words 0.1 us later than the other
    assert ph["exchange"]["p50"] == pytest.approx(0.5)
    assert ph["fold_waves"]["p50"] == pytest.approx(0.25) and ph["fold_words"]["p50"] == pytest.approx(0.3)
    assert ph["decide"]["n"] == 3 and ph["decide"]["p50"] == pytest.approx(0.7)
    assert out["last_draw_us"]["tile_search"]["p50"] == pytest.approx(0.4)
    assert out["last_draw_us"]["pick_and_write"]["p50"] == pytest.approx(2.5)
    assert out["slowest_request"]["index"] == 1 and len(out["slowest_request"]["exchanges"]) == 3
    md = bench.timeline_markdown(dict(timeline="walk", step="s", unit="us", **out))
    assert "| phases_us.pass | 1.00" in md and "slowest_request.exchanges:" in md


def _draw_records(n, t_start, last_every):
    import numpy as np
    D = np.zeros((16384, 64), dtype=np.int64)
    for i in range(n):
        t = t_start + 0.01 * i
        pts = [t, t + 2.0, t + 10.0, t + 10.5]
        if i % last_every == last_every - 1:
            pts += [t + 12.0, t + 12.75, t + 15.25, t + 15.75]
        for j, v in enumerate(pts):
            D[i, j] = _tick(v)
    return D


def test_timeline_chain_phases_from_records():
    import numpy as np
    S = np.zeros((16384, 64), dtype=np.int64)
    for i in range(100):
        S[i, 0], S[i, 1] = _tick(0.2 * i), _tick(0.2 * i + 3.5)
    D = _draw_records(32, 25.0, 8)
    out = bench.timeline_chain(S, D, 100, 32)
    st = out["stats"]
    assert st["first_start"] == 0.0 and st["last_start"] == pytest.approx(19.8)
    assert st["last_end"] == pytest.approx(23.3) and st["block_us"]["p50"] == pytest.approx(3.5)
    dr = out["draw"]
    assert dr["first_start"] == pytest.approx(25.0) and dr["break_row_us"]["p50"] == pytest.approx(2.0)
    assert dr["tiles_us"]["p50"] == pytest.approx(8.0) and dr["count_us"]["p50"] == pytest.approx(0.5)
    lb = dr["last_block"]
    assert lb["gather_us"]["n"] == 4 and lb["gather_us"]["p50"] == pytest.approx(1.5)
    assert lb["find_tile_us"]["p50"] == pytest.approx(0.75) and lb["pick_us"]["p50"] == pytest.approx(2.5)
    assert lb["write_us"]["p50"] == pytest.approx(0.5)
    assert dr["last_end"] == pytest.approx(25.0 + 0.31 + 15.75)


def test_timeline_ragged_rows_from_records():
    import numpy as np
    rows, per_row = 3, 10
    L = np.zeros((65536, 4), dtype=np.int64)
    for i in range(rows):
        for j in range(per_row):
            r = L[i * per_row + j]
            t = 5.0 * i + 0.1 * j
            r[0] = _tick(t)
            if j < per_row >> i:  # row 0 all, row 1 half, row 2 a fifth
                r[1], r[2] = _tick(t + 0.05), _tick(t + 2.0)
                if j == (per_row >> i) - 1:
                    r[3] = _tick(t + 3.0)
    D = _draw_records(8, 20.0, 4)
    out = bench.timeline_ragged(L, D, rows, per_row, 8)
    st = out["stats"]
    assert out["stats_blocks"] == 30 and st["blocks_not_loading"] == 30 - (10 + 5 + 2)
    assert [r["loaded"] for r in st["rows"]] == [10, 5, 2]
    assert [r["decided"] for r in st["rows"]] == [1, 1, 1]
    assert st["rows"][1]["start_first"] == pytest.approx(5.0) and st["rows"][1]["start_last"] == pytest.approx(5.9)
    assert st["rows"][2]["loaded_end_last"] == pytest.approx(10.1 + 2.0)
    assert st["last_stamp"] == pytest.approx(10.1 + 3.0)  # row 2's decision
    assert out["draw"]["last_block"]["end_at"]["n"] == 2
    md = bench.timeline_markdown(dict(timeline="ragged", step="s", unit="us", **out))
    assert "| row | blocks | loaded |" in md
