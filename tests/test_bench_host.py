"""CPU tests of bench.py's host logic: argument contract, trace and counter summaries, the
traffic line's source gating. No GPU: nothing here imports torch's device side or the library."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_defaults_fit_the_contract():
    a = bench.parse_args([])
    assert a.gpus == 1 and a.steps > 0 and a.warmup >= 0 and a.workload is None


def write_trace(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for name, start, end in rows:
            w.writerow({"Kernel_Name": name, "Start_Timestamp": start, "End_Timestamp": end})


def test_summarize_trace_statistics(tmp_path):
    p = tmp_path / "trace_kernel_trace.csv"
    write_trace(p, [("k1", 0, 10), ("k1", 100, 130), ("k1", 200, 220), ("k2", 0, 5), ("k2", 9, 16)])
    r = run_bench("--summarize-trace", str(p))
    assert r.returncode == 0, r.stderr
    rows = {d["kernel"]: d for d in map(json.loads, r.stdout.splitlines())}
    assert rows["k1"] == {"kernel": "k1", "count": 3, "mean_ns": 20.0, "median_ns": 20,
                          "min_ns": 10, "max_ns": 30}
    assert rows["k2"]["count"] == 2 and rows["k2"]["median_ns"] == 6.0
    # ordered by total time, largest first
    assert list(rows) == ["k1", "k2"]


def write_counters(folder, run, rows):
    os.makedirs(folder, exist_ok=True)
    with open(os.path.join(folder, f"{run}_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Grid_Size", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for kern, grid, ctr, val in rows:
            w.writerow({"Kernel_Name": kern, "Grid_Size": grid, "Counter_Name": ctr,
                        "Counter_Value": val})


def test_summarize_counters_scales_by_the_copy(tmp_path):
    """A 1 MiB copy reading FETCH 512 KiB and WRITE 1024 KiB gives scales 2 and 1; a kernel with
    FETCH 100 KiB and WRITE 50 KiB then moved 204800 + 51200 bytes. Kernels launched at two grid
    sizes stay apart."""
    for ctr, copy_kib, k_kib in (("FETCH_SIZE", 512, (100, 300)), ("WRITE_SIZE", 1024, (50, 70))):
        d = tmp_path / f"pmc_{ctr}"
        write_counters(d, "copy", [("void copy_kernel<1, true>()", 65536, ctr, copy_kib)])
        write_counters(d, "w.bwd_rows", [("bwd_rows_kernel", 256, ctr, k_kib[0]),
                                         ("bwd_rows_kernel", 256, ctr, k_kib[0]),
                                         ("bwd_rows_kernel", 512, ctr, k_kib[1])])
    r = run_bench("--summarize-counters", str(tmp_path), "--copy-probe-mib", "1")
    assert r.returncode == 0, r.stderr
    recs = [json.loads(x) for x in r.stdout.splitlines()]
    cal = [x["calibration"] for x in recs if "calibration" in x][0]
    assert cal["fetch_scale"] == 2.0 and cal["write_scale"] == 1.0
    t = {x["kernel"]: x for x in recs if "traffic_bytes" in x}
    a = t["bwd_rows_kernel [grid 256]"]
    assert (a["read_bytes"], a["write_bytes"], a["traffic_bytes"]) == (204800, 51200, 256000)
    b = t["bwd_rows_kernel [grid 512]"]
    assert b["traffic_bytes"] == 300 * 1024 * 2 + 70 * 1024
    means = [x for x in recs if x.get("counter") == "FETCH_SIZE" and x["run"] == "w.bwd_rows"]
    assert {m["dispatches"] for m in means} == {2, 1}


def test_traffic_line_is_gated_by_the_kernel_sources(tmp_path, monkeypatch):
    doc = tmp_path / "traffic.md"
    doc.write_text("traffic: kernel=bwd_rows_kernel workload=bf16_4096x4096 "
                   f"bytes_per_launch=123 sources={bench.kernel_source_hash()}\n")
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(doc))
    assert bench.read_traffic("bf16_4096x4096") == 123.0
    assert bench.read_traffic("fp16_8192x8192") is None  # recorded for the headline only
    doc.write_text("traffic: kernel=bwd_rows_kernel workload=bf16_4096x4096 "
                   "bytes_per_launch=123 sources=0000000000000000\n")
    assert bench.read_traffic("bf16_4096x4096") is None  # stale: the kernels changed since


def test_summary_median_and_mean():
    s = bench.summary([3e-6, 1e-6, 2e-6, 10e-6])
    assert s == {"mean_us": 4.0, "median_us": 2.5, "min_us": 1.0}
