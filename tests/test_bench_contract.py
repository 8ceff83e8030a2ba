"""Host-side checks of the benchmark's bookkeeping (no GPU): the one-GPU guard, the counter
scaling that turns two rocprofv3 counter runs into HBM bytes per launch, the staleness rule of
that figure, and the algorithmic byte counts of the 1M decode."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
import workloads  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def _counter_csv(path, counter, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for name, value in rows:
            wr.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_counter_runs_scale_by_the_calibration_copy(tmp_path, monkeypatch):
    """FETCH_SIZE reads half the true bytes of a 256 MiB copy and WRITE_SIZE all of them: the
    scan's counts are scaled by the same factors (small copies of torch's own are ignored)."""
    kib = bench.COPY_BYTES / 1024
    scan = "void csa2::k_idx_scan<false, 0>(...)"
    copy = "__amd_rocclr_copyBuffer"
    _counter_csv(tmp_path / "fetch", "FETCH_SIZE",
                 [(scan, 66000.0), (scan, 66010.0), (copy, kib / 2), (copy, kib / 2), (copy, 4.0)])
    _counter_csv(tmp_path / "write", "WRITE_SIZE", [(scan, 4768.0), (copy, kib), (copy, kib)])
    out = tmp_path / "pmc.json"
    monkeypatch.setattr(bench, "PMC_FILE", str(out))
    assert bench.summarize_pmc(str(tmp_path / "fetch"), str(tmp_path / "write")) == 0
    d = json.loads(out.read_text())
    assert d["fetch_scale"] == 2.0 and d["write_scale"] == 1.0
    assert d["hbm_bytes_per_launch"] == int((66005.0 * 2 + 4768.0) * 1024)
    assert d["source_sha1"] == bench.scan_source_hash()
    assert d["dispatches"] == {"scan_fetch": 2, "copy_fetch": 2, "scan_write": 1, "copy_write": 2}
    # the figure is reported only while the scan's sources hash to the profiled ones
    assert bench.traffic_from_profile() == d["hbm_bytes_per_launch"]
    d["source_sha1"] = "0" * 40
    out.write_text(json.dumps(d))
    assert bench.traffic_from_profile() is None


def test_decode_1m_algorithmic_bytes():
    """The scan reads every key row (2^20 x 128 B) plus the query and its weights; the step adds
    the pool, the Top-K outputs, 4 Reindex layers and 20 attention layers."""
    w = workloads.WORKLOADS["decode_1m"]
    assert bench.scan_algorithmic_bytes(w) == (1 << 20) * 128 + 32 * 128 * 2 + 32 * 4
    assert bench.step_algorithmic_bytes(w) == 147942016


def test_kernel_trace_summary_and_its_staleness(tmp_path, monkeypatch):
    """A rocprofv3 --stats table becomes per-kernel averages (template variants merged by call
    count); the scan's duration is reported only while its sources hash to the profiled ones."""
    d = tmp_path / "trace" / "host"
    d.mkdir(parents=True)
    with open(d / "123_kernel_stats.csv", "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage"])
        wr.writeheader()
        wr.writerow({"Name": "void csa2::k_idx_scan<false, 0>(unsigned char const*, ...)", "Calls": 30,
                     "TotalDurationNs": 30 * 25000, "AverageNs": 25000.0, "Percentage": 40})
        wr.writerow({"Name": "csa2::k_pool(unsigned long const*, ...)", "Calls": 30, "TotalDurationNs": 300000,
                     "AverageNs": 10000.0, "Percentage": 20})
        wr.writerow({"Name": "void csa2::k_ri_score<false>(...)", "Calls": 10, "TotalDurationNs": 40000,
                     "AverageNs": 4000.0, "Percentage": 5})
        wr.writerow({"Name": "void csa2::k_ri_score<true>(...)", "Calls": 30, "TotalDurationNs": 240000,
                     "AverageNs": 8000.0, "Percentage": 5})
        wr.writerow({"Name": "__amd_rocclr_copyBuffer", "Calls": 3, "TotalDurationNs": 3, "AverageNs": 1.0,
                     "Percentage": 0})
    out = tmp_path / "kernels.json"
    monkeypatch.setattr(bench, "KERNEL_FILE", str(out))
    assert bench.summarize_trace(str(tmp_path / "trace"), "decode_1m", 30) == 0
    k = json.loads(out.read_text())["kernels"]
    assert k["k_idx_scan"] == {"calls": 30, "avg_us": 25.0}
    assert k["k_ri_score"] == {"calls": 40, "avg_us": 7.0}
    assert "copy" not in json.dumps(k)
    assert bench.kernel_duration_from_profile("k_idx_scan", "decode_1m") == 25.0
    assert bench.kernel_duration_from_profile("k_idx_scan", "decode_b8_128k") is None
    d2 = json.loads(out.read_text())
    d2["source_sha1"] = "0" * 40
    out.write_text(json.dumps(d2))
    assert bench.kernel_duration_from_profile("k_idx_scan", "decode_1m") is None
