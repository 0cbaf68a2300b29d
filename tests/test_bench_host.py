"""Host logic of bench.py, on the CPU: the one-GPU refusal, the kernel-trace summary (which
dispatches are the timed ones), the counter summary (bytes scaled by the device copy's
counters, traffic per element, clock), the rule that counter traffic is reported only for
the kernel sources it was taken on, and the tolerance figure the oracle legs report. No GPU
and no rocprofv3 output needed: the CSV files are written here in rocprofv3's column
layout."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
import wkv_inputs  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def _write_trace(folder, kernels):
    """kernels: list of (name, [durations in ns]) launched in that order, interleaved."""
    os.makedirs(folder, exist_ok=True)
    cols = ["Kind", "Kernel_Name", "Start_Timestamp", "End_Timestamp"]
    t = 1_000_000
    with open(os.path.join(folder, "run_kernel_trace.csv"), "w", newline="") as f:
        wr = csv.DictWriter(f, cols)
        wr.writeheader()
        n = len(kernels[0][1])
        for i in range(n):
            for name, durs in kernels:
                wr.writerow({"Kind": "KERNEL_DISPATCH", "Kernel_Name": name,
                             "Start_Timestamp": t, "End_Timestamp": t + durs[i]})
                t += durs[i] + 1000


def test_trace_summary_takes_the_timed_dispatches(tmp_path):
    settle, warmup, steps = 3, 2, 4
    n = settle + warmup + steps + 5  # the other legs launch the same kernels afterwards
    fwd = [100_000] * (settle + warmup) + [200_000] * steps + [50_000] * 5
    bwd = [300_000] * (settle + warmup) + [400_000] * steps + [60_000] * 5
    red = [1_000] * (settle + warmup) + [6_000] * steps + [2_000] * 5
    _write_trace(str(tmp_path), [("void wkvdev::" + bench.KERNELS["forward"] + "(long)", fwd),
                                 ("void wkvdev::" + bench.KERNELS["backward"] + "(long)", bwd),
                                 ("wkvdev::" + bench.REDUCE_KERNEL + "(long)", red)])
    out = bench.summarize_trace(str(tmp_path), settle, warmup, steps)
    rows = [l for l in out.splitlines() if l.startswith("| `")]
    assert len(rows) == 3
    timed = [float(r.split("|")[5]) for r in rows]
    assert timed == [200.0, 400.0, 6.0]
    assert all(int(r.split("|")[2]) == n for r in rows)
    assert "timed means: 406.0 us" in out


def _write_counters(folder, counter, per_kernel):
    """per_kernel: {kernel name: [value per dispatch]}; one row per dispatch."""
    os.makedirs(folder, exist_ok=True)
    cols = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp",
            "End_Timestamp"]
    with open(os.path.join(folder, "run_counter_collection.csv"), "w", newline="") as f:
        wr = csv.DictWriter(f, cols)
        wr.writeheader()
        d = 0
        for name, vals in per_kernel.items():
            for val in vals:
                d += 1
                wr.writerow({"Dispatch_Id": d, "Kernel_Name": name, "Counter_Name": counter,
                             "Counter_Value": val, "Start_Timestamp": 0,
                             "End_Timestamp": 100_000})


def test_counter_summary_scales_by_the_copy(tmp_path):
    fwd_name = "void wkvdev::" + bench.COUNTER_KERNELS["forward"][0] + "(long)"
    copy_kib = bench.COPY_BYTES / 1024
    l3b = wkv_inputs.WORKLOADS["l3b"]
    n = l3b["B"] * l3b["T"] * l3b["C"]
    # FETCH_SIZE reads half the copy's bytes (so its scale is 2), WRITE_SIZE all of them
    fetch = {"__amd_rocclr_copyBuffer": [copy_kib / 2] * 3, fwd_name: [1000.0, 1000.0, 1200.0]}
    write = {"__amd_rocclr_copyBuffer": [copy_kib] * 3, fwd_name: [500.0, 500.0, 500.0]}
    busy = {fwd_name: [2.2e9 * 8 * 100e-6] * 3}  # 2.2 GHz over 100 us on 8 dies
    _write_counters(str(tmp_path / "f"), "FETCH_SIZE", fetch)
    _write_counters(str(tmp_path / "w"), "WRITE_SIZE", write)
    _write_counters(str(tmp_path / "g"), "GRBM_GUI_ACTIVE", busy)
    out = bench.summarize_counter_sets([str(tmp_path / "f"), str(tmp_path / "w"),
                                        str(tmp_path / "g")])
    assert out["scale"]["FETCH_SIZE"] == pytest.approx(2.0)
    assert out["scale"]["WRITE_SIZE"] == pytest.approx(1.0)
    rec = out["kernels"]["forward"]
    assert rec["FETCH_SIZE"] == 1000.0 and rec["WRITE_SIZE"] == 500.0  # medians
    assert rec["traffic_bytes"] == pytest.approx(1024 * (2 * 1000.0 + 500.0))
    assert rec["traffic_bytes_per_elem"] == pytest.approx(1024 * 2500.0 / n)
    assert rec["clock_ghz"] == pytest.approx(2.2)
    assert out["source_sha256"] == bench.source_hash()


def test_counter_traffic_only_for_the_sources_it_was_taken_on(tmp_path, monkeypatch):
    rec = {"source_sha256": bench.source_hash(),
           "kernels": {"backward": {"traffic_bytes": 123.0}}}
    path = tmp_path / "c.json"
    path.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "COUNTERS", str(path))
    assert bench.counter_traffic("backward") == 123.0
    assert bench.counter_traffic("forward") is None
    rec["source_sha256"] = "0" * 64
    path.write_text(json.dumps(rec))
    assert bench.counter_traffic("backward") is None
    monkeypatch.setattr(bench, "COUNTERS", str(tmp_path / "missing.json"))
    assert bench.counter_traffic("backward") is None


def test_committed_counter_summary_matches_the_sources():
    """The committed summary is the one bench.py reports traffic from: it must have been
    taken on the kernel sources as they are."""
    with open(bench.COUNTERS) as f:
        rec = json.load(f)
    assert rec["source_sha256"] == bench.source_hash()
    for op in ("forward", "backward"):
        assert rec["kernels"][op]["traffic_bytes"] > 0


def test_violation_is_the_operators_tolerance():
    """The bench line's parity figure: the largest |x - r| / (1e-4 max(|r|, 0.1))."""
    import numpy as np
    r = np.array([1.0, -2.0, 0.01, 0.0])
    assert bench._violation([r], [r]) == 0.0
    g = r + np.array([1e-4, 0.0, 0.0, 0.0])
    assert bench._violation([g], [r]) == pytest.approx(1.0)
    g = r + np.array([0.0, 0.0, 5e-6, 0.0])
    assert bench._violation([g, r], [r, r]) == pytest.approx(0.5)
    g = r.copy()
    g[3] = np.nan
    assert bench._violation([g], [r]) == float("inf")
    assert bench._violation([np.zeros(0)], [np.zeros(0)]) is None
