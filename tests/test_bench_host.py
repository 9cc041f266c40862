"""bench.py's host-side logic, on the CPU: the one-GPU guard, the counter
traffic lookup and the oracle baseline record (no GPU call is made)."""
import dataclasses
import hashlib
import os
import subprocess
import sys


import bench
from sparse_mask_search_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_follows_the_kernel_source(monkeypatch):
    with open(bench.KERNEL_SOURCE, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()
    monkeypatch.setattr(bench, "TRAFFIC_SHA", sha)
    fetch, write = bench.TRAFFIC_KIB["16:32-8192x28672-bf16"]
    assert bench.measured_traffic("16:32-8192x28672-bf16") == int(
        fetch * 1024 * bench.FETCH_SCALE + write * 1024 * bench.WRITE_SCALE)
    assert bench.measured_traffic("no-such-workload") is None
    monkeypatch.setattr(bench, "TRAFFIC_SHA", "0" * 64)  # counters of another kernel
    assert bench.measured_traffic("16:32-8192x28672-bf16") is None


def test_every_traffic_entry_names_a_workload():
    for name in bench.TRAFFIC_KIB:
        assert name in wl.WORKLOADS or name == bench.MODEL7B


def test_cpu_baseline_record():
    w = wl.WORKLOADS["2:4-1024x1024-f32"]
    W = wl.generate(w.name)
    rec = bench.cpu_baseline(w, W, 2.0)
    assert rec["kind"] == "oracle" and rec["unit"] == "Gweights/s"
    assert rec["value"] > 0 and rec["cores"] >= 1
    assert rec["nproc"] == os.cpu_count() and rec["cpu"]
    assert rec["sample"].startswith("the whole matrix")  # 1 M weights fit any budget
    assert rec["single_thread"]["value"] > 0
    assert "first block-row" in rec["single_thread"]["sample"]


def test_cpu_baseline_samples_block_rows_beyond_the_budget():
    w = wl.WORKLOADS["8:16-4096x11008-bf16"]
    W = wl.generate(w.name, rows=64 * w.M)
    # pretend the matrix has 256 block-rows: the whole of it would exceed the budget
    big = dataclasses.replace(w, rows=256 * w.M)
    rec = bench.cpu_baseline(big, W, 0.05)
    assert rec["sample"].startswith("first "), rec["sample"]
