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


PROFILE_OF = {
    "16:32-8192x28672-bf16": "mask_kernel_16x32_8192x28672_bf16.md",
    "16:32-8192x28672-bf16-tau200": "mask_kernel_16x32_8192x28672_bf16_tau200.md",
    "8:16-4096x11008-bf16": "mask_kernel_8x16_4096x11008_bf16.md",
    "4:8-4096x4096-f32": "mask_kernel_4x8_4096x4096_f32.md",
    "2:4-1024x1024-f32": "mask_kernel_2x4_1024x1024_f32.md",
    "7b-model-batched": "batched_kernel_7b_model_bf16.md",
}


def _profile_counters(fname):
    """(kernel source sha256, [(FETCH_SIZE, WRITE_SIZE) KiB per mask/batched kernel row])
    from a committed rocprofv3 summary."""
    text = open(os.path.join(ROOT, "profiles", fname)).read()
    sha = text.split("sha256 `", 1)[1].split("`", 1)[0]
    rows = []
    section = text.split("## HBM traffic", 1)[1].split("\n## ", 1)[0]
    for line in section.splitlines():
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) == 8 and cells[0].startswith(("mask_kernel", "batched_kernel")):
            rows.append((float(cells[1].replace(",", "")), float(cells[2].replace(",", ""))))
    return sha, rows


def test_traffic_table_matches_the_committed_profiles():
    """The counter bytes bench.py reports are the ones the profiles hold, taken
    on the kernel source the table is keyed to."""
    assert set(PROFILE_OF) == set(bench.TRAFFIC_KIB)
    for name, fname in PROFILE_OF.items():
        sha, rows = _profile_counters(fname)
        assert sha == bench.TRAFFIC_SHA, fname
        assert rows, fname
        fetch = sum(r[0] for r in rows)
        write = sum(r[1] for r in rows)
        want_f, want_w = bench.TRAFFIC_KIB[name]
        # the profiles print one decimal place
        assert abs(fetch - want_f) <= 0.05 * len(rows) + 1e-6, (name, fetch, want_f)
        assert abs(write - want_w) <= 0.05 * len(rows) + 1e-6, (name, write, want_w)
