#!/usr/bin/env python3
"""Benchmark of transposable N:M mask search on one MI355X.

Default workload: 16:32 on an 8192 x 28672 bf16 matrix (235 M weights,
229,376 blocks of 32 x 32), tau = 40, 200 Dykstra iterations, 32 local-search
steps -- the configuration the headline metric is quoted on.  One "step" is
one tsenor_mask call: gather, Dykstra, rounding (greedy, local search, fill)
and the bit-packed mask write over the whole matrix, inputs resident in HBM.

`--workload 7b-model-batched` times instead one tsenor_mask_batched call over
the 224 projections of a 32-layer 7B-shaped model (8:16 on q/k/v/o 4096x4096,
16:32 on gate/up 4096x11008 and down 11008x4096; tau 30, 150 iterations,
16 steps; 6.48 G weights, 12.1 GiB of bf16 resident on the GPU).

Prints ONE JSON line on stdout; progress goes to stderr.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Gweights/s masked (16:32, 8192×28672) + % of VALU/exp roofline"
PEAK_HBM_GBS = 8000.0
# fp32 VALU lane-operations per second: 256 CUs x 4 SIMDs x 32 fp32 lanes per
# clock (a wave64 fp32 op retires in 2 clocks on one SIMD) x 2.4 GHz = 78.6 T
# (the vector-fp32 peak of 157.3 TFLOP/s counts an FMA as two).
PEAK_VALU_TOPS = 256 * 128 * 2.4e9 / 1e12
# per element and Dykstra cycle: P*V (mul), *U with clamp to [0,1] (the clip),
# row sum (add), column sum (fma)
OPS_PER_ELEM_ITER = 4
KERNEL_SOURCE = os.path.join(ROOT, "sparse_mask_search_amd", "csrc", "tsenor_kernels.hip")
# HBM bytes per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE runs of this benchmark
# (profiles/mask_kernel_*.md, profiles/batched_kernel_7b_model_bf16.md): KiB per
# dispatch scaled by what the same counters read for a 1 GiB device copy (x 2.0
# read, x 1.0 written), valid only for the kernel source they were taken on.  The
# 7B-shaped model's entry sums its two launches.
TRAFFIC_SHA = "17b7ab9157e5540d8343a4176867ce8f047cace810c0c9498b49fcf3ca872448"
TRAFFIC_KIB = {  # workload: (FETCH_SIZE, WRITE_SIZE) in KiB per launch
    "16:32-8192x28672-bf16": (471926.84375, 63500.328125),
    "16:32-8192x28672-bf16-tau200": (550135.21875, 66092.765625),
    "8:16-4096x11008-bf16": (68201.9375, 5832.796875),
    "4:8-4096x4096-f32": (61764.21875, 3074.8125),
    "2:4-1024x1024-f32": (2137.9375, 256.0),
    "7b-model-batched": (8640354.3125 + 3712244.875, 953938.015625 + 262822.265625),
}
FETCH_SCALE, WRITE_SCALE = 2.0, 1.0


def measured_traffic(workload):
    """Counter-based HBM bytes per launch, or None once the kernel has changed."""
    import hashlib
    t = TRAFFIC_KIB.get(workload)
    if t is None:
        return None
    with open(KERNEL_SOURCE, "rb") as f:
        if hashlib.sha256(f.read()).hexdigest() != TRAFFIC_SHA:
            return None
    return int(t[0] * 1024 * FETCH_SCALE + t[1] * 1024 * WRITE_SCALE)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def timed_steps(step, steps):
    """Run `steps` steps back to back between two HIP events on the launch
    stream (torch's current stream, the one the library launches on), with a
    device synchronisation on both sides.  Returns (ms per step by the
    events -- the launches' average duration including the gaps between
    them -- and ms per step by the host clock)."""
    import torch
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    a.record()
    for _ in range(steps):
        step()
    b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return a.elapsed_time(b) / steps, wall * 1e3 / steps


def warm_up(step, count, min_seconds=1.0, cap=5000):
    """Untimed warmup: `count` steps, or with count None as many steps as fill
    at least `min_seconds` of wall time (at least 3), so that the GPU clocks
    have settled before the timed region -- short launches run ~15% slower
    for the first few tens of milliseconds of a busy GPU.  Returns the number
    of steps run."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while (n < count) if count is not None else (
            n < 3 or (time.perf_counter() - t0 < min_seconds and n < cap)):
        step()
        n += 1
        if count is None and n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


def cpu_model():
    """The host CPU's model name (Linux /proc/cpuinfo), or the platform string."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or platform.machine()


def cpu_baseline(w, W_np, seconds):
    """The oracle (fp64 Dykstra + rounding, OpenMP over blocks) on the same
    matrix: in full when that is expected to take at most about 1.5 x
    `seconds` of host time, else on its first block-rows sized to `seconds`;
    a sample that runs in less than min(10 s, `seconds`) is repeated until it
    has.  Also a single-thread rate on the first block-row (repeated to 1 s)."""
    import numpy as np

    import oracle
    from sparse_mask_search_amd import workloads as wl

    def run(block_rows, nthreads=0):
        rows = block_rows * w.M
        Wf = wl.bf16_bits_to_f32(W_np[:rows]) if W_np.dtype == np.uint16 else W_np[:rows]
        Wf = np.ascontiguousarray(Wf)
        t0 = time.perf_counter()
        oracle.tsenor(Wf, w.N, w.M, w.tau, w.iters, w.ls_steps, nthreads=nthreads)
        return time.perf_counter() - t0, rows * w.cols

    def repeated(block_rows, nthreads, min_seconds, first=None):
        t, n, reps = (first[0], first[1], 1) if first else (0.0, 0, 0)
        while reps == 0 or t < min_seconds:
            dt, dn = run(block_rows, nthreads)
            t, n, reps = t + dt, n + dn, reps + 1
        return t, n, reps

    oracle.build(force=False)
    cores = oracle.max_threads()
    nbr = w.rows // w.M
    # Rate probe: the first block-row, then 4x as many until the probe runs at
    # least 0.25 s (a single short block-row is mostly per-call overhead, which
    # would make the whole matrix look dearer than it is).
    kp = 1
    tp, np_ = run(kp, cores)
    while tp < 0.25 and kp < nbr:
        kp = min(nbr, 4 * kp)
        tp, np_ = run(kp, cores)
    per_row = tp / kp
    full = per_row * nbr <= 1.5 * seconds
    k = nbr if full else int(max(1, min(nbr, round(seconds / max(per_row, 1e-3)))))
    t, n, reps = repeated(k, cores, min(10.0, seconds), first=(tp, np_) if k == kp else None)
    ts, ns, reps1 = repeated(1, 1, 1.0)
    oracle.dykstra(np.zeros((w.M, w.M), np.float32), 1, w.M, 0.0, 1, nthreads=cores)  # restore
    what = (f"the whole matrix: {w.rows} x {w.cols} = {n // reps} weights, {w.blocks} blocks"
            if full else
            f"first {k} of {nbr} block-rows: {k * w.M} x {w.cols} = {n // reps} weights, "
            f"{k * (w.cols // w.M)} blocks")
    if reps > 1:
        what += f", run {reps} times"
    return {"value": n / t / 1e9, "unit": "Gweights/s", "cores": cores,
            "kind": "oracle", "sample": f"{what}, {t:.1f} s",
            "cpu": cpu_model(), "nproc": os.cpu_count(),
            "single_thread": {"value": ns / ts / 1e9, "unit": "Gweights/s",
                              "sample": f"first block-row ({w.M} x {w.cols})"
                                        + (f" run {reps1} times" if reps1 > 1 else "")
                                        + f", {ts:.1f} s"}}


def memory_pass(W, M, steps=20):
    """Rate of the memory side alone (tsenor_bench_memory_pass: W read once
    by blocks, block max, one bit per weight written) against HBM peak."""
    import torch

    import sparse_mask_search_amd as sms
    out = torch.empty((W.shape[0], (W.shape[1] + 31) // 32), dtype=torch.int32, device=W.device)
    warm_up(lambda: sms.memory_pass(W, M, out=out), None, min_seconds=0.5)
    ms, _ = timed_steps(lambda: sms.memory_pass(W, M, out=out), steps)
    nbytes = W.numel() * W.element_size() + out.numel() * 4
    gbs = nbytes / (ms / 1e3) / 1e9
    return {"kernel": "memory_pass_kernel (tsenor_bench_memory_pass)", "kernel_ms": round(ms, 4),
            "bytes": nbytes, "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4)}


MODEL7B = "7b-model-batched"


def _gen_layer(layer):
    from sparse_mask_search_amd import workloads as wl
    return layer, [(nm, N, M, W) for nm, N, M, W in wl.model7b_layer(layer)]


def model7b_resident():
    """Every projection of the 7B-shaped model as bf16 CUDA tensors, generated
    on the host in parallel (one seeded generator per layer)."""
    import multiprocessing as mp

    import numpy as np
    import torch

    from sparse_mask_search_amd import workloads as wl
    mats = [None] * wl.MODEL7B_LAYERS
    workers = max(1, min(8, (os.cpu_count() or 1)))
    with mp.get_context("spawn").Pool(workers) as pool:
        for layer, items in pool.imap_unordered(_gen_layer, range(wl.MODEL7B_LAYERS)):
            mats[layer] = [(torch.from_numpy(W.view(np.int16)).cuda().view(torch.bfloat16), N, M, nm)
                           for nm, N, M, W in items]
            log(f"[bench] layer {layer} resident")
    return [m for layer in mats for m in layer]


def cpu_baseline_7b():
    """The oracle on every projection of layer 0 in full (202 M weights); the
    model's time is extrapolated as 32 x layer 0 (the layers differ only in
    their seeded values)."""
    import numpy as np

    import oracle
    from sparse_mask_search_amd import workloads as wl

    oracle.build(force=False)
    t_layer, n_layer = 0.0, 0
    for nm, N, M, W in wl.model7b_layer(0):
        Wf = np.ascontiguousarray(wl.bf16_bits_to_f32(W))
        t0 = time.perf_counter()
        oracle.tsenor(Wf, N, M, wl.MODEL7B_TAU, wl.MODEL7B_ITERS, wl.MODEL7B_LS)
        t_layer += time.perf_counter() - t0
        n_layer += Wf.size
    return {"value": n_layer / t_layer / 1e9, "unit": "Gweights/s",
            "cores": oracle.max_threads(), "kind": "oracle",
            "sample": f"layer 0 in full ({n_layer} weights, 7 projections) in {t_layer:.1f} s; "
                      f"model time extrapolated as 32 x layer 0 = {32 * t_layer:.0f} s",
            "extrapolated": True, "cpu": cpu_model(), "nproc": os.cpu_count()}


def main_7b(args):
    import numpy as np
    import torch

    import sparse_mask_search_amd as sms
    from sparse_mask_search_amd import workloads as wl

    t0 = time.perf_counter()
    mats = model7b_resident()
    log(f"[bench] 224 matrices resident in {time.perf_counter() - t0:.1f} s")
    outs = [torch.empty((W.shape[0], W.shape[1] // 32), dtype=torch.int32, device="cuda")
            for W, _, _, _ in mats]
    items = [(W, N, M, o) for (W, N, M, _), o in zip(mats, outs)]
    weights = sum(W.numel() for W, _, _, _ in mats)
    blocks = sum(W.numel() // (M * M) for W, _, M, _ in mats)
    elem_iters = weights * (wl.MODEL7B_ITERS - 1)

    def step():
        sms.mask_batched([(W, N, M) for W, N, M, _ in items], wl.MODEL7B_TAU, wl.MODEL7B_ITERS,
                         wl.MODEL7B_LS, outs=[o for _, _, _, o in items])

    args.warmup = warm_up(step, args.warmup)
    log(f"[bench] warmed up with {args.warmup} steps; timing {args.steps} steps")
    ms, ms_wall = timed_steps(step, args.steps)
    log(f"[bench] ms/step on the stream {ms:.2f}; wall {ms_wall:.2f}")
    ops = OPS_PER_ELEM_ITER * elem_iters
    achieved = ops / (ms / 1e3) / 1e12
    rec = {
        "metric": "Gweights/s masked (7B-shaped model, 224 projections, one batched call)",
        "value": round(weights / (ms_wall / 1e3) / 1e9, 4),
        "unit": "Gweights/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_wall, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": MODEL7B, "matrices": len(mats), "weights": weights,
                   "blocks": blocks, "input_dtype": "bf16", "tau": wl.MODEL7B_TAU,
                   "iters": wl.MODEL7B_ITERS, "ls_steps": wl.MODEL7B_LS,
                   "recipe": "per layer l: seed 1000+l; q,k,v,o,gate,up,down = 0.02*normal "
                             "+ 0.1% +-U(0.5,2) outliers, bf16"},
        "blocks_per_s": round(blocks / (ms_wall / 1e3), 1),
        "roofline": {"bound": "alu", "achieved": round(achieved, 3), "peak": PEAK_VALU_TOPS,
                     "unit": "Tops/s", "frac": round(achieved / PEAK_VALU_TOPS, 4),
                     "traffic": measured_traffic(MODEL7B),
                     "kernel": "batched_kernel (one launch per N:M class)",
                     "kernel_ms": round(ms, 3), "ops_per_launch": ops},
    }
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle on layer 0 in full)")
        rec["cpu_baseline"] = cpu_baseline_7b()
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warmup steps (default: as many as fill 1 s)")
    ap.add_argument("--workload", default="16:32-8192x28672-bf16")
    ap.add_argument("--cpu-seconds", type=float, default=30.0,
                    help="host-time budget of the oracle baseline (the whole matrix when it "
                         "is expected to take at most 1.5 x this)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--polish-steps", type=int, default=0,
                    help="add the optional 2-opt polish (at most this many swaps per block)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the method has no "
              "cross-GPU step, and the benchmark measures a single MI355X.", file=sys.stderr)
        sys.exit(2)

    if args.workload == MODEL7B:
        return main_7b(args)

    import numpy as np
    import torch

    import sparse_mask_search_amd as sms
    from sparse_mask_search_amd import workloads as wl

    w = wl.WORKLOADS[args.workload]
    log(f"[bench] generating {w.name} ({w.rows}x{w.cols} {w.dtype}) ...")
    t0 = time.perf_counter()
    W_np = wl.generate(w.name)
    log(f"[bench] generated in {time.perf_counter() - t0:.1f} s")
    if W_np.dtype == np.uint16:
        W = torch.from_numpy(W_np.view(np.int16)).cuda().view(torch.bfloat16)
    else:
        W = torch.from_numpy(W_np).cuda()
    out = torch.empty((w.rows, (w.cols + 31) // 32), dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()

    def step():
        sms.mask(W, w.N, w.M, w.tau, w.iters, w.ls_steps, out=out, polish_steps=args.polish_steps)

    args.warmup = warm_up(step, args.warmup)
    log(f"[bench] warmed up with {args.warmup} steps; timing {args.steps} steps")
    ms, ms_wall = timed_steps(step, args.steps)
    log(f"[bench] ms/step on the stream {ms:.4f}; wall {ms_wall:.4f}")

    gw = w.weights / (ms_wall / 1e3) / 1e9
    ops = OPS_PER_ELEM_ITER * w.weights * (w.iters - 1)
    achieved = ops / (ms / 1e3) / 1e12
    hbm_bytes = w.weights * (2 if w.dtype == "bf16" else 4) + w.rows * ((w.cols + 31) // 32) * 4
    rec = {
        "metric": METRIC,
        "value": round(gw, 4),
        "unit": "Gweights/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_wall, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "N": w.N, "M": w.M, "rows": w.rows, "cols": w.cols,
                   "input_dtype": w.dtype, "tau": w.tau, "iters": w.iters,
                   "ls_steps": w.ls_steps, "polish_steps": args.polish_steps,
                   "blocks": w.blocks, "recipe": w.recipe, "seed": w.seed},
        "blocks_per_s": round(w.blocks / (ms_wall / 1e3), 1),
        "roofline": {"bound": "alu", "achieved": round(achieved, 3), "peak": PEAK_VALU_TOPS,
                     "unit": "Tops/s", "frac": round(achieved / PEAK_VALU_TOPS, 4),
                     "traffic": measured_traffic(w.name) if args.polish_steps == 0 else None,
                     "kernel": "mask_kernel (gather + Dykstra + rounding + pack, one launch)"
                               if args.polish_steps == 0 else
                               "mask_kernel with the optional stages (gather + Dykstra + rounding"
                               " + 2-opt polish + pack, one launch)",
                     "kernel_ms": round(ms, 4),
                     "ops_per_launch": ops,
                     "hbm_algorithmic_bytes": hbm_bytes,
                     "hbm_achieved_gbs": round(hbm_bytes / (ms / 1e3) / 1e9, 1)},
    }
    if w.M in (16, 32):
        log("[bench] memory side alone")
        rec["memory_pass"] = memory_pass(W, w.M)
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline (oracle, budget ~{args.cpu_seconds:.0f} s)")
        rec["cpu_baseline"] = cpu_baseline(w, W_np, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
