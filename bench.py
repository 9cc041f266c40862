#!/usr/bin/env python3
"""Benchmark of transposable N:M mask search on one MI355X.

Default workload: 16:32 on an 8192 x 28672 bf16 matrix (235 M weights,
229,376 blocks of 32 x 32), tau = 40, 200 Dykstra iterations, 32 local-search
steps -- the configuration the headline metric is quoted on.  One "step" is
one tsenor_mask call: gather, Dykstra, rounding (greedy, local search, fill)
and the bit-packed mask write over the whole matrix, inputs resident in HBM.

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


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_baseline(w, W_np, seconds):
    """The oracle (fp64 Dykstra + rounding, OpenMP over blocks) on the first
    block-rows of the same matrix, sized to about `seconds` of host time."""
    import numpy as np

    import oracle
    from sparse_mask_search_amd import workloads as wl

    def run(block_rows):
        rows = block_rows * w.M
        Wf = wl.bf16_bits_to_f32(W_np[:rows]) if W_np.dtype == np.uint16 else W_np[:rows]
        Wf = np.ascontiguousarray(Wf)
        t0 = time.perf_counter()
        oracle.tsenor(Wf, w.N, w.M, w.tau, w.iters, w.ls_steps)
        return time.perf_counter() - t0, rows * w.cols

    oracle.build(force=False)
    t1, n1 = run(1)
    k = int(max(1, min(w.rows // w.M, round(seconds / max(t1, 1e-3)))))
    t, n = run(k) if k > 1 else (t1, n1)
    return {"value": n / t / 1e9, "unit": "Gweights/s", "cores": oracle.max_threads(),
            "kind": "oracle",
            "sample": f"first {k} block-row(s): {k * w.M} x {w.cols} = {n} weights, "
                      f"{k * (w.cols // w.M)} blocks, {t:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="16:32-8192x28672-bf16")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the method has no "
              "cross-GPU step and this build measures a single MI355X.", file=sys.stderr)
        sys.exit(2)

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
        sms.mask(W, w.N, w.M, w.tau, w.iters, w.ls_steps, out=out)

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in ev:
        a.record()
        step()
        b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = [a.elapsed_time(b) for a, b in ev]
    ms = float(np.mean(kern_ms))
    ms_wall = wall * 1e3 / args.steps
    log(f"[bench] kernel ms/step mean {ms:.3f} (min {min(kern_ms):.3f} max {max(kern_ms):.3f}); "
        f"wall {ms_wall:.3f}")

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
                   "ls_steps": w.ls_steps, "blocks": w.blocks, "recipe": w.recipe,
                   "seed": w.seed},
        "blocks_per_s": round(w.blocks / (ms_wall / 1e3), 1),
        "roofline": {"bound": "alu", "achieved": round(achieved, 3), "peak": PEAK_VALU_TOPS,
                     "unit": "Tops/s", "frac": round(achieved / PEAK_VALU_TOPS, 4),
                     "traffic": None,
                     "kernel": "mask_kernel (gather + Dykstra + rounding + pack, one launch)",
                     "kernel_ms": round(ms, 4),
                     "ops_per_launch": ops,
                     "hbm_algorithmic_bytes": hbm_bytes,
                     "hbm_achieved_gbs": round(hbm_bytes / (ms / 1e3) / 1e9, 1)},
    }
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline (oracle, ~{args.cpu_seconds:.0f} s)")
        rec["cpu_baseline"] = cpu_baseline(w, W_np, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
