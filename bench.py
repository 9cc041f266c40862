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
# (profiles/mask_kernel_16x32_8192x28672_bf16.md), valid only for the kernel source
# they were taken on.
TRAFFIC = {
    "16:32-8192x28672-bf16": {
        "kernel_sha256": "44d5bcbae597b5fd18928972487b9c9fe71f544ac279254fc9a478d48fdf9ef1",
        "read_bytes": 907017.4375 * 1024 * 2.0, "write_bytes": 968147.953125 * 1024 * 1.0},
}


def measured_traffic(workload):
    """Counter-based HBM bytes per launch, or None once the kernel has changed."""
    import hashlib
    t = TRAFFIC.get(workload)
    if t is None:
        return None
    with open(KERNEL_SOURCE, "rb") as f:
        if hashlib.sha256(f.read()).hexdigest() != t["kernel_sha256"]:
            return None
    return int(t["read_bytes"] + t["write_bytes"])


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


def cpu_baseline_7b(seconds):
    """The oracle on the first block-rows of every projection of layer 0; the
    rate is extrapolated to the model's mix of 8:16 and 16:32 weights."""
    import numpy as np

    import oracle
    from sparse_mask_search_amd import workloads as wl

    oracle.build(force=False)
    mats = list(wl.model7b_layer(0))
    budget = seconds / len(mats)
    t_model, n_sample, t_sample = 0.0, 0, 0.0
    for nm, N, M, W in mats:
        def run(k):
            Wf = np.ascontiguousarray(wl.bf16_bits_to_f32(W[:k * M]))
            t0 = time.perf_counter()
            oracle.tsenor(Wf, N, M, wl.MODEL7B_TAU, wl.MODEL7B_ITERS, wl.MODEL7B_LS)
            return time.perf_counter() - t0, Wf.size
        t1, n1 = run(1)
        k = int(max(1, min(W.shape[0] // M, round(budget / max(t1, 1e-3)))))
        t, n = run(k) if k > 1 else (t1, n1)
        t_model += t / n * W.size * wl.MODEL7B_LAYERS
        n_sample += n
        t_sample += t
    weights = sum(W.size for _, _, _, W in mats) * wl.MODEL7B_LAYERS
    return {"value": weights / t_model / 1e9, "unit": "Gweights/s", "cores": oracle.max_threads(),
            "kind": "oracle",
            "sample": f"first block-rows of each layer-0 projection: {n_sample} weights in "
                      f"{t_sample:.1f} s, per-projection rates weighted by the model's weights"}


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

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
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
    log(f"[bench] ms/step mean {ms:.2f} (min {min(kern_ms):.2f} max {max(kern_ms):.2f}); wall {ms_wall:.2f}")
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
                     "traffic": None,
                     "kernel": "batched_kernel (one launch per N:M class)",
                     "kernel_ms": round(ms, 3), "ops_per_launch": ops},
    }
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline (oracle, ~{args.cpu_seconds:.0f} s)")
        rec["cpu_baseline"] = cpu_baseline_7b(args.cpu_seconds)
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="16:32-8192x28672-bf16")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
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
                   "ls_steps": w.ls_steps, "polish_steps": args.polish_steps,
                   "blocks": w.blocks, "recipe": w.recipe, "seed": w.seed},
        "blocks_per_s": round(w.blocks / (ms_wall / 1e3), 1),
        "roofline": {"bound": "alu", "achieved": round(achieved, 3), "peak": PEAK_VALU_TOPS,
                     "unit": "Tops/s", "frac": round(achieved / PEAK_VALU_TOPS, 4),
                     "traffic": measured_traffic(w.name) if args.polish_steps == 0 else None,
                     "kernel": "mask_kernel (gather + Dykstra + rounding + pack, one launch)"
                               + (" + refine_kernel" if args.polish_steps else ""),
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
