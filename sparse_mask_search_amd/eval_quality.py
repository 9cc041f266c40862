"""Quality and cost of the method against the exact per-block optimum.

    python -m sparse_mask_search_amd.eval_quality [--workload NAME] [--polish K ...]

For a synthetic workload (see workloads.py) it times the method
(tsenor_mask_ex with at most K polish swaps per block), then certifies the
exact optimum of every block with tsenor_exact started from the method's mask,
and reports the relative gap (optimum - kept |W|) / optimum over all blocks,
plus the time of the exact solver from the method's mask and from a circulant
start.  One JSON line per measurement.  Everything runs on the GPU.
"""
import argparse
import json
import time

import numpy as np

from . import _lib as L
from . import workloads as wl


def _block_objective(torch, mask, A64, rows, cols, M):
    bits = torch.arange(32, device=mask.device, dtype=torch.int64)
    Z = ((mask.to(torch.int64).unsqueeze(-1) >> bits) & 1).reshape(rows, -1)[:, :cols]
    return (Z.double() * A64).reshape(rows // M, M, cols // M, M).sum((1, 3))


def _timed(torch, fn, reps=1):
    fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        out = fn()
    torch.cuda.synchronize()
    return out, (time.perf_counter() - t0) / reps


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--workload", default="16:32-8192x28672-bf16", choices=sorted(wl.WORKLOADS))
    ap.add_argument("--polish", type=int, action="append", default=None,
                    help="polish steps to evaluate (repeatable; default 0 and 8)")
    ap.add_argument("--max-cancel", type=int, default=100000)
    ap.add_argument("--no-circulant", action="store_true", help="skip the exact solve from scratch")
    args = ap.parse_args(argv)
    torch = L._torch()
    if not torch.cuda.is_available():
        raise SystemExit("eval_quality needs a GPU")
    w = wl.WORKLOADS[args.workload]
    Wn = wl.generate(args.workload)
    if Wn.dtype == np.uint16:
        W = torch.from_numpy(Wn.view(np.int16)).cuda().view(torch.bfloat16)
    else:
        W = torch.from_numpy(Wn).cuda()
    A64 = W.float().abs().double()
    exact_mask, t_exact = _timed(
        torch, lambda: L.exact(W, w.N, w.M, start=None, max_cancel=args.max_cancel,
                               return_objective=True)) if not args.no_circulant else (None, None)
    for K in (args.polish or [0, 8]):
        (m, _), t_m = _timed(torch, lambda: L.mask(W, w.N, w.M, w.tau, w.iters, w.ls_steps,
                                                   polish_steps=K), reps=3)
        (mx, opt), t_x = _timed(torch, lambda: L.exact(W, w.N, w.M, start=m,
                                                       max_cancel=args.max_cancel,
                                                       return_objective=True))
        got = _block_objective(torch, m, A64, w.rows, w.cols, w.M)
        ok = ~torch.isnan(opt)
        gap = ((opt - got) / torch.where(opt > 0, opt, torch.ones_like(opt)))[ok]
        rec = {"workload": args.workload, "polish_steps": K, "method_ms": round(t_m * 1e3, 3),
               "exact_from_method_ms": round(t_x * 1e3, 1),
               "blocks": int(opt.numel()), "uncertified_blocks": int((~ok).sum()),
               "gap_mean": float(gap.mean()), "gap_median": float(gap.median()),
               "gap_p99": float(torch.quantile(gap.float(), 0.99)), "gap_max": float(gap.max()),
               "blocks_optimal": float((gap <= 1e-12).double().mean())}
        if t_exact is not None:
            rec["exact_from_circulant_ms"] = round(t_exact * 1e3, 1)
        print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
