"""Timing of the 2:4 consumer of transposable masks against the dense bf16
product (torch.matmul), forward Y = X W^T and data gradient dX = dY W.

    python -m sparse_mask_search_amd.bench_spmm24 [--shape N,OUT,IN ...] [--reps R]

W [OUT, IN] bf16 (0.02 * normal, seeded) gets a 2:4 transposable mask from the
library's own search; both W and W^T are compressed under that one mask.  One
JSON line per shape and direction, with times in ms and dense-equivalent
TFLOP/s (2 N OUT IN flops; the sparse product performs half of them).
"""
import argparse
import json

from . import _lib as L


def _time(torch, fn, reps):
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--shape", action="append", default=None,
                    help="N,OUT,IN (repeatable); default: 4096,4096,4096 and 8192,8192,28672")
    ap.add_argument("--reps", type=int, default=20)
    ap.add_argument("--no-dense", action="store_true")
    args = ap.parse_args(argv)
    torch = L._torch()
    if not torch.cuda.is_available():
        raise SystemExit("bench_spmm24 needs a GPU")
    shapes = [tuple(int(x) for x in s.split(",")) for s in (args.shape or
              ["4096,4096,4096", "8192,8192,28672"])]
    gen = torch.Generator(device="cuda").manual_seed(0)
    for (n, out_f, in_f) in shapes:
        W = (0.02 * torch.randn(out_f, in_f, device="cuda", generator=gen)).to(torch.bfloat16)
        mask, _ = L.mask(W, 2, 4, 20.0, 50, 4)
        for direction, tr in (("forward", False), ("data_gradient", True)):
            vals, meta, bad = L.compress24(W, mask, transpose=tr)
            m_, k_ = (in_f, out_f) if tr else (out_f, in_f)
            X = torch.randn(n, k_, device="cuda", generator=gen).to(torch.bfloat16)
            Y = torch.empty(n, m_, device="cuda")
            ts = _time(torch, lambda: L.spmm24(X, vals, meta, out=Y), args.reps)
            rec = {"shape": [n, out_f, in_f], "direction": direction, "sparse_ms": round(ts, 4),
                   "sparse_tflops_dense_equiv": round(2.0 * n * m_ * k_ / ts / 1e9, 1),
                   "overfull_groups": int(bad.item())}
            if not args.no_dense:
                Wd = W if tr else W.t().contiguous()
                td = _time(torch, lambda: torch.matmul(X, Wd), args.reps)
                rec["dense_ms"] = round(td, 4)
                rec["dense_tflops"] = round(2.0 * n * m_ * k_ / td / 1e9, 1)
            print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
