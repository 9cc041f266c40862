"""tsenor_mask_noalloc (the entry point that allocates nothing) against
tsenor_mask, called through the C ABI on the same seeded inputs.

Both entry points run the same kernels, so the masks must be bit-identical and
S identical (the fractional-S bar is 1e-4; equality is asserted).  The calls
run back to back on one stream: a large 16:32 call, a smaller 16:32 call and a
smaller 4:8 fp32 call, each right after a larger one.  Every result is also
checked for feasibility and against the oracle's rounding of its own S.
"""
import ctypes

import numpy as np
import pytest

import oracle
import sparse_mask_search_amd as sms
from sparse_mask_search_amd import workloads as wl
from gpu_util import as_f32, assert_feasible, to_device, words

pytestmark = pytest.mark.gpu

CASES = [  # M, N, block columns, block rows, bf16, tau, iters, ls
    (32, 16, 43, 3, True, 40.0, 60, 32),
    (32, 16, 11, 1, True, 40.0, 60, 32),
    (8, 4, 9, 2, False, 20.0, 50, 8),
]


def _inputs(k, M, nbc, nbr, bf16):
    W = np.concatenate([wl.random_blocks(500 + 10 * k + r, nbc, M, "outlier") for r in range(nbr)])
    W = W.astype(np.float32)
    return wl.f32_to_bf16_bits(W) if bf16 else W


def _call(fn, Wt, N, M, tau, iters, ls, mask, frac):
    rows, cols = Wt.shape
    dt = sms.BF16 if Wt.dtype.is_floating_point and Wt.element_size() == 2 else sms.F32
    return fn(ctypes.c_void_p(Wt.data_ptr()), dt, rows, cols, Wt.stride(0), N, M, tau, iters, ls,
              ctypes.c_void_p(mask.data_ptr()),
              ctypes.c_void_p(frac.data_ptr() if frac is not None else 0), None)


def test_noalloc_equals_mask_calls_in_a_row():
    import torch
    l = sms.lib()
    for k, (M, N, nbc, nbr, bf16, tau, iters, ls) in enumerate(CASES):
        print(f"[case] noalloc call {k}: {N}:{M} {nbr * M}x{nbc * M} bf16={bf16}", flush=True)
        W_np = _inputs(k, M, nbc, nbr, bf16)
        Wt = to_device(W_np)
        rows, cols = Wt.shape
        wpr = (cols + 31) // 32
        m_na = torch.full((rows, wpr), -1, dtype=torch.int32, device="cuda")
        f_na = torch.full((rows, cols), -1.0, dtype=torch.float32, device="cuda")
        m_ref = torch.zeros((rows, wpr), dtype=torch.int32, device="cuda")
        f_ref = torch.zeros((rows, cols), dtype=torch.float32, device="cuda")
        assert _call(l.tsenor_mask_noalloc, Wt, N, M, tau, iters, ls, m_na, f_na) == 0
        torch.cuda.synchronize()
        assert _call(l.tsenor_mask, Wt, N, M, tau, iters, ls, m_ref, f_ref) == 0
        torch.cuda.synchronize()
        assert torch.equal(m_na, m_ref), k
        assert torch.equal(f_na, f_ref), k
        Wf = as_f32(W_np)
        S = f_na.cpu().numpy()
        assert_feasible(words(m_na), rows, cols, N, M)
        ref, _ = oracle.round_matrix(S, Wf, N, M, ls)
        assert np.array_equal(words(m_na), ref), k
        S64, _ = oracle.dykstra(Wf, N, M, tau, iters)
        assert float(np.abs(S - S64).max()) < 1e-4, k
        # without frac_out: the same mask
        m2 = torch.zeros_like(m_na)
        assert _call(l.tsenor_mask_noalloc, Wt, N, M, tau, iters, ls, m2, None) == 0
        torch.cuda.synchronize()
        assert torch.equal(m2, m_ref), k


def test_noalloc_rejects_bad_arguments_before_any_launch():
    """Argument errors come back as status codes, exactly as tsenor_mask's."""
    import torch
    l = sms.lib()
    Wt = to_device(np.ones((32, 64), np.float32))
    m = torch.zeros((32, 2), dtype=torch.int32, device="cuda")
    good = dict(N=2, M=4, tau=20.0, iters=5, ls=2)
    for bad, want in [(dict(M=6), 3), (dict(N=0), 3), (dict(tau=-1.0), 4), (dict(iters=0), 4),
                      (dict(ls=-1), 4)]:
        a = dict(good, **bad)
        assert _call(l.tsenor_mask_noalloc, Wt, a["N"], a["M"], a["tau"], a["iters"], a["ls"],
                     m, None) == want, bad
    assert l.tsenor_mask_noalloc(None, 0, 32, 64, 64, 2, 4, 20.0, 5, 2,
                                 ctypes.c_void_p(m.data_ptr()), None, None) == 1
