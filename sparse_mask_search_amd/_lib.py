"""ctypes binding of libtsenor.so: the same entry points as include/tsenor.h."""
from __future__ import annotations

import ctypes
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(HERE, "libtsenor.so")

F32, BF16 = 0, 1
_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I = ctypes.c_int
_F = ctypes.c_float


class TsenorError(RuntimeError):
    def __init__(self, status: int, where: str):
        l = lib()
        msg = l.tsenor_status_str(status).decode()
        if status == 6:
            msg += ": " + l.tsenor_last_error().decode()
        super().__init__(f"{where}: {msg} (status {status})")
        self.status = status


class _Matrix(ctypes.Structure):
    _fields_ = [("W", _P), ("dtype", _I), ("rows", _I64), ("cols", _I64), ("ld", _I64),
                ("N", _I), ("M", _I), ("mask_out", _P), ("frac_out", _P)]


def library_path() -> str:
    return _LIB_PATH


def lib():
    """Load libtsenor.so (raises if it has not been built: there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"{_LIB_PATH} is missing; build it with `python -m sparse_mask_search_amd.build`")
        l = ctypes.CDLL(_LIB_PATH)
        l.tsenor_mask.argtypes = [_P, _I, _I64, _I64, _I64, _I, _I, _F, _I, _I, _P, _P, _P]
        l.tsenor_mask.restype = _I
        l.tsenor_mask_ex.argtypes = [_P, _I, _I64, _I64, _I64, _I, _I, _F, _I, _I, _I, _P, _P, _P,
                                     _P]
        l.tsenor_mask_ex.restype = _I
        l.tsenor_mask_noalloc.argtypes = [_P, _I, _I64, _I64, _I64, _I, _I, _F, _I, _I, _P, _P, _P]
        l.tsenor_mask_noalloc.restype = _I
        l.tsenor_exact.argtypes = [_P, _I, _I64, _I64, _I64, _I, _I, _P, _I, _P, _P, _P]
        l.tsenor_exact.restype = _I
        l.tsenor_compress24.argtypes = [_P, _I64, _I64, _I64, _P, _I, _P, _P, _P, _P]
        l.tsenor_compress24.restype = _I
        l.tsenor_spmm24.argtypes = [_P, _I64, _I64, _P, _P, _I64, _I64, _P, _I64, _P]
        l.tsenor_spmm24.restype = _I
        l.tsenor_round.argtypes = [_P, _I64, _P, _I, _I64, _I64, _I64, _I, _I, _I, _P, _P]
        l.tsenor_round.restype = _I
        l.tsenor_mask_batched.argtypes = [ctypes.POINTER(_Matrix), _I, _F, _I, _I, _P]
        l.tsenor_mask_batched.restype = _I
        l.tsenor_mask_batched_ex.argtypes = [ctypes.POINTER(_Matrix), _I, _F, _I, _I, _I,
                                             ctypes.POINTER(_P), _P]
        l.tsenor_mask_batched_ex.restype = _I
        l.tsenor_bench_memory_pass.argtypes = [_P, _I, _I64, _I64, _I64, _I, _P, _P]
        l.tsenor_bench_memory_pass.restype = _I
        l.tsenor_status_str.argtypes = [_I]
        l.tsenor_status_str.restype = ctypes.c_char_p
        l.tsenor_last_error.argtypes = []
        l.tsenor_last_error.restype = ctypes.c_char_p
        l.tsenor_version.restype = _I
        _lib = l
    return _lib


def version() -> int:
    return int(lib().tsenor_version())


def _torch():
    import torch
    return torch


def _weights(W):
    torch = _torch()
    if not isinstance(W, torch.Tensor) or not W.is_cuda:
        raise TypeError("W must be a CUDA (HIP) torch tensor")
    if W.dim() != 2 or W.stride(1) != 1:
        raise ValueError("W must be 2-D with unit column stride")
    if W.dtype == torch.float32:
        return F32
    if W.dtype == torch.bfloat16:
        return BF16
    raise TypeError("W must be float32 or bfloat16")


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _mask_buffer(W, out=None):
    """A fresh mask buffer for W, or `out` after checking that the kernels may
    write [rows][ceil(cols/32)] contiguous words into it."""
    torch = _torch()
    rows, cols = W.shape
    shape = (rows, (cols + 31) // 32)
    if out is None:
        return torch.empty(shape, dtype=torch.int32, device=W.device)
    if (out.dtype != torch.int32 or out.device != W.device or tuple(out.shape) != shape
            or not out.is_contiguous()):
        raise ValueError(f"mask buffer must be a contiguous int32 tensor of shape {shape} "
                         f"on {W.device}")
    return out


def mask(W, N: int, M: int, tau: float, iters: int, ls_steps: int, return_frac: bool = False,
         out=None, frac_out=None, stream=None, polish_steps: int = 0, prev_mask=None):
    """Transposable N:M mask of W (fp32 or bf16 CUDA tensor).

    Returns (mask, frac): mask is int32 [rows, ceil(cols/32)] holding the
    uint32 bit words (bit c%32 of word c/32 = column c); frac is the fp32
    fractional solution S [rows, cols] if requested, else None.
    polish_steps > 0 adds up to that many 2-opt swaps per block; prev_mask (a
    mask tensor like the output, may be `out` itself) makes every block keep
    it where it is feasible and keeps more |W| (tsenor_mask_ex)."""
    torch = _torch()
    dt = _weights(W)
    rows, cols = W.shape
    out = _mask_buffer(W, out)
    if frac_out is None and return_frac:
        frac_out = torch.empty((rows, cols), dtype=torch.float32, device=W.device)
    elif frac_out is not None and (frac_out.dtype != torch.float32 or frac_out.device != W.device
                                   or tuple(frac_out.shape) != (rows, cols)
                                   or not frac_out.is_contiguous()):
        raise ValueError(f"frac_out must be a contiguous float32 tensor of shape {(rows, cols)} "
                         f"on {W.device}")
    fp = ctypes.c_void_p(frac_out.data_ptr() if frac_out is not None else 0)
    if polish_steps == 0 and prev_mask is None:
        st = lib().tsenor_mask(ctypes.c_void_p(W.data_ptr()), dt, rows, cols, W.stride(0), N, M,
                               float(tau), int(iters), int(ls_steps),
                               ctypes.c_void_p(out.data_ptr()), fp, _stream(stream))
        if st != 0:
            raise TsenorError(st, "tsenor_mask")
        return out, frac_out
    if prev_mask is not None:
        prev_mask = _mask_buffer(W, prev_mask)  # same checks as an output buffer
    st = lib().tsenor_mask_ex(ctypes.c_void_p(W.data_ptr()), dt, rows, cols, W.stride(0), N, M,
                              float(tau), int(iters), int(ls_steps), int(polish_steps),
                              ctypes.c_void_p(prev_mask.data_ptr() if prev_mask is not None else 0),
                              ctypes.c_void_p(out.data_ptr()), fp, _stream(stream))
    if st != 0:
        raise TsenorError(st, "tsenor_mask_ex")
    return out, frac_out


def mask_noalloc(W, N: int, M: int, tau: float, iters: int, ls_steps: int, out, frac_out=None,
                 stream=None):
    """tsenor_mask_noalloc: the mask of W into the caller's `out` (and S into
    `frac_out` when given), with the library allocating nothing and recording
    no event (the path needs no workspace)."""
    dt = _weights(W)
    rows, cols = W.shape
    if out is None:
        raise ValueError("mask_noalloc needs a caller-supplied mask buffer")
    out = _mask_buffer(W, out)
    if frac_out is not None:
        torch = _torch()
        if (frac_out.dtype != torch.float32 or frac_out.device != W.device
                or tuple(frac_out.shape) != (rows, cols) or not frac_out.is_contiguous()):
            raise ValueError(f"frac_out must be a contiguous float32 tensor of shape "
                             f"{(rows, cols)} on {W.device}")
    st = lib().tsenor_mask_noalloc(ctypes.c_void_p(W.data_ptr()), dt, rows, cols, W.stride(0), N,
                                   M, float(tau), int(iters), int(ls_steps),
                                   ctypes.c_void_p(out.data_ptr()),
                                   ctypes.c_void_p(frac_out.data_ptr() if frac_out is not None else 0),
                                   _stream(stream))
    if st != 0:
        raise TsenorError(st, "tsenor_mask_noalloc")
    return out, frac_out


def exact(W, N: int, M: int, start=None, max_cancel: int = 4096, out=None,
          return_objective: bool = False, stream=None):
    """Exact optimum mask of every block (tsenor_exact).  start: a feasible
    mask tensor to start from (e.g. the output of mask()), or None.  Returns
    (mask, objective) with objective an fp64 [rows/M, cols/M] tensor of
    per-block optima (NaN where not certified) if requested, else None."""
    torch = _torch()
    dt = _weights(W)
    rows, cols = W.shape
    out = _mask_buffer(W, out)
    if start is not None:
        start = _mask_buffer(W, start)
    objv = (torch.empty((rows // M, cols // M), dtype=torch.float64, device=W.device)
            if return_objective else None)
    st = lib().tsenor_exact(ctypes.c_void_p(W.data_ptr()), dt, rows, cols, W.stride(0), N, M,
                            ctypes.c_void_p(start.data_ptr() if start is not None else 0),
                            int(max_cancel), ctypes.c_void_p(out.data_ptr()),
                            ctypes.c_void_p(objv.data_ptr() if objv is not None else 0),
                            _stream(stream))
    if st != 0:
        raise TsenorError(st, "tsenor_exact")
    return out, objv


def compress24(W, mask_words, transpose: bool = False, stream=None):
    """2:4 compressed operand A = W (or W^T) under a 2:4 mask (tsenor_compress24).
    W: bf16 CUDA tensor [rows, cols]; mask_words: the int32 mask of mask().
    Returns (values bf16 [arows, k/2], meta int32 [arows, k/32], bad) with bad
    a CUDA int32 tensor holding the number of groups with more than two kept
    entries."""
    torch = _torch()
    if W.dtype != torch.bfloat16 or not W.is_cuda or W.dim() != 2 or W.stride(1) != 1:
        raise TypeError("W must be a 2-D bfloat16 CUDA tensor with unit column stride")
    rows, cols = W.shape
    _mask_buffer(W, mask_words)
    arows, k = (cols, rows) if transpose else (rows, cols)
    vals = torch.empty((arows, k // 2), dtype=torch.bfloat16, device=W.device)
    meta = torch.empty((arows, max(1, k // 32)), dtype=torch.int32, device=W.device)
    bad = torch.zeros(1, dtype=torch.int32, device=W.device)
    st = lib().tsenor_compress24(ctypes.c_void_p(W.data_ptr()), rows, cols, W.stride(0),
                                 ctypes.c_void_p(mask_words.data_ptr()), int(bool(transpose)),
                                 ctypes.c_void_p(vals.data_ptr()), ctypes.c_void_p(meta.data_ptr()),
                                 ctypes.c_void_p(bad.data_ptr()), _stream(stream))
    if st != 0:
        raise TsenorError(st, "tsenor_compress24")
    return vals, meta, bad


def spmm24(X, values, meta, out=None, stream=None):
    """Y = X A^T on the sparse matrix cores (tsenor_spmm24).  X: bf16 CUDA
    tensor [n, k]; values/meta from compress24 (A is [m, k]).  Returns fp32
    [n, m]."""
    torch = _torch()
    if X.dtype != torch.bfloat16 or not X.is_cuda or X.dim() != 2 or X.stride(1) != 1:
        raise TypeError("X must be a 2-D bfloat16 CUDA tensor with unit column stride")
    n, k = X.shape
    m = values.shape[0]
    if values.shape[1] * 2 != k or meta.shape != (m, k // 32) or not values.is_contiguous() \
            or not meta.is_contiguous():
        raise ValueError("compressed operand does not match X")
    if out is None:
        out = torch.empty((n, m), dtype=torch.float32, device=X.device)
    elif out.dtype != torch.float32 or tuple(out.shape) != (n, m) or out.stride(1) != 1:
        raise ValueError(f"out must be a float32 tensor of shape {(n, m)} with unit column stride")
    st = lib().tsenor_spmm24(ctypes.c_void_p(X.data_ptr()), n, X.stride(0),
                             ctypes.c_void_p(values.data_ptr()), ctypes.c_void_p(meta.data_ptr()),
                             m, k, ctypes.c_void_p(out.data_ptr()), out.stride(0), _stream(stream))
    if st != 0:
        raise TsenorError(st, "tsenor_spmm24")
    return out


def round_mask(S, W, N: int, M: int, ls_steps: int, out=None, stream=None):
    """Rounding only (greedy, local search, fill) of a fractional S [rows, cols]."""
    torch = _torch()
    dt = _weights(W)
    if S.dtype != torch.float32 or not S.is_cuda or S.dim() != 2 or S.stride(1) != 1:
        raise TypeError("S must be a 2-D float32 CUDA tensor with unit column stride")
    if tuple(S.shape) != tuple(W.shape):
        raise ValueError("S and W shapes differ")
    rows, cols = W.shape
    out = _mask_buffer(W, out)
    st = lib().tsenor_round(ctypes.c_void_p(S.data_ptr()), S.stride(0),
                            ctypes.c_void_p(W.data_ptr()), dt, rows, cols, W.stride(0), N, M,
                            int(ls_steps), ctypes.c_void_p(out.data_ptr()), _stream(stream))
    if st != 0:
        raise TsenorError(st, "tsenor_round")
    return out


def mask_batched(items, tau: float, iters: int, ls_steps: int, return_frac: bool = False,
                 outs=None, stream=None, polish_steps: int = 0, prev_masks=None):
    """Many matrices in one call (one launch per N:M and dtype class).
    items: iterable of (W, N, M); outs: optional list of mask buffers, one per
    item.  polish_steps and prev_masks (a list with one previous mask or None
    per item; an entry may be the item's output buffer) add tsenor_mask_ex's
    optional stages.  Returns a list of (mask, frac_or_None) in the same order."""
    torch = _torch()
    items = list(items)
    if outs is not None and len(outs) != len(items):
        raise ValueError("outs must hold one mask buffer per item")
    if prev_masks is not None and len(prev_masks) != len(items):
        raise ValueError("prev_masks must hold one entry (a mask or None) per item")
    arr = (_Matrix * max(1, len(items)))()
    prevs = (_P * max(1, len(items)))()
    res = []
    for k, (W, N, M) in enumerate(items):
        dt = _weights(W)
        rows, cols = W.shape
        m = _mask_buffer(W, outs[k] if outs is not None else None)
        f = torch.empty((rows, cols), dtype=torch.float32, device=W.device) if return_frac else None
        arr[k] = _Matrix(W.data_ptr(), dt, rows, cols, W.stride(0), N, M, m.data_ptr(),
                         f.data_ptr() if f is not None else 0)
        if prev_masks is not None and prev_masks[k] is not None:
            prevs[k] = _mask_buffer(W, prev_masks[k]).data_ptr()  # same checks as an output
        res.append((m, f))
    if polish_steps == 0 and prev_masks is None:
        st = lib().tsenor_mask_batched(arr, len(items), float(tau), int(iters), int(ls_steps),
                                       _stream(stream))
        where = "tsenor_mask_batched"
    else:
        st = lib().tsenor_mask_batched_ex(arr, len(items), float(tau), int(iters), int(ls_steps),
                                          int(polish_steps),
                                          prevs if prev_masks is not None else None,
                                          _stream(stream))
        where = "tsenor_mask_batched_ex"
    if st != 0:
        raise TsenorError(st, where)
    return res


def memory_pass(W, M: int, out=None, stream=None):
    """Measurement only (tsenor_bench_memory_pass): the memory side of the mask
    search alone -- W read once by M x M blocks, the block max of |W|, and the
    packed bits (2|W| >= block max) written in the mask layout."""
    dt = _weights(W)
    rows, cols = W.shape
    out = _mask_buffer(W, out)
    st = lib().tsenor_bench_memory_pass(ctypes.c_void_p(W.data_ptr()), dt, rows, cols,
                                        W.stride(0), M, ctypes.c_void_p(out.data_ptr()),
                                        _stream(stream))
    if st != 0:
        raise TsenorError(st, "tsenor_bench_memory_pass")
    return out


def unpack(mask_words, cols: int):
    """int32/uint32 words [rows, ceil(cols/32)] -> bool [rows, cols] (same device)."""
    torch = _torch()
    w = mask_words.to(torch.int64) & 0xFFFFFFFF
    bits = (w.unsqueeze(-1) >> torch.arange(32, device=w.device)) & 1
    return bits.reshape(w.shape[0], -1)[:, :cols].bool()
