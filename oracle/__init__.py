"""CPU oracle for transposable N:M mask search -- TEST INFRASTRUCTURE ONLY.

Only the test-suite, the smoke check and the CPU-baseline leg of the benchmark
may import this package.  It wraps ``tsenor_oracle.c`` (plain C, fp64 Dykstra,
deterministic rounding, exact min-cost-flow optimum) through ctypes and adds a
few pure-numpy exact checkers for tiny blocks.  It imports nothing from the
HIP library package and shares no code with it.

Method source: pith.science review of "TSENOR: Highly-Efficient Algorithm for
Finding Transposable N:M Sparse Masks" (arXiv 2505.23949), sections "What
carries the argument" and "Core claim".
"""
from __future__ import annotations

import ctypes
import itertools
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tsenor_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I = ctypes.c_int
_D = ctypes.c_double


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2 -fopenmp, no fast-math, no contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
             "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or (
                os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.oracle_dykstra.argtypes = [_P, _I64, _I64, _I64, _I, _I, _D, _I, _P, _P, _I]
        lib.oracle_dykstra_blocks.argtypes = [_P, _I64, _I64, _I64, _I, _I, _D, _I,
                                              _P, _I64, _P, _P, _I]
        lib.oracle_round_block.argtypes = [_P, _P, _I, _I, _I, _P, _P, _P, _P, _P]
        lib.oracle_dykstra_blocks_f32.argtypes = [_P, _I64, _I64, _I64, _I, _I, ctypes.c_float,
                                                  _I, _P, _I64, _P, _I]
        lib.oracle_round.argtypes = [_P, _I64, _P, _I64, _I64, _I64, _I, _I, _I, _P, _P, _I]
        lib.oracle_round_block_ex.argtypes = [_P, _P, _I, _I, _I, _I, _P, _P, _P, _P]
        lib.oracle_round_ex.argtypes = [_P, _I64, _P, _I64, _I64, _I64, _I, _I, _I, _I, _P, _P,
                                        _P, _I]
        lib.oracle_exact_opt_block.argtypes = [_P, _I, _I, _P]
        lib.oracle_exact_opt_block.restype = _D
        lib.oracle_exact_opt_blocks.argtypes = [_P, _I64, _I64, _I64, _I, _I, _P, _I64, _P, _I]
        lib.oracle_max_threads.restype = _I
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _f32(W) -> np.ndarray:
    W = np.ascontiguousarray(np.asarray(W, dtype=np.float32))
    if W.ndim != 2:
        raise ValueError("W must be 2-D")
    return W


def _check(status: int, what: str):
    if status != 0:
        names = {1: "bad argument", 2: "non-finite input", 3: "rounding invariant violated"}
        raise ValueError(f"oracle {what}: {names.get(status, status)}")


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def dykstra(W, N: int, M: int, tau: float, iters: int, nthreads: int = 0):
    """fp64 Dykstra on every block.  Returns (S64, S32), each [rows, cols]."""
    W = _f32(W)
    rows, cols = W.shape
    S64 = np.empty((rows, cols), np.float64)
    S32 = np.empty((rows, cols), np.float32)
    _check(_load().oracle_dykstra(_ptr(W), rows, cols, cols, N, M, float(tau), iters,
                                  _ptr(S64), _ptr(S32), nthreads), "dykstra")
    return S64, S32


def dykstra_blocks(W, N: int, M: int, tau: float, iters: int, block_ids, nthreads: int = 0):
    """fp64 Dykstra on the listed blocks (id = bi*(cols/M)+bj).
    Returns (S64, S32), each [len(block_ids), M, M]."""
    W = _f32(W)
    rows, cols = W.shape
    ids = np.ascontiguousarray(np.asarray(block_ids, dtype=np.int64))
    S64 = np.empty((len(ids), M, M), np.float64)
    S32 = np.empty((len(ids), M, M), np.float32)
    _check(_load().oracle_dykstra_blocks(_ptr(W), rows, cols, cols, N, M, float(tau), iters,
                                         _ptr(ids), len(ids), _ptr(S64), _ptr(S32),
                                         nthreads), "dykstra_blocks")
    return S64, S32


def round_block(S32, A, N: int, ls_steps: int, trace: bool = False, moves: bool = False):
    """Greedy + local search + fill on one block.  Returns (Z uint8 [M,M], info)
    with info = (shortfall after greedy, local-search moves, fill moves); with
    trace=True also the greedy-only mask and the fp32 score of every applied
    move, in order; with moves=True as well (after those) the applied moves
    as an int array [n, 4] of (i, j, i', j'), local-search moves first."""
    S32 = np.ascontiguousarray(np.asarray(S32, dtype=np.float32))
    A = np.ascontiguousarray(np.asarray(A, dtype=np.float32))
    M = S32.shape[0]
    Z = np.zeros((M, M), np.uint8)
    Zg = np.zeros((M, M), np.uint8)
    scores = np.zeros(M * M, np.float32)
    ijs = np.zeros((M * M, 4), np.int32)
    info = np.zeros(3, np.int32)
    _check(_load().oracle_round_block(_ptr(S32), _ptr(A), N, M, ls_steps, _ptr(Z),
                                      _ptr(info), _ptr(Zg), _ptr(scores), _ptr(ijs)),
           "round_block")
    info = tuple(int(x) for x in info)
    n = info[1] + info[2]
    if trace and moves:
        return Z, info, Zg, scores[:n].copy(), ijs[:n].copy()
    if trace:
        return Z, info, Zg, scores[:n].copy()
    if moves:
        return Z, info, ijs[:n].copy()
    return Z, info


def dykstra_blocks_f32(W, N: int, M: int, tau: float, iters: int, block_ids, nthreads: int = 0):
    """The Dykstra steps in fp32 (expf/logf) on the listed blocks: the method's
    own fp32 sensitivity.  Returns S32 [len(block_ids), M, M]."""
    W = _f32(W)
    rows, cols = W.shape
    ids = np.ascontiguousarray(np.asarray(block_ids, dtype=np.int64))
    S = np.empty((len(ids), M, M), np.float32)
    _check(_load().oracle_dykstra_blocks_f32(_ptr(W), rows, cols, cols, N, M, float(tau), iters,
                                             _ptr(ids), len(ids), _ptr(S), nthreads),
           "dykstra_blocks_f32")
    return S


def round_matrix(S32, W, N: int, M: int, ls_steps: int, nthreads: int = 0):
    """Rounding of every block.  Returns (mask uint32 [rows, ceil(cols/32)],
    stats = [blocks with shortfall, total shortfall, R2 moves, R3 moves])."""
    S32 = np.ascontiguousarray(np.asarray(S32, dtype=np.float32))
    W = _f32(W)
    rows, cols = W.shape
    if S32.shape != W.shape:
        raise ValueError("S32 and W shapes differ")
    mask = np.zeros((rows, (cols + 31) // 32), np.uint32)
    stats = np.zeros(4, np.int64)
    _check(_load().oracle_round(_ptr(S32), cols, _ptr(W), cols, rows, cols, N, M, ls_steps,
                                _ptr(mask), _ptr(stats), nthreads), "round")
    return mask, stats


def round_block_ex(S32, A, N: int, ls_steps: int, polish_steps: int, prev=None):
    """round_block followed by the optional 2-opt polish (at most polish_steps
    swaps) and the keep-better safeguard against `prev` (0/1 [M,M] or None).
    Returns (Z, info, gains) with info = (shortfall, local-search moves, fill
    moves, polish swaps, 1 if prev was kept) and the applied swap gains."""
    S32 = np.ascontiguousarray(np.asarray(S32, dtype=np.float32))
    A = np.ascontiguousarray(np.asarray(A, dtype=np.float32))
    M = S32.shape[0]
    Z = np.zeros((M, M), np.uint8)
    info = np.zeros(5, np.int32)
    gains = np.zeros(max(1, polish_steps), np.float32)
    P = None if prev is None else np.ascontiguousarray(np.asarray(prev, dtype=np.uint8))
    _check(_load().oracle_round_block_ex(_ptr(S32), _ptr(A), N, M, ls_steps, polish_steps,
                                         _ptr(P) if P is not None else None, _ptr(Z),
                                         _ptr(info), _ptr(gains)), "round_block_ex")
    info = tuple(int(x) for x in info)
    return Z, info, gains[:info[3]].copy()


def round_matrix_ex(S32, W, N: int, M: int, ls_steps: int, polish_steps: int,
                    prev_mask=None, nthreads: int = 0):
    """round_matrix with the optional stages.  prev_mask: packed uint32 words
    like the output, or None.  Returns (mask, stats) with stats = [blocks with
    shortfall, total shortfall, R2 moves, R3 moves, R4 swaps, blocks that kept
    the previous mask]."""
    S32 = np.ascontiguousarray(np.asarray(S32, dtype=np.float32))
    W = _f32(W)
    rows, cols = W.shape
    if S32.shape != W.shape:
        raise ValueError("S32 and W shapes differ")
    mask = np.zeros((rows, (cols + 31) // 32), np.uint32)
    P = None
    if prev_mask is not None:
        P = np.ascontiguousarray(np.asarray(prev_mask, dtype=np.uint32))
        if P.shape != mask.shape:
            raise ValueError("prev_mask shape differs from the mask's")
    stats = np.zeros(6, np.int64)
    _check(_load().oracle_round_ex(_ptr(S32), cols, _ptr(W), cols, rows, cols, N, M, ls_steps,
                                   polish_steps, _ptr(P) if P is not None else None, _ptr(mask),
                                   _ptr(stats), nthreads), "round_ex")
    return mask, stats


def tsenor(W, N: int, M: int, tau: float, iters: int, ls_steps: int, nthreads: int = 0):
    """Whole method on every block: returns (mask, S64, S32, stats)."""
    S64, S32 = dykstra(W, N, M, tau, iters, nthreads)
    mask, stats = round_matrix(S32, W, N, M, ls_steps, nthreads)
    return mask, S64, S32, stats


def exact_opt_block(A, N: int):
    """Exact optimum (objective, mask) of one block by min-cost flow."""
    A = np.ascontiguousarray(np.asarray(A, dtype=np.float32))
    M = A.shape[0]
    Z = np.zeros((M, M), np.uint8)
    obj = _load().oracle_exact_opt_block(_ptr(A), N, M, _ptr(Z))
    return float(obj), Z


def exact_opt_blocks(W, N: int, M: int, block_ids, nthreads: int = 0) -> np.ndarray:
    W = _f32(W)
    rows, cols = W.shape
    ids = np.ascontiguousarray(np.asarray(block_ids, dtype=np.int64))
    opt = np.empty(len(ids), np.float64)
    _check(_load().oracle_exact_opt_blocks(_ptr(W), rows, cols, cols, N, M, _ptr(ids),
                                           len(ids), _ptr(opt), nthreads), "exact_opt")
    return opt


# --------------------------------------------------------------------------
# Pure-numpy helpers (tiny blocks only).

def feasible_masks(M: int, N: int) -> np.ndarray:
    """All M x M 0/1 matrices with exactly N ones in every row and column,
    by brute-force enumeration (row patterns, filtered on column sums)."""
    pats = [np.array(p, np.uint8) for p in itertools.product((0, 1), repeat=M)
            if sum(p) == N]
    out = []
    for rows in itertools.product(pats, repeat=M):
        Z = np.stack(rows)
        if np.all(Z.sum(0) == N):
            out.append(Z)
    return np.stack(out)


def unpack_mask(words: np.ndarray, cols: int) -> np.ndarray:
    """uint32 words [rows, ceil(cols/32)] -> bool [rows, cols], LSB first."""
    words = np.asarray(words, dtype=np.uint32)
    bits = (words[:, :, None] >> np.arange(32, dtype=np.uint32)) & 1
    return bits.reshape(words.shape[0], -1)[:, :cols].astype(bool)


def block_view(X: np.ndarray, M: int) -> np.ndarray:
    """[rows, cols] -> [rows/M, cols/M, M, M] (copy)."""
    r, c = X.shape
    return X.reshape(r // M, M, c // M, M).transpose(0, 2, 1, 3).copy()


# --------------------------------------------------------------------------
# 2:4 compressed operand (the consumer of transposable masks; format as in
# include/tsenor.h's tsenor_compress24 -- restated here from its definition).

def compress24(W_bits, mask_words, transpose: bool = False):
    """A = W (or W^T) restricted to the mask, compressed 2:4 along its rows.
    W_bits: uint16 bf16 bit patterns [rows, cols]; mask_words: uint32 packed
    mask.  Returns (values uint16 [arows, k/2], meta uint32 [arows, k/32],
    groups with more than two kept entries)."""
    W_bits = np.asarray(W_bits, dtype=np.uint16)
    rows, cols = W_bits.shape
    Z = unpack_mask(np.asarray(mask_words, dtype=np.uint32), cols)
    A, ZA = (W_bits.T, Z.T) if transpose else (W_bits, Z)
    arows, k = A.shape
    if k % 32:
        raise ValueError("k must be a multiple of 32")
    vals = np.zeros((arows, k // 2), np.uint16)
    meta = np.zeros((arows, k // 32), np.uint32)
    bad = 0
    for r in range(arows):
        for g in range(k // 4):
            pos = [j for j in range(4) if ZA[r, 4 * g + j]]
            bad += len(pos) > 2
            pos = pos[:2]
            if len(pos) == 0:
                code = 0 | (1 << 2)
            elif len(pos) == 1:
                code = pos[0] | ((2 if pos[0] == 3 else 3) << 2)
            else:
                code = pos[0] | (pos[1] << 2)
            for s_, p in enumerate(pos):
                vals[r, 2 * g + s_] = A[r, 4 * g + p]
            meta[r, g // 8] |= np.uint32(code << (4 * (g % 8)))
    return vals, meta, bad


def decompress24(vals, meta, k: int):
    """Dense fp32 [arows, k] from the compressed operand (unused slots are 0)."""
    vals = np.asarray(vals, dtype=np.uint16)
    arows = vals.shape[0]
    out = np.zeros((arows, k), np.float32)
    f = (vals.astype(np.uint32) << 16).view(np.float32)
    for r in range(arows):
        for g in range(k // 4):
            code = (int(meta[r, g // 8]) >> (4 * (g % 8))) & 0xF
            for s_, p in enumerate((code & 3, code >> 2)):
                out[r, 4 * g + p] += f[r, 2 * g + s_]
    return out
