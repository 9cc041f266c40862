"""Seeded synthetic weight matrices for the mask-search workloads.

This module holds input generation only -- none of the method's arithmetic --
so that both the HIP library's tests/benchmark and the CPU oracle can consume
the identical arrays.  Draws use numpy's PCG64 (``default_rng(seed)``) in
float64, in the order listed per workload; fp32 is ``astype(float32)`` and
bf16 is round-to-nearest-even of that fp32 value (returned as raw uint16 bits;
widening bf16 -> fp32 is exact).

The shapes and distributions stand in for weight blocks of LLaMA-class models
(attention projections 4096x4096, MLP 4096x11008 / 11008x4096 / 8192x28672),
which the TSENOR evaluation samples from real checkpoints that are not used
here.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    N: int
    M: int
    rows: int
    cols: int
    dtype: str  # "f32" or "bf16"
    tau: float
    iters: int
    ls_steps: int
    seed: int
    recipe: str = field(default="", compare=False)

    @property
    def weights(self) -> int:
        return self.rows * self.cols

    @property
    def blocks(self) -> int:
        return (self.rows // self.M) * (self.cols // self.M)


WORKLOADS = {
    "2:4-1024x1024-f32": Workload(
        "2:4-1024x1024-f32", 2, 4, 1024, 1024, "f32", 20.0, 50, 4, 0,
        "standard_normal"),
    "4:8-4096x4096-f32": Workload(
        "4:8-4096x4096-f32", 4, 8, 4096, 4096, "f32", 20.0, 100, 8, 1,
        "0.02*normal + 0.1% +-U(0.5,2) outliers"),
    "8:16-4096x11008-bf16": Workload(
        "8:16-4096x11008-bf16", 8, 16, 4096, 11008, "bf16", 30.0, 150, 16, 2,
        "0.02*student_t(4)"),
    "16:32-8192x28672-bf16": Workload(
        "16:32-8192x28672-bf16", 16, 32, 8192, 28672, "bf16", 40.0, 200, 32, 3,
        "0.015*student_t(3)*lognormal(0,0.5) per column"),
    # The same matrix in the pages' default regime: temperature 0.005 * max|W|
    # read as tau = 200 on block-max-normalised scores, 300 iterations, 10
    # local-search steps.
    "16:32-8192x28672-bf16-tau200": Workload(
        "16:32-8192x28672-bf16-tau200", 16, 32, 8192, 28672, "bf16", 200.0, 300, 10, 3,
        "0.015*student_t(3)*lognormal(0,0.5) per column (as 16:32-8192x28672-bf16)"),
}

# 7B-shaped model: per layer (seed 1000 + layer) q, k, v, o, gate, up, down.
MODEL7B_LAYERS = 32
MODEL7B_MATS = (("q", 4096, 4096, 8, 16), ("k", 4096, 4096, 8, 16),
                ("v", 4096, 4096, 8, 16), ("o", 4096, 4096, 8, 16),
                ("gate", 4096, 11008, 16, 32), ("up", 4096, 11008, 16, 32),
                ("down", 11008, 4096, 16, 32))
MODEL7B_TAU, MODEL7B_ITERS, MODEL7B_LS = 30.0, 150, 16

_CHUNK_ROWS = 512  # row-chunked draws bound host memory on the big shapes


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest-even), returned as uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _outliers(rng: np.random.Generator, W: np.ndarray) -> None:
    n = W.size
    k = int(round(0.001 * n))
    pos = rng.choice(n, k, replace=False)
    vals = rng.choice(np.array([-1.0, 1.0]), k) * rng.uniform(0.5, 2.0, k)
    W.reshape(-1)[pos] = vals


def _normal_outlier_matrix(rng, rows, cols):
    W = 0.02 * rng.standard_normal((rows, cols))
    _outliers(rng, W)
    return W


def generate(name: str, rows: int = None) -> np.ndarray:
    """Weights of a named workload: fp32 array, or uint16 bf16 bits.  With
    `rows`, only the first rows of the same matrix (the row-chunked bf16
    workloads stop drawing there; the fp32 ones draw in full and slice)."""
    w = WORKLOADS[name]
    if rows is not None:
        if rows <= 0 or rows > w.rows:
            raise ValueError("rows out of range")
        if w.M in (16, 32):
            import dataclasses
            w = dataclasses.replace(w, rows=rows)
        else:
            return np.ascontiguousarray(generate(name)[:rows])
    rng = np.random.default_rng(w.seed)
    if w.M == 4:
        W = rng.standard_normal((w.rows, w.cols))
        return W.astype(np.float32)
    if w.M == 8:
        return _normal_outlier_matrix(rng, w.rows, w.cols).astype(np.float32)
    if w.M == 16:
        out = np.empty((w.rows, w.cols), np.uint16)
        for r0 in range(0, w.rows, _CHUNK_ROWS):
            r1 = min(w.rows, r0 + _CHUNK_ROWS)
            out[r0:r1] = f32_to_bf16_bits(
                (0.02 * rng.standard_t(4, (r1 - r0, w.cols))).astype(np.float32))
        return out
    if w.M == 32:
        s = rng.lognormal(0.0, 0.5, w.cols)
        out = np.empty((w.rows, w.cols), np.uint16)
        for r0 in range(0, w.rows, _CHUNK_ROWS):
            r1 = min(w.rows, r0 + _CHUNK_ROWS)
            x = 0.015 * rng.standard_t(3, (r1 - r0, w.cols)) * s[None, :]
            out[r0:r1] = f32_to_bf16_bits(x.astype(np.float32))
        return out
    raise KeyError(name)


def wanda_scores(W: np.ndarray, seed: int) -> np.ndarray:
    """Wanda-style importance scores |W_ij| * ||X_j|| as an fp32 matrix, with
    synthetic per-input-column activation norms ||X_j|| ~ LogNormal(0, 1)
    drawn from default_rng(seed) -- an example of a score matrix other than
    |W| that the mask search can be run on."""
    rng = np.random.default_rng(seed)
    norms = rng.lognormal(0.0, 1.0, W.shape[1])
    return (np.abs(W.astype(np.float64)) * norms[None, :]).astype(np.float32)


def model7b_layer(layer: int, which=None):
    """Yield (name, N, M, bf16-bits matrix) for one layer of the 7B-shaped model,
    drawing every matrix in order from one generator seeded 1000 + layer."""
    rng = np.random.default_rng(1000 + layer)
    for (nm, rows, cols, N, M) in MODEL7B_MATS:
        W = _normal_outlier_matrix(rng, rows, cols)
        if which is None or nm in which:
            yield nm, N, M, f32_to_bf16_bits(W.astype(np.float32))


def random_blocks(seed: int, nblocks: int, M: int, kind: str = "normal") -> np.ndarray:
    """Small fp32 test matrices [M, nblocks*M] (a row of blocks) with a chosen
    value distribution: normal, outlier, student_t, ties (values from a 3-level
    set), zero (all-zero blocks), uniform."""
    rng = np.random.default_rng(seed)
    shape = (M, nblocks * M)
    if kind == "normal":
        W = rng.standard_normal(shape)
    elif kind == "outlier":
        W = 0.02 * rng.standard_normal(shape)
        _outliers(rng, W)
        # make sure there is at least one outlier per few blocks
        W[rng.integers(0, M, nblocks), np.arange(nblocks) * M + rng.integers(0, M, nblocks)] = 1.5
    elif kind == "student_t":
        W = 0.02 * rng.standard_t(3, shape)
    elif kind == "ties":
        W = rng.choice(np.array([0.25, 0.5, 1.0, -0.5]), shape)
    elif kind == "zero":
        W = np.zeros(shape)
    elif kind == "uniform":
        W = rng.uniform(-1.0, 1.0, shape)
    else:
        raise ValueError(kind)
    return W.astype(np.float32)
