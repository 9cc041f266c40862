"""A numpy model (fp32) of the kernels' scaling-form Dykstra iteration and its
scale guard -- test infrastructure, used only to show on the CPU that a test
input reaches the guard's linear fold before the GPU runs it.

The kernels run cycle 1 in log2 space (C1 then C2 with max-shifted
log-sum-exp), keep P = 2^Y, and run every later cycle as
    E = min(P V U, 1);  U *= N / rowsum(E);  V *= N / colsum(E * a).
Every fourth cycle a block whose row or column scales left [2^-40, 2^40]
folds them into its kernel.  A block whose cycle-1 kernel reaches below
2^-100 is "deep" and folds in log2 space; any other block folds linearly
(P <- P V U).  This model follows those steps in fp32 (it is not
bit-identical to the kernels: sums run in numpy's order) and reports, per
block, whether it is deep and how often it folded.
"""
import numpy as np

DEEP_LOG2 = -100.0
GUARD = 2.0 ** 40


def blocks_of(W, M):
    rows, cols = W.shape
    A = np.abs(np.asarray(W, np.float32))
    return A.reshape(rows // M, M, cols // M, M).transpose(0, 2, 1, 3).reshape(-1, M, M)


def guard_events(W, N, M, tau, iters):
    """(folds per block, deep flag per block) of the modelled iteration."""
    f = np.float32
    A = blocks_of(W, M)
    m = A.max((1, 2), keepdims=True)
    scale = np.where(m > 0, f(tau * 1.4426950408889634) / np.where(m > 0, m, f(1)), f(0))
    P = (A * scale.astype(f)).astype(f)
    l2N = f(np.log2(N))
    mx = P.max(2, keepdims=True)
    P = (P + (l2N - mx - np.log2(np.exp2(P - mx).sum(2, keepdims=True, dtype=f)))).astype(f)
    mx = P.max(1, keepdims=True)
    P = (P + (l2N - mx - np.log2(np.exp2(P - mx).sum(1, keepdims=True, dtype=f)))).astype(f)
    deep = P.min((1, 2)) < DEEP_LOG2
    P = np.exp2(P).astype(f)
    U = np.ones((P.shape[0], M, 1), f)
    V = np.ones((P.shape[0], 1, M), f)
    folds = np.zeros(P.shape[0], np.int64)
    for it in range(1, iters):
        E = np.minimum((P * V) * U, f(1))
        a = (f(N) / E.sum(2, keepdims=True, dtype=f)).astype(f)
        U = (U * a).astype(f)
        V = (V * (f(N) / (E * a).sum(1, keepdims=True, dtype=f))).astype(f)
        if it % 4 == 0:
            bad = (((U < 1 / GUARD) | (U > GUARD)).any((1, 2))
                   | ((V < 1 / GUARD) | (V > GUARD)).any((1, 2)))
            if bad.any():
                folds += bad
                k = np.nonzero(bad & ~deep)[0]
                P[k] = (P[k] * V[k]) * U[k]
                U[bad] = 1
                V[bad] = 1
    return folds, deep
