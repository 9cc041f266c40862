"""Pins of the oracle's optional stages after the fill: the 2-opt polish (R4)
and the keep-better safeguard against a previous mask (R5).

These stages are not on the pages; their reading:
a swap takes kept (i, j), (i', j'), i < i', with Z_ij' = Z_i'j = 0, to (i, j'),
(i', j); gain (A_ij' - A_i'j') + (A_i'j - A_ij) in fp32; best gain, ties to the
smallest (i, j, i', j'), applied only if > 0; the safeguard keeps a feasible
previous mask whose fp64 objective is strictly larger.

Independent checks: with small-integer scores every fp32 operation is exact,
so brute force in exact integer arithmetic decides local optimality and the
objective change of every swap; a hand-derived 4x4 case fixes the first swap;
the exact optimum (min-cost flow, pinned in test_oracle_exact) bounds and, as a
previous mask, replaces the result.
"""
import itertools

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.filterwarnings("ignore")


def _swaps(Z, A):
    """Every admissible swap (i<i') with its exact integer gain."""
    M = Z.shape[0]
    out = []
    for i, ip in itertools.combinations(range(M), 2):
        for j in range(M):
            if not Z[i, j] or Z[ip, j]:
                continue
            for jp in range(M):
                if Z[ip, jp] and not Z[i, jp]:
                    g = int(A[i, jp]) + int(A[ip, j]) - int(A[i, j]) - int(A[ip, jp])
                    out.append(((i, j, ip, jp), g))
    return out


def _int_case(rng, M, N, hi=50):
    A = rng.integers(0, hi, (M, M)).astype(np.float32)
    S = rng.random((M, M)).astype(np.float32)
    return S, A


@pytest.mark.parametrize("M,N", [(4, 2), (8, 4), (8, 3), (16, 8), (32, 16)])
def test_polish_reaches_a_2opt_local_optimum(M, N):
    rng = np.random.default_rng(M * 10 + N)
    for _ in range(6 if M <= 16 else 2):
        S, A = _int_case(rng, M, N)
        Z0, _ = oracle.round_block(S, A, N, ls_steps=M)
        Z, info, gains = oracle.round_block_ex(S, A, N, M, 10 ** 6)
        assert info[4] == 0
        assert (Z.sum(0) == N).all() and (Z.sum(1) == N).all()
        # no admissible swap is improving (exact arithmetic)
        assert all(g <= 0 for _, g in _swaps(Z, A))
        # objective grew by exactly the applied gains, each positive
        assert (gains > 0).all()
        assert float((Z * A).sum() - (Z0 * A).sum()) == float(gains.astype(np.float64).sum())
        # and never beyond the exact optimum
        opt, _ = oracle.exact_opt_block(A, N)
        assert (Z * A).sum() <= opt + 1e-9


@pytest.mark.parametrize("M,N", [(4, 2), (8, 3), (16, 5)])
def test_each_swap_is_the_lexicographic_best(M, N):
    """One step at a time: the applied swap has the largest exact gain, and
    among equal gains the smallest (i, j, i', j') -- small scores force ties."""
    rng = np.random.default_rng(7 + M)
    for _ in range(8):
        S, A = _int_case(rng, M, N, hi=4)
        Z, _ = oracle.round_block(S, A, N, ls_steps=M)
        for step in range(6):
            cand = _swaps(Z, A)
            Z1, info, gains = oracle.round_block_ex(S, A, N, M, step + 1)
            if not cand or max(g for _, g in cand) <= 0:
                assert info[3] == step
                break
            best = max(g for _, g in cand)
            i, j, ip, jp = min(k for k, g in cand if g == best)
            Z2 = Z.copy()
            Z2[i, j] = Z2[ip, jp] = 0
            Z2[i, jp] = Z2[ip, j] = 1
            assert info[3] == step + 1 and gains[-1] == best
            assert np.array_equal(Z1, Z2)
            Z = Z2


def test_hand_derived_first_swap():
    """4x4, N = 2.  S makes the greedy take the two diagonal 2x2 tiles (no
    shortfall, so no local search or fill).  Scores: 1 on those tiles, 5 at
    (0,2) and (2,0), 0 elsewhere.  Swap (0,0),(2,2) -> (0,2),(2,0) gains
    (5 - 1) + (5 - 1) = 8; every other admissible swap gains at most 3
    (e.g. (0,0),(2,3): (0 - 1) + (5 - 1)).  One step takes exactly that swap."""
    hi, lo = 0.9, 0.1
    S = np.array([[hi, hi, lo, lo], [hi, hi, lo, lo], [lo, lo, hi, hi], [lo, lo, hi, hi]],
                 np.float32)
    A = np.array([[1, 1, 5, 0], [1, 1, 0, 0], [5, 0, 1, 1], [0, 0, 1, 1]], np.float32)
    Z0, info0 = oracle.round_block(S, A, 2, ls_steps=4)
    assert info0 == (0, 0, 0)
    assert np.array_equal(Z0, (S > 0.5).astype(np.uint8))
    Z, info, gains = oracle.round_block_ex(S, A, 2, 4, 1)
    assert info[3] == 1 and gains[0] == 8.0
    expect = np.array([[0, 1, 1, 0], [1, 1, 0, 0], [1, 0, 0, 1], [0, 0, 1, 1]], np.uint8)
    assert np.array_equal(Z, expect)


def test_keep_better_previous_mask():
    rng = np.random.default_rng(3)
    M, N = 8, 3
    S, A = _int_case(rng, M, N)
    Z, info, _ = oracle.round_block_ex(S, A, N, 2, 0)
    opt, Zopt = oracle.exact_opt_block(A, N)
    # a strictly better feasible previous mask is taken
    if (Zopt * A).sum() > (Z * A).sum():
        Zk, infok, _ = oracle.round_block_ex(S, A, N, 2, 0, prev=Zopt)
        assert infok[4] == 1 and np.array_equal(Zk, Zopt)
    # an equal one is not (ties keep the new mask), a worse one is not
    Ze, infoe, _ = oracle.round_block_ex(S, A, N, 2, 0, prev=Z)
    assert infoe[4] == 0 and np.array_equal(Ze, Z)
    worst = np.zeros((M, M), np.uint8)
    for i in range(M):  # a feasible circulant mask with the smallest scores first
        for k in range(N):
            worst[i, (i + k) % M] = 1
    if (worst * A).sum() < (Z * A).sum():
        Zw, infow, _ = oracle.round_block_ex(S, A, N, 2, 0, prev=worst)
        assert infow[4] == 0 and np.array_equal(Zw, Z)
    # an infeasible previous mask is ignored however large its objective
    full = np.ones((M, M), np.uint8)
    Zi, infoi, _ = oracle.round_block_ex(S, A, N, 2, 0, prev=full)
    assert infoi[4] == 0 and np.array_equal(Zi, Z)


def test_matrix_level_stages():
    rng = np.random.default_rng(11)
    N, M, rows, cols = 4, 8, 32, 48
    W = (rng.integers(-20, 21, (rows, cols))).astype(np.float32)
    S = rng.random((rows, cols)).astype(np.float32)
    base, st = oracle.round_matrix(S, W, N, M, 4)
    same, st2 = oracle.round_matrix_ex(S, W, N, M, 4, 0)
    assert np.array_equal(base, same) and (st2[:4] == st).all() and st2[4] == st2[5] == 0
    pol, st3 = oracle.round_matrix_ex(S, W, N, M, 4, 50)
    A = np.abs(W)
    Zb = oracle.unpack_mask(base, cols).astype(np.float64)
    Zp = oracle.unpack_mask(pol, cols).astype(np.float64)
    assert (Zp * A).sum() >= (Zb * A).sum() and st3[4] > 0
    # the polished mask as the previous mask of an unpolished run: every block
    # that the polish improved takes it
    back, st4 = oracle.round_matrix_ex(S, W, N, M, 4, 0, prev_mask=pol)
    assert np.array_equal(back, pol)
    improved = 0
    for bi in range(rows // M):
        for bj in range(cols // M):
            sl = (slice(bi * M, bi * M + M), slice(bj * M, bj * M + M))
            improved += (Zp[sl] * A[sl]).sum() > (Zb[sl] * A[sl]).sum()
    assert st4[5] == improved
