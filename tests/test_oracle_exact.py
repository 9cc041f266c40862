"""Pins for the oracle's exact optimum (min-cost flow) of the per-block problem.

The per-block problem and the integrality of its LP relaxation (bipartite
b-matching polytope, total unimodularity) are stated in the pith.science
review of TSENOR, "Core claim".  Every check here compares the oracle's
min-cost flow against something computed another way: brute force over the
feasible masks, scipy's HiGHS LP, scipy's assignment solver (N = 1), and
closed forms (N = M, N = M - 1).
"""
import json
import os

import numpy as np
import pytest
from scipy.optimize import linear_sum_assignment, linprog

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _blocks(seed, n, M, kind):
    rng = np.random.default_rng(seed)
    if kind == "normal":
        X = rng.standard_normal((n, M, M))
    elif kind == "ties":
        X = rng.choice([0.5, 1.0, 2.0], (n, M, M))
    elif kind == "outlier":
        X = 0.02 * rng.standard_normal((n, M, M))
        X[:, 0, 0] = 1.5
    else:
        X = rng.standard_t(3, (n, M, M))
    return np.abs(X).astype(np.float32)


def test_feasible_counts_match_golden():
    with open(os.path.join(GOLDEN, "feasible_counts.json")) as f:
        counts = json.load(f)["counts"]
    for M, N, expected in counts:
        Z = oracle.feasible_masks(M, N)
        assert len(Z) == expected, (M, N)
        assert np.all(Z.sum(1) == N) and np.all(Z.sum(2) == N)
        assert len({z.tobytes() for z in Z}) == expected


@pytest.mark.parametrize("N", [1, 2, 3])
@pytest.mark.parametrize("kind", ["normal", "ties", "outlier", "t"])
def test_mcf_equals_bruteforce_4x4(N, kind):
    masks = oracle.feasible_masks(4, N).astype(np.float64)
    A = _blocks(11 + N, 150, 4, kind)
    for a in A:
        brute = np.max((masks * a.astype(np.float64)).sum((1, 2)))
        obj, Z = oracle.exact_opt_block(a, N)
        assert obj == pytest.approx(brute, rel=1e-12, abs=1e-12)
        assert np.all(Z.sum(0) == N) and np.all(Z.sum(1) == N)
        assert (Z * a.astype(np.float64)).sum() == pytest.approx(obj, rel=1e-12)


@pytest.mark.parametrize("M,N", [(8, 4), (8, 3), (16, 8), (16, 5)])
def test_mcf_equals_highs_lp(M, N):
    A = _blocks(3 + M + N, 12, M, "t")
    # LP: max <S, A>, rows and columns sum to N, 0 <= S <= 1
    Aeq = np.zeros((2 * M, M * M))
    for i in range(M):
        Aeq[i, i * M:(i + 1) * M] = 1
        Aeq[M + i, i::M] = 1
    beq = np.full(2 * M, float(N))
    for a in A:
        res = linprog(-a.astype(np.float64).ravel(), A_eq=Aeq, b_eq=beq, bounds=(0, 1),
                      method="highs")
        assert res.status == 0
        obj, _ = oracle.exact_opt_block(a, N)
        assert obj == pytest.approx(-res.fun, rel=1e-9)
        # integrality of the LP vertex (total unimodularity)
        assert np.allclose(res.x, np.round(res.x), atol=1e-7)


@pytest.mark.parametrize("M", [4, 8, 16, 32])
def test_mcf_n1_equals_assignment(M):
    A = _blocks(5 * M, 10, M, "normal")
    for a in A:
        r, c = linear_sum_assignment(a.astype(np.float64), maximize=True)
        best = a.astype(np.float64)[r, c].sum()
        obj, _ = oracle.exact_opt_block(a, 1)
        assert obj == pytest.approx(best, rel=1e-12)


@pytest.mark.parametrize("M", [4, 8, 32])
def test_mcf_closed_forms(M):
    A = _blocks(7 * M, 5, M, "t").astype(np.float64)
    for a in A:
        obj, Z = oracle.exact_opt_block(a.astype(np.float32), M)
        assert obj == pytest.approx(a.sum(), rel=1e-12) and Z.all()
        # N = M - 1 is the complement of a minimum-weight assignment
        r, c = linear_sum_assignment(a)
        obj, _ = oracle.exact_opt_block(a.astype(np.float32), M - 1)
        assert obj == pytest.approx(a.sum() - a[r, c].sum(), rel=1e-12)
