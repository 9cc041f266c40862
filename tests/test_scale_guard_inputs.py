"""The inputs of the GPU scale-fold test reach the kernels' linear fold
(CPU only, by the fp32 model in tests/scale_guard_model.py).

With N close to M the converged S is nearly all ones, so entries with a small
Gibbs kernel need row and column scales near 1 / kernel: at tau = 40 that is
up to 2^57, past the guard's 2^40, in blocks that are not deep (cycle-1
kernel above 2^-100).  The GPU test tests/test_gpu_parity.py
(test_scale_fold_inputs) runs the same inputs against the oracle.
"""
import numpy as np
import pytest

from scale_guard_model import guard_events
from sparse_mask_search_amd import workloads as wl

FOLD_CASES = [(31, 32, 40.0, 60), (15, 16, 40.0, 60), (7, 8, 40.0, 60), (3, 4, 60.0, 60)]


def fold_input(N, M, seed=7):
    """A few block-rows of normal weights: the scale-fold test's input."""
    return np.concatenate([wl.random_blocks(seed + r, 12, M, "normal") for r in range(3)])


@pytest.mark.parametrize("N,M,tau,iters", FOLD_CASES)
def test_fold_inputs_reach_the_linear_fold(N, M, tau, iters):
    W = fold_input(N, M)
    folds, deep = guard_events(W, N, M, tau, iters)
    assert not deep.any()
    assert (folds > 0).mean() > 0.3, (folds > 0).mean()
