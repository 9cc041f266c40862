"""The checkers the GPU parity tests rely on reject what they must (CPU only).

assert_feasible must fail on a single flipped mask bit and on a bit set beyond
the last column of a ragged row; assert_S_close must fail once S is off by
2e-4 anywhere and pass at half the tolerance.  Inputs come from the oracle.
"""
import numpy as np
import pytest

import oracle
from sparse_mask_search_amd import workloads as wl
from gpu_util import assert_S_close, assert_feasible


def _case(M=8, N=4, nbc=5):
    W = np.concatenate([wl.random_blocks(21, nbc, M, "student_t"),
                        wl.random_blocks(22, nbc, M, "outlier")])
    mask, S64, S32, _ = oracle.tsenor(W, N, M, 20.0, 30, M)
    return W, mask, S64, N, M


def test_flipped_bit_is_infeasible():
    W, mask, _, N, M = _case()
    rows, cols = W.shape
    assert_feasible(mask, rows, cols, N, M)
    for r, c in [(0, 0), (3, 17), (rows - 1, cols - 1)]:
        bad = mask.copy()
        bad[r, c // 32] ^= np.uint32(1 << (c % 32))
        with pytest.raises(AssertionError):
            assert_feasible(bad, rows, cols, N, M)


def test_bit_beyond_last_column_is_rejected():
    W, mask, _, N, M = _case(nbc=5)  # 40 columns: the second word of a row is ragged
    rows, cols = W.shape
    assert cols % 32 != 0
    bad = mask.copy()
    bad[1, -1] |= np.uint32(1 << 31)
    with pytest.raises(AssertionError):
        assert_feasible(bad, rows, cols, N, M)


def test_S_tolerance_is_enforced():
    _, _, S64, _, _ = _case()
    S = S64.astype(np.float32)
    assert assert_S_close(S, S64) < 1e-6
    off = S64.copy()
    off[5, 7] += 2e-4
    with pytest.raises(AssertionError):
        assert_S_close(off.astype(np.float32), S64)
    half = S64 + 5e-5
    assert_S_close(half, S64)
    with pytest.raises(AssertionError):
        assert_S_close(S[:, :-1], S64)
