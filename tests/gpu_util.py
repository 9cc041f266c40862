"""Shared helpers of the GPU tests: move seeded inputs to the device, run the
library, and compare with the oracle.  Imported by tests only."""
import numpy as np

import oracle
from sparse_mask_search_amd import workloads as wl


def to_device(W_np):
    """fp32 ndarray -> float32 CUDA tensor; uint16 bf16 bits -> bfloat16 tensor."""
    import torch
    if W_np.dtype == np.uint16:
        return torch.from_numpy(W_np.view(np.int16).copy()).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(W_np, dtype=np.float32)).cuda()


def as_f32(W_np):
    return wl.bf16_bits_to_f32(W_np) if W_np.dtype == np.uint16 else W_np


def words(mask_t):
    return mask_t.cpu().numpy().view(np.uint32)


def block_counts(mask_words, rows, cols, M):
    """Ones per row and per column of every M x M block: ([bi,bj,M], [bi,bj,M])."""
    Z = oracle.unpack_mask(mask_words, cols).astype(np.int32)
    B = Z.reshape(rows // M, M, cols // M, M).transpose(0, 2, 1, 3)
    return B.sum(3), B.sum(2)


def assert_feasible(mask_words, rows, cols, N, M):
    r, c = block_counts(mask_words, rows, cols, M)
    assert (r == N).all() and (c == N).all(), "infeasible block"
    wpr = (cols + 31) // 32
    if cols % 32:
        tail = mask_words[:, wpr - 1] >> np.uint32(cols % 32)
        assert not tail.any(), "bits beyond the last column"


def sample_block_ids(nblocks, k, seed):
    rng = np.random.default_rng(seed)
    k = min(k, nblocks)
    ids = rng.choice(nblocks, k, replace=False)
    # always include the first and last block (edges of the grid)
    return np.unique(np.concatenate([ids, [0, nblocks - 1]]))


def gather_blocks(X, M, ids, cols):
    nbc = cols // M
    out = np.empty((len(ids), M, M), X.dtype)
    for n, b in enumerate(ids):
        bi, bj = divmod(int(b), nbc)
        out[n] = X[bi * M:(bi + 1) * M, bj * M:(bj + 1) * M]
    return out


S_TOL = 1e-4  # fractional S, max-abs against the fp64 oracle


def assert_S_close(S, S64, tol=S_TOL):
    """GPU S (fp32) within `tol` max-abs of the oracle's fp64 S, shapes equal."""
    S = np.asarray(S, dtype=np.float64)
    S64 = np.asarray(S64, dtype=np.float64)
    assert S.shape == S64.shape, (S.shape, S64.shape)
    err = float(np.abs(S - S64).max()) if S.size else 0.0
    assert err < tol, f"max |S - S64| = {err:.3e} >= {tol:g}"
    return err
