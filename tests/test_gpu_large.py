"""A matrix of more than 2^31 elements: every offset into W, S and the mask
is 64-bit.  The block-rows just below and just above element 2^31 and the
last block-row are compared with the oracle in full (S within 1e-4 of the
fp64 oracle, masks equal to the oracle's rounding of the GPU's S), and every
block of the matrix is checked feasible on the GPU."""
import numpy as np
import pytest

import oracle
import sparse_mask_search_amd as sms
from sparse_mask_search_amd import workloads as wl
from gpu_util import assert_S_close, assert_feasible

pytestmark = pytest.mark.gpu

ROWS, COLS = 67584, 32768          # 2,214,592,512 elements, > 2^31
N, M, TAU, ITERS, LS = 16, 32, 40.0, 30, 8


def _block_counts_ok(torch, mask_t, rows, cols, N, M, chunk_rows=8192):
    """Every M x M block has N ones per row and per column (on the GPU)."""
    bits = torch.arange(32, device=mask_t.device, dtype=torch.int32)
    for r0 in range(0, rows, chunk_rows):
        w = mask_t[r0:r0 + chunk_rows]
        Z = ((w.unsqueeze(-1) >> bits) & 1).reshape(w.shape[0], -1)[:, :cols].to(torch.int16)
        B = Z.reshape(-1, M, cols // M, M)
        if not (bool((B.sum(3) == N).all()) and bool((B.sum(1) == N).all())):
            return False
    return True


def test_beyond_2_31_elements():
    torch = pytest.importorskip("torch")
    assert ROWS * COLS > 2**31 and ROWS % M == 0 and COLS % M == 0
    print(f"[large] {ROWS}x{COLS} bf16 {N}:{M}, tau {TAU}, T {ITERS}, L {LS}", flush=True)
    g = torch.Generator(device="cuda").manual_seed(31)
    W = torch.empty((ROWS, COLS), dtype=torch.bfloat16, device="cuda")
    for r0 in range(0, ROWS, 8192):  # seeded, generated in slices to bound the fp32 temporary
        n = min(8192, ROWS - r0)
        W[r0:r0 + n] = (torch.randn((n, COLS), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    mask_t, S_t = sms.mask(W, N, M, TAU, ITERS, LS, return_frac=True)
    torch.cuda.synchronize()
    assert _block_counts_ok(torch, mask_t, ROWS, COLS, N, M)
    first_above = (2**31 // COLS) // M          # block-row starting at element 2^31
    for br in (first_above - 1, first_above, ROWS // M - 1):
        r0 = br * M
        Wb = W[r0:r0 + M].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        Wf = wl.bf16_bits_to_f32(Wb)
        S = S_t[r0:r0 + M].cpu().numpy()
        mw = mask_t[r0:r0 + M].cpu().numpy().view(np.uint32)
        assert_feasible(mw, M, COLS, N, M)
        ref, _ = oracle.round_matrix(S, Wf, N, M, LS)
        assert np.array_equal(mw, ref), f"block-row {br}"
        S64, _ = oracle.dykstra(Wf, N, M, TAU, ITERS)
        err = assert_S_close(S, S64)
        print(f"[large] block-row {br} (elements from {r0 * COLS}): max|S-S64| {err:.3e}",
              flush=True)
