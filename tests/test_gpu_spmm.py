"""GPU: the 2:4 consumer of transposable masks.  The compressed operand is
bit-exact with the oracle's encoder for W and W^T under a 2:4 mask from the
library's own search; Y = X A^T on the sparse matrix cores matches the fp64
product with the masked weights for the forward (A = W) and data-gradient
(A = W^T) products, within fp32 accumulation error."""
import numpy as np
import pytest

import oracle
import sparse_mask_search_amd as sms
from sparse_mask_search_amd import workloads as wl
from gpu_util import to_device, words

pytestmark = pytest.mark.gpu


def _case(seed, rows, cols):
    import torch
    rng = np.random.default_rng(seed)
    Wb = wl.f32_to_bf16_bits((0.05 * rng.standard_normal((rows, cols))).astype(np.float32))
    W = to_device(Wb)
    m, _ = sms.mask(W, 2, 4, 20.0, 50, 4)
    torch.cuda.synchronize()
    return Wb, W, m


@pytest.mark.parametrize("rows,cols", [(128, 256), (384, 128)])
def test_compress_matches_oracle(rows, cols):
    import torch
    print(f"[case] compress {rows}x{cols}", flush=True)
    Wb, W, m = _case(rows + cols, rows, cols)
    for tr in (False, True):
        vals, meta, bad = sms.compress24(W, m, transpose=tr)
        torch.cuda.synchronize()
        v0, m0, b0 = oracle.compress24(Wb, words(m), transpose=tr)
        assert int(bad.item()) == b0 == 0
        assert np.array_equal(vals.cpu().view(torch.int16).numpy().view(np.uint16), v0)
        assert np.array_equal(meta.cpu().numpy().view(np.uint32), m0)


def test_overfull_groups_counted_on_gpu():
    import torch
    rng = np.random.default_rng(3)
    Wb = wl.f32_to_bf16_bits(rng.standard_normal((32, 64)).astype(np.float32))
    W = to_device(Wb)
    mw = rng.integers(0, 2 ** 32, (32, 2), dtype=np.uint64).astype(np.uint32)
    mt = torch.from_numpy(mw.view(np.int32)).cuda()
    vals, meta, bad = sms.compress24(W, mt)
    torch.cuda.synchronize()
    v0, m0, b0 = oracle.compress24(Wb, mw)
    assert int(bad.item()) == b0 > 0
    assert np.array_equal(meta.cpu().numpy().view(np.uint32), m0)


# The last two shapes give tile grids (m-tiles x n-tiles) whose workgroups are
# spread over the 8 XCDs in groups of up to 8 m-tiles: 10 x 4 tiles of 256 and
# 9 x 8 tiles of 128 in the forward product (ragged last groups), 1 x 8 tiles
# of 128 in both data-gradient products.
@pytest.mark.parametrize("n,rows,cols", [(128, 256, 384), (256, 512, 256), (512, 768, 1408),
                                         (1024, 2560, 128), (1024, 1152, 128)])
def test_forward_and_data_gradient(n, rows, cols):
    import torch
    print(f"[case] spmm n={n} W {rows}x{cols}", flush=True)
    Wb, W, m = _case(7 * n + rows, rows, cols)
    rng = np.random.default_rng(n)
    Z = oracle.unpack_mask(words(m), cols)
    Wd = wl.bf16_bits_to_f32(Wb).astype(np.float64) * Z
    Xb = wl.f32_to_bf16_bits(rng.standard_normal((n, cols)).astype(np.float32))
    Gb = wl.f32_to_bf16_bits(rng.standard_normal((n, rows)).astype(np.float32))
    X, G = to_device(Xb), to_device(Gb)
    Xd, Gd = wl.bf16_bits_to_f32(Xb).astype(np.float64), wl.bf16_bits_to_f32(Gb).astype(np.float64)
    vf, mf, _ = sms.compress24(W, m)                 # A = W    [rows, cols]
    vb, mb, _ = sms.compress24(W, m, transpose=True)  # A = W^T  [cols, rows]
    Y = sms.spmm24(X, vf, mf)     # Y  = X  W^T  [n, rows]
    dX = sms.spmm24(G, vb, mb)    # dX = dY W    [n, cols]
    torch.cuda.synchronize()
    for got, ref, bound in ((Y, Xd @ Wd.T, np.abs(Xd) @ np.abs(Wd).T),
                            (dX, Gd @ Wd, np.abs(Gd) @ np.abs(Wd))):
        err = np.abs(got.cpu().numpy() - ref)
        assert (err <= 1e-5 * bound + 1e-30).all(), err.max()


@pytest.mark.parametrize("cols", [64, 128, 192, 320, 384])
def test_forward_k_step_counts(cols):
    """m, n multiples of 256 (the LDS-ring kernel) with 1, 2, 3, 5 and 6
    k-steps of 64: every position of the three-buffer ring at the end of the
    loop, and rings shorter than the prefetch distance."""
    import torch
    n, rows = 256, 512
    print(f"[case] spmm k-steps n={n} W {rows}x{cols}", flush=True)
    Wb, W, m = _case(11 + cols, rows, cols)
    rng = np.random.default_rng(12)
    Z = oracle.unpack_mask(words(m), cols)
    Wd = wl.bf16_bits_to_f32(Wb).astype(np.float64) * Z
    Xb = wl.f32_to_bf16_bits(rng.standard_normal((n, cols)).astype(np.float32))
    Xd = wl.bf16_bits_to_f32(Xb).astype(np.float64)
    vf, mf, _ = sms.compress24(W, m)
    Y = sms.spmm24(to_device(Xb), vf, mf)
    torch.cuda.synchronize()
    err = np.abs(Y.cpu().numpy() - Xd @ Wd.T)
    assert (err <= 1e-5 * (np.abs(Xd) @ np.abs(Wd).T) + 1e-30).all(), err.max()
