"""The measurement-only memory pass (include/tsenor_bench.h) against numpy:
for every M x M block, bit (2|W| >= block max |W|) of every weight, in the
mask layout; small ragged cases and the full 16:32 workload matrix."""
import numpy as np
import pytest

import sparse_mask_search_amd as sms
from sparse_mask_search_amd import workloads as wl
from gpu_util import as_f32, to_device, words

pytestmark = pytest.mark.gpu


def _expected(Wf, M):
    rows, cols = Wf.shape
    A = np.abs(Wf)
    m = A.reshape(rows // M, M, cols // M, M).max((1, 3))
    mfull = np.repeat(np.repeat(m, M, 0), M, 1)
    Z = (np.float32(2.0) * A >= mfull).astype(np.uint64)
    wpr = (cols + 31) // 32
    Zp = np.zeros((rows, wpr * 32), np.uint64)
    Zp[:, :cols] = Z
    return (Zp.reshape(rows, wpr, 32) << np.arange(32, dtype=np.uint64)).sum(2).astype(np.uint32)


@pytest.mark.parametrize("M", [16, 32])
@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("nbc", [3, 17, 40])  # ragged against the 512- and 256-column strips
def test_memory_pass_small(M, bf16, nbc):
    rng = np.random.default_rng(M * 100 + nbc)
    W = (rng.standard_normal((2 * M, nbc * M)) * rng.lognormal(0, 1, nbc * M)).astype(np.float32)
    W[:M, :M] = 0.0  # an all-zero block: every bit is set (0 >= 0)
    Wn = wl.f32_to_bf16_bits(W) if bf16 else W
    out = sms.memory_pass(to_device(Wn), M)
    import torch
    torch.cuda.synchronize()
    assert np.array_equal(words(out), _expected(as_f32(Wn), M))


def test_memory_pass_headline_matrix():
    name = "16:32-8192x28672-bf16"
    Wn = wl.generate(name)
    out = sms.memory_pass(to_device(Wn), 32)
    import torch
    torch.cuda.synchronize()
    got = words(out)
    Wf = as_f32(Wn)
    for r0 in range(0, Wf.shape[0], 1024):  # bounded host memory
        assert np.array_equal(got[r0:r0 + 1024], _expected(Wf[r0:r0 + 1024], 32)), r0
