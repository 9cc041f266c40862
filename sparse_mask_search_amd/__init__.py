"""MI355X-native transposable N:M mask search (TSENOR-style).

Thin Python binding over the C ABI of ``libtsenor.so`` (include/tsenor.h):
argument marshalling only -- every step of the method runs in the library's
HIP kernels.  PyTorch provides device memory and the current stream.

    import torch, sparse_mask_search_amd as sms
    W = torch.randn(4096, 4096, device="cuda", dtype=torch.bfloat16)
    mask, S = sms.mask(W, N=8, M=16, tau=30.0, iters=150, ls_steps=16, return_frac=True)
    keep = sms.unpack(mask, W.shape[1])          # bool [rows, cols]

Method: pith.science review of "TSENOR: Highly-Efficient Algorithm for Finding
Transposable N:M Sparse Masks" (arXiv 2505.23949), "What carries the argument".
"""
from __future__ import annotations

from ._lib import (F32, BF16, TsenorError, compress24, exact, lib, library_path, mask,
                   mask_batched, mask_noalloc, memory_pass, round_mask, spmm24, unpack, version)

__all__ = ["F32", "BF16", "TsenorError", "compress24", "exact", "lib", "library_path", "mask",
           "mask_batched", "mask_noalloc", "memory_pass", "round_mask", "spmm24", "unpack",
           "version"]
