"""Calls of tsenor_mask on several streams at once.

tsenor_mask uses no buffer shared between calls (the kernels need no
workspace), so it does not order its launch after the device's other calls,
and calls on different streams may run at the same time.  This test
interleaves calls on two streams (different matrices, M and dtypes, separate
outputs), together with ordered calls (a previous mask that is the output
itself, which goes through the library's cached copy), and checks every result
bit for bit against the same call made alone on the default stream.
"""
import numpy as np
import pytest

import sparse_mask_search_amd as sms
from sparse_mask_search_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _matrix(seed, rows, cols, bf16):
    import torch
    W = (0.02 * np.random.default_rng(seed).standard_t(4, (rows, cols))).astype(np.float32)
    if bf16:
        return torch.from_numpy(wl.f32_to_bf16_bits(W).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(W).cuda()


def test_concurrent_streams_equal_single_stream():
    import torch
    cases = [  # (seed, rows, cols, bf16, N, M, tau, iters, ls)
        (1, 512, 2048, True, 16, 32, 40.0, 60, 32),
        (2, 256, 4096, False, 8, 16, 30.0, 50, 16),
        (3, 1024, 1024, False, 2, 4, 20.0, 50, 4),
        (4, 512, 1024, True, 4, 8, 20.0, 40, 8),
    ]
    mats = [_matrix(c[0], c[1], c[2], c[3]) for c in cases]
    ref = []
    for W, c in zip(mats, cases):
        m, _ = sms.mask(W, *c[4:])
        ref.append(m.clone())
    torch.cuda.synchronize()

    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [[torch.empty_like(r) for r in ref] for _ in range(3)]
    prev = [r.clone() for r in ref]  # ordered calls: previous mask == output
    for rep in range(3):
        for k, (W, c) in enumerate(zip(mats, cases)):
            s = streams[(k + rep) % 2]
            with torch.cuda.stream(s):
                sms.mask(W, *c[4:], out=outs[rep][k], stream=s)
                if rep == 1:
                    sms.mask(W, *c[4:], out=prev[k], prev_mask=prev[k], stream=s)
    torch.cuda.synchronize()
    for rep in range(3):
        for k in range(len(cases)):
            assert torch.equal(outs[rep][k], ref[k]), (rep, cases[k])
    # the previous mask is the method's own mask: kept where it is no worse, so
    # the result equals it
    for k in range(len(cases)):
        assert torch.equal(prev[k], ref[k]), cases[k]
