"""C-ABI checks that need no GPU: the library loads, exports every entry point
declared in include/tsenor.h, and rejects every invalid argument with its status
code before touching the device (no HIP call is made on these paths)."""
import ctypes
import math
import os
import re
import subprocess

import pytest

import sparse_mask_search_amd as sms

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tsenor.h")
BENCH_HEADER = os.path.join(ROOT, "include", "tsenor_bench.h")
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced on the rejected paths

OK, NULL, SHAPE, NM, PARAM, DTYPE, HIP = range(7)


def declared():
    text = open(HEADER).read() + open(BENCH_HEADER).read()
    return sorted(set(re.findall(r"^(?:int|const char\*)\s+(tsenor_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol():
    names = declared()
    assert names == ["tsenor_bench_memory_pass", "tsenor_compress24", "tsenor_exact",
                     "tsenor_last_error", "tsenor_mask",
                     "tsenor_mask_batched", "tsenor_mask_batched_ex", "tsenor_mask_ex",
                     "tsenor_mask_noalloc", "tsenor_round", "tsenor_spmm24", "tsenor_status_str",
                     "tsenor_version"]
    out = subprocess.check_output(["nm", "-D", "--defined-only", sms.library_path()], text=True)
    exported = set(re.findall(r"\bT (tsenor_\w+)", out))
    for n in names:
        assert n in exported, n
        assert hasattr(sms.lib(), n)


def test_status_strings():
    l = sms.lib()
    for s in range(8):
        assert l.tsenor_status_str(s).decode() != "unknown status"
    assert l.tsenor_status_str(99).decode() == "unknown status"
    assert sms.version() == 0x000100


def _mask(W=FAKE, dtype=1, rows=64, cols=64, ld=64, N=2, M=4, tau=20.0, iters=10, ls=4,
          mask=FAKE, frac=None):
    return sms.lib().tsenor_mask(W, dtype, rows, cols, ld, N, M, tau, iters, ls, mask, frac, None)


@pytest.mark.parametrize("kw,code", [
    (dict(W=None), NULL), (dict(mask=None), NULL),
    (dict(dtype=2), DTYPE), (dict(dtype=-1), DTYPE),
    (dict(M=6, N=3), NM), (dict(M=64, N=8), NM), (dict(N=0), NM), (dict(N=5), NM),
    (dict(rows=0), SHAPE), (dict(cols=-4), SHAPE), (dict(rows=66), SHAPE), (dict(cols=62), SHAPE),
    (dict(ld=60), SHAPE),
    (dict(tau=-1.0), PARAM), (dict(tau=math.inf), PARAM), (dict(tau=math.nan), PARAM),
    (dict(iters=0), PARAM), (dict(ls=-1), PARAM),
])
def test_mask_rejects(kw, code):
    assert _mask(**kw) == code


def _noalloc(W=FAKE, dtype=1, rows=64, cols=64, ld=64, N=2, M=4, tau=20.0, iters=10, ls=4,
             mask=FAKE, frac=None):
    return sms.lib().tsenor_mask_noalloc(W, dtype, rows, cols, ld, N, M, tau, iters, ls, mask,
                                         frac, None)


@pytest.mark.parametrize("kw,code", [
    (dict(W=None), NULL), (dict(mask=None), NULL), (dict(dtype=2), DTYPE),
    (dict(M=6, N=3), NM), (dict(N=0), NM), (dict(rows=66), SHAPE), (dict(ld=60), SHAPE),
    (dict(tau=math.nan), PARAM), (dict(iters=0), PARAM), (dict(ls=-1), PARAM),
])
def test_mask_noalloc_rejects(kw, code):
    """The entry point that allocates nothing validates exactly like
    tsenor_mask, on the host, before any HIP call."""
    assert _noalloc(**kw) == code
    assert _mask(**kw) == code


def test_mask_ex_rejects():
    """The extended entry point validates like tsenor_mask, plus polish_steps."""
    l = sms.lib()
    r = lambda W=FAKE, rows=64, N=2, ls=4, polish=0, prev=None, mask=FAKE: l.tsenor_mask_ex(
        W, 1, rows, 64, 64, N, 4, 20.0, 10, ls, polish, prev, mask, None, None)
    assert r(polish=-1) == PARAM
    assert r(W=None, polish=3) == NULL
    assert r(mask=None, prev=FAKE) == NULL
    assert r(rows=66, polish=2) == SHAPE
    assert r(N=7) == NM
    assert r(ls=-2, prev=FAKE) == PARAM


def test_exact_rejects():
    l = sms.lib()
    r = lambda W=FAKE, rows=64, N=2, M=4, mc=10, mask=FAKE: l.tsenor_exact(
        W, 0, rows, 64, 64, N, M, None, mc, mask, None, None)
    assert r(W=None) == NULL
    assert r(mask=None) == NULL
    assert r(mc=-1) == PARAM
    assert r(rows=63) == SHAPE
    assert r(M=7) == NM


def test_spmm24_rejects():
    l = sms.lib()
    c = lambda W=FAKE, rows=64, cols=64, ld=64, mask=FAKE, tr=0, v=FAKE, m=FAKE: l.tsenor_compress24(
        W, rows, cols, ld, mask, tr, v, m, None, None)
    assert c(W=None) == NULL and c(v=None) == NULL and c(mask=None) == NULL
    assert c(tr=2) == PARAM
    assert c(cols=48, ld=48) == SHAPE          # k = 48 not a multiple of 32
    assert c(rows=48, tr=1) == SHAPE
    assert c(ld=32) == SHAPE
    s = lambda X=FAKE, n=128, ldx=64, v=FAKE, meta=FAKE, m=128, k=64, Y=FAKE, ldy=128: \
        l.tsenor_spmm24(X, n, ldx, v, meta, m, k, Y, ldy, None)
    assert s(X=None) == NULL and s(Y=None) == NULL
    assert s(n=96) == SHAPE and s(m=64) == SHAPE and s(k=48, ldx=48) == SHAPE
    assert s(ldx=60, k=32) == SHAPE and s(ldy=100) == SHAPE
    assert s(X=ctypes.c_void_p(0x1008)) == SHAPE  # misaligned


def test_round_rejects():
    l = sms.lib()
    r = lambda S=FAKE, lds=64, W=FAKE, dt=0, rows=64, cols=64, ld=64, N=2, M=4, ls=2, mask=FAKE: \
        l.tsenor_round(S, lds, W, dt, rows, cols, ld, N, M, ls, mask, None)
    assert r(S=None) == NULL
    assert r(W=None) == NULL
    assert r(mask=None) == NULL
    assert r(lds=32) == SHAPE
    assert r(ls=-3) == PARAM
    assert r(M=12) == NM
    assert r(dt=7) == DTYPE


def test_batched_rejects():
    l = sms.lib()
    M = sms._lib._Matrix
    good = M(0x1000, 1, 64, 64, 64, 8, 16, 0x1000, 0)
    bad = M(0x1000, 1, 64, 60, 64, 8, 16, 0x1000, 0)
    arr = (M * 2)(good, bad)
    assert l.tsenor_mask_batched(arr, 2, 20.0, 5, 2, None) == SHAPE
    assert l.tsenor_mask_batched(arr, -1, 20.0, 5, 2, None) == PARAM
    assert l.tsenor_mask_batched(None, 3, 20.0, 5, 2, None) == NULL
    assert l.tsenor_mask_batched(arr, 1, -2.0, 5, 2, None) == PARAM
    assert l.tsenor_mask_batched(arr, 1, 20.0, 0, 2, None) == PARAM
    assert l.tsenor_mask_batched(None, 0, 20.0, 5, 2, None) == OK  # empty batch: no-op
    # the extended form validates the same way, plus polish_steps
    assert l.tsenor_mask_batched_ex(arr, 2, 20.0, 5, 2, 0, None, None) == SHAPE
    assert l.tsenor_mask_batched_ex(arr, 1, 20.0, 5, 2, -1, None, None) == PARAM
    assert l.tsenor_mask_batched_ex(None, 3, 20.0, 5, 2, 4, None, None) == NULL
    assert l.tsenor_mask_batched_ex(None, 0, 20.0, 5, 2, 4, None, None) == OK


def test_binding_requires_device_tensors():
    torch = pytest.importorskip("torch")
    with pytest.raises(TypeError):
        sms.mask(torch.zeros(8, 8), 2, 4, 20.0, 5, 2)


def test_memory_pass_rejects():
    """The measurement-only memory pass validates on the host before any HIP call."""
    l = sms.lib()
    r = lambda W=FAKE, dt=1, rows=64, cols=64, ld=64, M=32, mask=FAKE: l.tsenor_bench_memory_pass(
        W, dt, rows, cols, ld, M, mask, None)
    assert r(W=None) == NULL and r(mask=None) == NULL
    assert r(dt=3) == DTYPE
    assert r(M=8) == NM and r(M=4) == NM
    assert r(rows=48) == SHAPE and r(ld=60) == SHAPE and r(ld=68) == SHAPE  # 68*2 % 16 != 0
    assert r(W=ctypes.c_void_p(0x1002)) == SHAPE  # 16-byte alignment
