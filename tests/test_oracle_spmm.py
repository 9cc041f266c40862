"""Pins of the oracle's 2:4 compressed operand (the consumer of transposable
masks): the format is defined in include/tsenor.h; these check the oracle's
encoder against a hand-derived word, the decoder round trip on masks the
oracle's own rounding produces, and the transposed encoding."""
import numpy as np

import oracle
from sparse_mask_search_amd import workloads as wl


def _bits(x):
    return wl.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def test_hand_derived_word():
    """One row, k = 32.  Kept positions per group of 4: g0 {1,3}, g1 {0,2},
    g2 {0,1}, g3 {2,3}, g4 {3} (one entry), g5 {} (none), g6 {0,3}, g7 {1,2}.
    Codes (first | second << 2): 0xD, 0x8, 0x4, 0xE, 3 | 2<<2 = 0xB, 0 | 1<<2
    = 0x4, 0xC, 0x9 -> word 0x9C4BE48D.  Values follow in group order."""
    keep = {0: (1, 3), 1: (0, 2), 2: (0, 1), 3: (2, 3), 4: (3,), 5: (), 6: (0, 3), 7: (1, 2)}
    W = np.arange(1, 33, dtype=np.float32)[None, :]
    mask = np.zeros((1, 1), np.uint32)
    for g, ps in keep.items():
        for p in ps:
            mask[0, 0] |= np.uint32(1 << (4 * g + p))
    vals, meta, bad = oracle.compress24(_bits(W), mask)
    assert bad == 0 and meta[0, 0] == 0x9C4BE48D
    expect = []
    for g in range(8):
        ps = list(keep[g]) + [None] * (2 - len(keep[g]))
        expect += [0.0 if p is None else W[0, 4 * g + p] for p in ps]
    got = (vals.astype(np.uint32) << 16).view(np.float32)[0]
    assert np.array_equal(got, np.array(expect, np.float32))


def test_round_trip_on_transposable_masks():
    rng = np.random.default_rng(4)
    rows, cols = 64, 96
    W = _bits(rng.standard_normal((rows, cols)))
    S = rng.random((rows, cols)).astype(np.float32)
    mask, _ = oracle.round_matrix(S, wl.bf16_bits_to_f32(W), 2, 4, 4)
    Z = oracle.unpack_mask(mask, cols)
    dense = wl.bf16_bits_to_f32(W) * Z
    for tr in (False, True):
        vals, meta, bad = oracle.compress24(W, mask, transpose=tr)
        assert bad == 0  # a transposable 2:4 mask is 2:4 along both dimensions
        k = rows if tr else cols
        back = oracle.decompress24(vals, meta, k)
        assert np.array_equal(back, dense.T if tr else dense)


def test_transposed_encoding_equals_encoding_of_the_transpose():
    rng = np.random.default_rng(5)
    W = _bits(rng.standard_normal((32, 64)))
    S = rng.random((32, 64)).astype(np.float32)
    mask, _ = oracle.round_matrix(S, wl.bf16_bits_to_f32(W), 2, 4, 2)
    Z = oracle.unpack_mask(mask, 64)
    ZT = Z.T.astype(np.uint32)
    maskT = np.zeros((64, 1), np.uint32)
    for c in range(32):
        maskT[:, 0] |= ZT[:, c] << np.uint32(c)
    a = oracle.compress24(W, mask, transpose=True)
    b = oracle.compress24(np.ascontiguousarray(W.T), maskT)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_overfull_groups_are_counted():
    W = _bits(np.ones((1, 32)))
    mask = np.array([[0x7]], np.uint32)  # group 0 keeps positions 0, 1, 2
    vals, meta, bad = oracle.compress24(W, mask)
    assert bad == 1 and (meta[0, 0] & 0xF) == (0 | 1 << 2)
