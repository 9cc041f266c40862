"""GPU parity: the HIP path against the oracle on the same seeded inputs.

Bars (the method as in the pith.science review of TSENOR, "What carries the
argument"; tolerances from the design): fractional S within 1e-4 max-abs of the
fp64 oracle; masks bit-exact with the oracle's rounding applied to the GPU's S,
and with the GPU's own rounding-only entry point on that S; every block
feasible (N ones per row and column).  Small cases span several groups, a
ragged last group and a partial last mask word; the workload-sized cases check
every block (the 2-opt polish at 16:32: whole sampled block-rows) at full size,
in the launch configuration the benchmark times.
"""
import os

import numpy as np
import pytest

import oracle
import sparse_mask_search_amd as sms
from sparse_mask_search_amd import workloads as wl
from gpu_util import (as_f32, assert_S_close, assert_feasible, gather_blocks, sample_block_ids,
                      to_device, words)

pytestmark = pytest.mark.gpu
S_TOL = 1e-4


def _note(*a):
    print("[case]", *a, flush=True)


def _run(W_np, N, M, tau, iters, ls):
    import torch
    W = to_device(W_np)
    mask, S = sms.mask(W, N, M, tau, iters, ls, return_frac=True)
    mask2 = sms.round_mask(S, W, N, M, ls)
    torch.cuda.synchronize()
    return W, words(mask), S.cpu().numpy(), words(mask2)


def _small(seed, M, nbc, nbr, kind, bf16):
    rng = np.random.default_rng(seed)
    W = wl.random_blocks(seed, nbc, M, kind)
    W = np.concatenate([W] + [wl.random_blocks(seed * 7 + r, nbc, M, kind) for r in range(1, nbr)])
    if kind != "zero":
        W[:M, :M] = 0.0  # one all-zero block
    W = W.astype(np.float32)
    return wl.f32_to_bf16_bits(W) if bf16 else W


SMALL = [  # M, blocks per row (ragged vs the group width), block rows
    (4, 70, 3), (8, 67, 2), (16, 37, 3), (32, 19, 2),
]


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("kind", ["student_t", "outlier", "ties"])
@pytest.mark.parametrize("M,nbc,nbr", SMALL)
def test_small_parity(M, nbc, nbr, kind, bf16):
    N = M // 2
    tau, iters, ls = (20.0, 60, M)
    W_np = _small(100 + M, M, nbc, nbr, kind, bf16)
    rows, cols = W_np.shape
    _note(f"small M={M} {rows}x{cols} {kind} bf16={bf16}")
    _, mask, S, mask2 = _run(W_np, N, M, tau, iters, ls)
    Wf = as_f32(W_np)
    S64, _ = oracle.dykstra(Wf, N, M, tau, iters)
    assert np.abs(S - S64).max() < S_TOL
    ref, _ = oracle.round_matrix(S, Wf, N, M, ls)
    assert np.array_equal(mask, ref)
    assert np.array_equal(mask2, ref)
    assert_feasible(mask, rows, cols, N, M)


@pytest.mark.parametrize("tau", [120.0, 300.0])
@pytest.mark.parametrize("M,nbc,nbr", SMALL)
def test_large_tau(M, nbc, nbr, tau):
    """Kernels whose log2 range exceeds fp32's (tau * log2(e) well past 126):
    the rescaling must then happen in log2 space or entries that underflow
    are lost; S stays within the contract and masks exact."""
    N = M // 2
    iters, ls = 150, M
    W_np = _small(300 + M, M, nbc, nbr, "outlier", M >= 16)
    rows, cols = W_np.shape
    _note(f"large tau={tau} M={M} {rows}x{cols}")
    _, mask, S, mask2 = _run(W_np, N, M, tau, iters, ls)
    Wf = as_f32(W_np)
    S64, _ = oracle.dykstra(Wf, N, M, tau, iters)
    err = np.abs(S - S64).max()
    print(f"tau {tau} M {M}: max|S-S64| = {err:.3e}", flush=True)
    assert err < S_TOL
    ref, _ = oracle.round_matrix(S, Wf, N, M, ls)
    assert np.array_equal(mask, ref) and np.array_equal(mask2, ref)
    assert_feasible(mask, rows, cols, N, M)


@pytest.mark.parametrize("iters", [1, 3])
@pytest.mark.parametrize("kind", ["student_t", "ties"])
@pytest.mark.parametrize("M,nbc,nbr", SMALL)
def test_local_search_heavy(M, nbc, nbr, kind, iters):
    """One or three Dykstra cycles leave S far from a transport plan: the
    greedy falls short in most blocks and the local search makes many moves,
    over tied scores too (the 'ties' weights take three magnitudes), so every
    stage of its lexicographic tie-break decides some moves."""
    N = M // 2
    ls = M * M
    W_np = _small(500 + M, M, nbc, nbr, kind, M >= 16)
    rows, cols = W_np.shape
    _note(f"heavy LS M={M} {rows}x{cols} {kind} iters={iters}")
    _, mask, S, mask2 = _run(W_np, N, M, 20.0, iters, ls)
    ref, stats = oracle.round_matrix(S, as_f32(W_np), N, M, ls)
    print(f"M={M} {kind} T={iters}: shortfall blocks {stats[0]}, R2 moves {stats[2]}, "
          f"R3 moves {stats[3]}", flush=True)
    assert stats[2] > 0
    assert np.array_equal(mask, ref) and np.array_equal(mask2, ref)
    assert_feasible(mask, rows, cols, N, M)


@pytest.mark.parametrize("ls", [1, 7, 1024])
@pytest.mark.parametrize("M", [4, 8, 16, 32])
def test_round_tied_scores(M, ls):
    """Rounding alone on S with four levels and |W| with three: ties in the
    sort order and in the swap scores everywhere; the move limit cuts the
    search early (1, 7) or never (1024)."""
    import torch
    rng = np.random.default_rng(900 + M + ls)
    N = M // 2
    nbc, nbr = 41, 2
    W_np = np.concatenate([wl.random_blocks(900 + M + r, nbc, M, "ties") for r in range(nbr)])
    S_np = (rng.integers(0, 4, W_np.shape) / 4.0).astype(np.float32)
    rows, cols = W_np.shape
    _note(f"tied round M={M} {rows}x{cols} ls={ls}")
    got = sms.round_mask(to_device(S_np), to_device(W_np), N, M, ls)
    torch.cuda.synchronize()
    ref, stats = oracle.round_matrix(S_np, W_np, N, M, ls)
    print(f"M={M} ls={ls}: R2 moves {stats[2]}, R3 moves {stats[3]}", flush=True)
    assert stats[2] > 0
    assert np.array_equal(words(got), ref)
    assert_feasible(words(got), rows, cols, N, M)


@pytest.mark.parametrize("M,N", [(4, 1), (8, 3), (16, 5), (32, 7), (32, 31), (16, 16)])
def test_other_n(M, N):
    W_np = _small(7 + N, M, 11, 2, "student_t", True)
    rows, cols = W_np.shape
    _note(f"N={N} M={M} {rows}x{cols}")
    _, mask, S, mask2 = _run(W_np, N, M, 15.0, 40, 5)
    Wf = as_f32(W_np)
    S64, _ = oracle.dykstra(Wf, N, M, 15.0, 40)
    assert np.abs(S - S64).max() < S_TOL
    ref, _ = oracle.round_matrix(S, Wf, N, M, 5)
    assert np.array_equal(mask, ref) and np.array_equal(mask2, ref)
    assert_feasible(mask, rows, cols, N, M)


@pytest.mark.parametrize("k", [-20, 9])
@pytest.mark.parametrize("M,bf16", [(8, False), (32, True)])
def test_power_of_two_scale_invariance(M, bf16, k):
    """W and W * 2^k: the block-max normalisation removes the factor exactly
    and the local-search scores scale exactly, so S and the mask are
    bit-identical (the oracle's own pin of the method, here on the GPU)."""
    import torch
    N = M // 2
    W_np = _small(600 + M, M, 13, 2, "student_t", False).astype(np.float32)
    W2_np = np.ldexp(W_np, k).astype(np.float32)
    if bf16:
        W_np, W2_np = wl.f32_to_bf16_bits(W_np), wl.f32_to_bf16_bits(W2_np)
    _note(f"scale 2^{k} M={M} bf16={bf16}")
    _, m1, S1, _ = _run(W_np, N, M, 30.0, 60, M)
    _, m2, S2, _ = _run(W2_np, N, M, 30.0, 60, M)
    assert np.array_equal(m1, m2)
    assert np.array_equal(S1, S2)


# cases per seed of the random tests (TSENOR_RANDOM_CASES raises it for a long sweep)
RANDOM_CASES = int(os.environ.get("TSENOR_RANDOM_CASES", "40"))


@pytest.mark.parametrize("seed", [11, 12, 13])
def test_random_configurations(seed):
    """Seeded random mixes of M, N (1..M), value distribution, tau (0..150),
    cycles (1..80), local-search steps (0..64) and dtype: S within the
    contract of the fp64 oracle, masks bit-exact with the oracle's rounding of
    the GPU's S, for the fused path and the rounding-only entry point."""
    import torch
    rng = np.random.default_rng(seed)
    for case in range(RANDOM_CASES):
        M = int(rng.choice([4, 8, 16, 32]))
        N = int(rng.integers(1, M + 1))
        nbc, nbr = int(rng.integers(1, 12)), int(rng.integers(1, 3))
        kind = str(rng.choice(["normal", "outlier", "student_t", "ties", "uniform"]))
        tau = float(rng.choice([0.0, 5.0, 20.0, 60.0, 150.0]))
        T = int(rng.choice([1, 2, 5, 20, 80]))
        L = int(rng.choice([0, 1, 3, 8, 64]))
        bf16 = bool(rng.integers(0, 2))
        W = np.concatenate([wl.random_blocks(seed * 10000 + 100 * case + r, nbc, M, kind)
                            for r in range(nbr)]).astype(np.float32)
        Wn = wl.f32_to_bf16_bits(W) if bf16 else W
        _note(f"random seed={seed} case={case}: M={M} N={N} {W.shape} {kind} tau={tau} "
              f"T={T} L={L} bf16={bf16}")
        _, mask, S, mask2 = _run(Wn, N, M, tau, T, L)
        Wf = as_f32(Wn)
        S64, _ = oracle.dykstra(Wf, N, M, tau, T)
        assert np.abs(S - S64).max() < S_TOL
        ref, _ = oracle.round_matrix(S, Wf, N, M, L)
        assert np.array_equal(mask, ref) and np.array_equal(mask2, ref)
        assert_feasible(mask, *W.shape, N, M)


@pytest.mark.parametrize("seed", [21, 22, 23])
def test_random_configurations_optional_stages(seed):
    """The random mixes above with the optional stages: 0..50 polish swaps and,
    in a third of the cases, a previous mask (a shorter solve of the same W,
    polished): masks bit-exact with the oracle's rounding with the same stages
    of the GPU's S, every block feasible."""
    import torch
    rng = np.random.default_rng(seed)
    for case in range(RANDOM_CASES):
        M = int(rng.choice([4, 8, 16, 32]))
        N = int(rng.integers(1, M + 1))
        nbc, nbr = int(rng.integers(1, 12)), int(rng.integers(1, 3))
        kind = str(rng.choice(["normal", "outlier", "student_t", "ties", "uniform"]))
        tau = float(rng.choice([0.0, 5.0, 20.0, 60.0, 150.0]))
        T = int(rng.choice([1, 2, 5, 20, 80]))
        L = int(rng.choice([0, 1, 3, 8, 64]))
        bf16 = bool(rng.integers(0, 2))
        K = int(rng.choice([0, 1, 4, 50]))
        use_prev = bool(rng.integers(0, 3) == 0)
        W = np.concatenate([wl.random_blocks(seed * 10000 + 100 * case + r, nbc, M, kind)
                            for r in range(nbr)]).astype(np.float32)
        Wn = wl.f32_to_bf16_bits(W) if bf16 else W
        _note(f"random stages seed={seed} case={case}: M={M} N={N} {W.shape} {kind} "
              f"tau={tau} T={T} L={L} bf16={bf16} K={K} prev={use_prev}")
        Wd = to_device(Wn)
        prev = None
        if use_prev:
            prev = sms.mask(Wd, N, M, tau, max(1, T // 2), L, polish_steps=3)[0].clone()
        m_t, S_t = sms.mask(Wd, N, M, tau, T, L, return_frac=True, polish_steps=K,
                            prev_mask=prev)
        torch.cuda.synchronize()
        S = S_t.cpu().numpy()
        mask = words(m_t)
        Wf = as_f32(Wn)
        ref, _ = oracle.round_matrix_ex(S, Wf, N, M, L, K,
                                        words(prev) if prev is not None else None)
        assert np.array_equal(mask, ref)
        assert_feasible(mask, *W.shape, N, M)


@pytest.mark.parametrize("M", [4, 8, 16, 32])
def test_closed_forms(M):
    """tau = 0: S = N/M everywhere and the mask is the block diagonal of N x N
    tiles; one iteration and no local search also match the oracle."""
    N = M // 2
    W_np = _small(3, M, 9, 2, "normal", False)
    rows, cols = W_np.shape
    _note(f"tau=0 M={M}")
    _, mask, S, _ = _run(W_np, N, M, 0.0, 7, 3)
    assert np.allclose(S, N / M, rtol=2e-6, atol=0)
    diag = np.zeros((M, M), bool)
    for k in range(M // N):
        diag[k * N:(k + 1) * N, k * N:(k + 1) * N] = True
    Z = oracle.unpack_mask(mask, cols)
    for bi in range(rows // M):
        for bj in range(cols // M):
            assert np.array_equal(Z[bi * M:(bi + 1) * M, bj * M:(bj + 1) * M], diag)
    _note(f"iters=1 ls=0 M={M}")
    _, mask, S, mask2 = _run(W_np, N, M, 25.0, 1, 0)
    S64, _ = oracle.dykstra(W_np, N, M, 25.0, 1)
    assert np.abs(S - S64).max() < S_TOL
    ref, _ = oracle.round_matrix(S, W_np, N, M, 0)
    assert np.array_equal(mask, ref) and np.array_equal(mask2, ref)


def test_strided_and_unaligned_rows():
    """ld > cols and an odd ld (scalar-load path) give the same result as the
    packed matrix."""
    import torch
    M, N = 16, 8
    W_np = _small(5, M, 9, 2, "student_t", True)
    rows, cols = W_np.shape
    for extra in (16, 3):
        _note(f"ld=cols+{extra}")
        big = np.zeros((rows, cols + extra), np.uint16)
        big[:, :cols] = W_np
        Wb = to_device(big)[:, :cols]
        m1, s1 = sms.mask(Wb, N, M, 20.0, 30, 8, return_frac=True)
        m0, s0 = sms.mask(to_device(W_np), N, M, 20.0, 30, 8, return_frac=True)
        torch.cuda.synchronize()
        assert torch.equal(m1, m0) and torch.equal(s1, s0)


def test_deterministic_and_frac_independent():
    import torch
    M, N = 32, 16
    W = to_device(_small(9, M, 19, 2, "outlier", True))
    _note("determinism")
    a, sa = sms.mask(W, N, M, 40.0, 50, 32, return_frac=True)
    b, _ = sms.mask(W, N, M, 40.0, 50, 32)
    c, sc = sms.mask(W, N, M, 40.0, 50, 32, return_frac=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(a, c) and torch.equal(sa, sc)


# ---------------------------------------------------------------- workloads

def _workload(name):
    w = wl.WORKLOADS[name]
    W_np = wl.generate(name)
    return w, W_np, as_f32(W_np)


def test_workload_2_4_full():
    """2:4 on 1024x1024 fp32: every block against the oracle, plus each
    block's brute-force optimum over the 90 feasible masks (gap reported)."""
    w, W_np, Wf = _workload("2:4-1024x1024-f32")
    _note(w.name)
    _, mask, S, mask2 = _run(W_np, w.N, w.M, w.tau, w.iters, w.ls_steps)
    S64, _ = oracle.dykstra(Wf, w.N, w.M, w.tau, w.iters)
    assert np.abs(S - S64).max() < S_TOL
    ref, _ = oracle.round_matrix(S, Wf, w.N, w.M, w.ls_steps)
    assert np.array_equal(mask, ref) and np.array_equal(mask2, ref)
    assert_feasible(mask, w.rows, w.cols, w.N, w.M)
    masks = oracle.feasible_masks(4, 2).astype(np.float64)
    A = oracle.block_view(np.abs(Wf.astype(np.float64)), 4).reshape(-1, 4, 4)
    Z = oracle.block_view(oracle.unpack_mask(mask, w.cols).astype(np.float64), 4).reshape(-1, 4, 4)
    opt = np.einsum("kij,bij->bk", masks, A).max(1)
    got = (Z * A).sum((1, 2))
    assert (got <= opt + 1e-9).all()
    gap = (opt - got) / np.where(opt > 0, opt, 1)
    print(f"2:4 gap vs brute force: mean {gap.mean():.4%} max {gap.max():.4%} "
          f"optimal {np.mean(gap < 1e-12):.2%}", flush=True)


@pytest.mark.parametrize("name", [
    "4:8-4096x4096-f32",
    "8:16-4096x11008-bf16",
    "16:32-8192x28672-bf16",
    "16:32-8192x28672-bf16-tau200",
])
def test_workload_every_block(name):
    """The full workload in the benchmark's launch configuration (one
    tsenor_mask call): S of every block within 1e-4 of the fp64 oracle, the
    mask of every block equal to the oracle's rounding of the GPU's S and to
    the GPU's rounding-only entry point, every block feasible."""
    import torch
    w, W_np, Wf = _workload(name)
    _note(w.name, "every block")
    W = to_device(W_np)
    mask_t, S_t = sms.mask(W, w.N, w.M, w.tau, w.iters, w.ls_steps, return_frac=True)
    mask2_t = sms.round_mask(S_t, W, w.N, w.M, w.ls_steps)
    torch.cuda.synchronize()
    mask = words(mask_t)
    assert np.array_equal(mask, words(mask2_t))
    assert_feasible(mask, w.rows, w.cols, w.N, w.M)
    S = S_t.cpu().numpy()
    del W, mask_t, S_t, mask2_t
    torch.cuda.empty_cache()
    ref, stats = oracle.round_matrix(S, Wf, w.N, w.M, w.ls_steps)
    assert np.array_equal(mask, ref)
    S64, _ = oracle.dykstra(Wf, w.N, w.M, w.tau, w.iters)
    err = assert_S_close(S, S64)
    print(f"{w.name}: max|S-S64| over all {w.blocks} blocks = {err:.3e}; blocks with a "
          f"shortfall {stats[0]}, local-search moves {stats[2]}, fill moves {stats[3]}",
          flush=True)


@pytest.mark.parametrize("name,block_rows", [
    ("8:16-4096x11008-bf16", None),          # every block
    ("16:32-8192x28672-bf16", (0, 1, 97, 128, 200, 255)),
])
def test_workload_polish(name, block_rows):
    """The optional 2-opt polish (8 swaps per block) at workload size, in the
    launch the benchmark's --polish-steps 8 line times: masks equal to the
    oracle's rounding with the same polish of the GPU's S (on every block, or
    on the listed block-rows), every block feasible."""
    import torch
    w, W_np, Wf = _workload(name)
    K = 8
    _note(w.name, f"polish {K}", "every block" if block_rows is None else f"block-rows {block_rows}")
    W = to_device(W_np)
    mask_t, S_t = sms.mask(W, w.N, w.M, w.tau, w.iters, w.ls_steps, return_frac=True,
                           polish_steps=K)
    torch.cuda.synchronize()
    mask = words(mask_t)
    assert_feasible(mask, w.rows, w.cols, w.N, w.M)
    rows = range(w.rows // w.M) if block_rows is None else block_rows
    swaps = 0
    for br in ([None] if block_rows is None else rows):
        sl = slice(None) if br is None else slice(br * w.M, (br + 1) * w.M)
        S = S_t[sl].cpu().numpy()
        ref, st = oracle.round_matrix_ex(S, np.ascontiguousarray(Wf[sl]), w.N, w.M, w.ls_steps, K)
        assert np.array_equal(mask[sl], ref), f"block-row {br}"
        swaps += int(st[4])
    assert swaps > 0
    print(f"{w.name} polish {K}: masks equal to the oracle's, {swaps} swaps", flush=True)


def test_model7b_layer_batched():
    """One batched call over a 7B-shaped layer (8:16 attention, 16:32 MLP)
    equals per-matrix calls bit for bit; for every projection, every block's
    mask equals the oracle's rounding of the GPU's S and every block's S is
    within 1e-4 of the fp64 oracle."""
    import torch
    mats = list(wl.model7b_layer(0))
    _note("7B layer 0 batched")
    Ws = [to_device(b) for (_, _, _, b) in mats]
    outs = sms.mask_batched([(W, N, M) for W, (_, N, M, _) in zip(Ws, mats)], wl.MODEL7B_TAU,
                            wl.MODEL7B_ITERS, wl.MODEL7B_LS, return_frac=True)
    torch.cuda.synchronize()
    for W, (nm, N, M, bits), (m, f) in zip(Ws, mats, outs):
        m1, f1 = sms.mask(W, N, M, wl.MODEL7B_TAU, wl.MODEL7B_ITERS, wl.MODEL7B_LS,
                          return_frac=True)
        torch.cuda.synchronize()
        assert torch.equal(m, m1) and torch.equal(f, f1), nm
        rows, cols = W.shape
        mw = words(m)
        assert_feasible(mw, rows, cols, N, M)
        Wf = as_f32(bits)
        S = f.cpu().numpy()
        ref, _ = oracle.round_matrix(S, Wf, N, M, wl.MODEL7B_LS)
        assert np.array_equal(mw, ref), nm
        S64, _ = oracle.dykstra(Wf, N, M, wl.MODEL7B_TAU, wl.MODEL7B_ITERS)
        err = assert_S_close(S, S64)
        print(f"7B layer 0 {nm}: max|S-S64| over every block = {err:.3e}", flush=True)


@pytest.mark.parametrize("N,M,tau,iters", [(31, 32, 40.0, 60), (15, 16, 40.0, 60),
                                          (7, 8, 40.0, 60), (3, 4, 60.0, 60)])
@pytest.mark.parametrize("bf16", [False, True])
def test_scale_fold_inputs(N, M, tau, iters, bf16):
    """Inputs whose scales leave the guard's range in blocks that are not
    deep, so the kernels fold them linearly into the kernel (shown on the
    CPU by tests/test_scale_guard_inputs.py): S within 1e-4 of the oracle,
    masks equal to the oracle's rounding of the GPU's S, every block
    feasible."""
    from test_scale_guard_inputs import fold_input
    W_np = fold_input(N, M)
    if bf16:
        W_np = wl.f32_to_bf16_bits(W_np)
    _note(f"scale fold {N}:{M} tau {tau} bf16={bf16}")
    rows, cols = W_np.shape
    _, mask, S, mask2 = _run(W_np, N, M, tau, iters, M)
    Wf = as_f32(W_np)
    assert np.array_equal(mask, mask2)
    assert_feasible(mask, rows, cols, N, M)
    S64, _ = oracle.dykstra(Wf, N, M, tau, iters)
    err = assert_S_close(S, S64)
    ref, _ = oracle.round_matrix(S, Wf, N, M, M)
    assert np.array_equal(mask, ref)
    print(f"scale fold {N}:{M}: max|S-S64| = {err:.3e}", flush=True)


def test_batched_mixed_classes():
    """A batch that interleaves every (M, dtype) class, with ragged shapes and
    a strided matrix, equals per-matrix calls and the oracle's rounding of the
    GPU's own S, block for block."""
    import torch
    rng = np.random.default_rng(77)
    specs = [(32, 16, 64, 96, "bf16"), (4, 2, 8, 36, "f32"), (16, 5, 48, 80, "bf16"),
             (8, 3, 24, 40, "f32"), (32, 31, 32, 64, "f32"), (4, 1, 12, 20, "bf16"),
             (8, 8, 16, 16, "bf16"), (16, 8, 32, 48, "f32")]
    _note("batched mixed classes")
    items, Ws, bits = [], [], []
    for M, N, rows, cols, dt in specs:
        W = rng.standard_normal((rows, cols)).astype(np.float32)
        Wn = wl.f32_to_bf16_bits(W) if dt == "bf16" else W
        Wt = to_device(Wn)
        if M == 16 and dt == "f32":  # strided rows: ld = cols + 8
            big = torch.zeros((rows, cols + 8), dtype=torch.float32, device="cuda")
            big[:, :cols] = Wt
            Wt = big[:, :cols]
        items.append((Wt, N, M))
        Ws.append(Wt)
        bits.append(Wn)
    tau, iters, ls = 25.0, 40, 6
    outs = sms.mask_batched(items, tau, iters, ls, return_frac=True)
    torch.cuda.synchronize()
    for (Wt, N, M), Wn, (m, f) in zip(items, bits, outs):
        m1, f1 = sms.mask(Wt, N, M, tau, iters, ls, return_frac=True)
        torch.cuda.synchronize()
        assert torch.equal(m, m1) and torch.equal(f, f1), (N, M)
        rows, cols = Wt.shape
        assert_feasible(words(m), rows, cols, N, M)
        Wf = as_f32(Wn)
        ref, _ = oracle.round_matrix(f.cpu().numpy(), Wf, N, M, ls)
        assert np.array_equal(words(m), ref), (N, M)
        S64, _ = oracle.dykstra_blocks(Wf, N, M, tau, iters,
                                       np.arange((rows // M) * (cols // M)))
        assert np.abs(gather_blocks(f.cpu().numpy(), M, np.arange(S64.shape[0]), cols)
                      - S64).max() < S_TOL


def test_batched_ex_equals_per_matrix_ex():
    """tsenor_mask_batched_ex over a batch of every (M, dtype) class, with the
    polish and with previous masks (one aliasing its output buffer, one
    absent, the others separate), equals tsenor_mask_ex per matrix and the
    oracle's extended rounding of the GPU's own S."""
    import torch
    rng = np.random.default_rng(78)
    specs = [(32, 16, 64, 96, "bf16"), (4, 2, 8, 36, "f32"), (16, 8, 48, 80, "bf16"),
             (8, 3, 24, 40, "f32"), (16, 5, 32, 48, "f32")]
    tau, iters, ls, K = 25.0, 40, 6, 5
    _note("batched_ex mixed classes")
    items, bits, originals, prevs, outs = [], [], [], [], []
    for k, (M, N, rows, cols, dt) in enumerate(specs):
        W = (0.02 * rng.standard_t(3, (rows, cols))).astype(np.float32)
        Wn = wl.f32_to_bf16_bits(W) if dt == "bf16" else W
        Wt = to_device(Wn)
        items.append((Wt, N, M))
        bits.append(Wn)
        # a previous mask polished further than this call will polish
        p, _ = sms.mask(Wt, N, M, tau, iters, ls, polish_steps=60)
        p = p.clone()
        p[::5, 0] ^= 1  # some blocks infeasible: they ignore it
        originals.append(None if k == 2 else p.clone())
        out = p.clone()
        outs.append(out)
        prevs.append(out if k == 0 else (None if k == 2 else p))  # k = 0 aliases its output
    res = sms.mask_batched(items, tau, iters, ls, return_frac=True, outs=outs,
                           polish_steps=K, prev_masks=prevs)
    torch.cuda.synchronize()
    kept = 0
    for (Wt, N, M), Wn, orig, (m, f) in zip(items, bits, originals, res):
        rows, cols = Wt.shape
        m1, f1 = sms.mask(Wt, N, M, tau, iters, ls, return_frac=True, polish_steps=K,
                          prev_mask=orig)
        torch.cuda.synchronize()
        assert torch.equal(m, m1) and torch.equal(f, f1), (N, M)
        assert_feasible(words(m), rows, cols, N, M)
        ref, st = oracle.round_matrix_ex(f.cpu().numpy(), as_f32(Wn), N, M, ls, K,
                                         prev_mask=None if orig is None else words(orig))
        assert np.array_equal(words(m), ref), (N, M)
        kept += int(st[5])
    print(f"blocks that kept the previous mask: {kept}", flush=True)
    assert kept > 0


def test_prev_mask_overlapping_outputs():
    """A previous mask held in memory that the call's own solves write is read
    before it is overwritten: in a batch, inside another matrix's output
    buffer (prev_masks[0] is mats[1].mask_out); for one matrix, as a view at
    a row offset into the output's buffer.  Results equal those with a
    separate copy of the previous mask."""
    import torch
    rng = np.random.default_rng(81)
    M, N, rows, cols = 16, 8, 48, 64
    tau, iters, ls, K = 25.0, 40, 6, 3
    _note("previous masks overlapping outputs")
    Ws = [to_device(wl.f32_to_bf16_bits((0.02 * rng.standard_t(3, (rows, cols))).astype(np.float32)))
          for _ in range(2)]
    # a previous mask for matrix 0 polished further than this call polishes
    p0, _ = sms.mask(Ws[0], N, M, tau, iters, ls, polish_steps=60)
    p0 = p0.clone()
    out0 = torch.zeros_like(p0)
    out1 = p0.clone()  # matrix 1's output buffer holds matrix 0's previous mask
    sms.mask_batched([(Ws[0], N, M), (Ws[1], N, M)], tau, iters, ls, outs=[out0, out1],
                     polish_steps=K, prev_masks=[out1, None])
    ref0, _ = sms.mask(Ws[0], N, M, tau, iters, ls, polish_steps=K, prev_mask=p0.clone())
    ref1, _ = sms.mask(Ws[1], N, M, tau, iters, ls, polish_steps=K)
    plain0, _ = sms.mask(Ws[0], N, M, tau, iters, ls, polish_steps=K)
    torch.cuda.synchronize()
    assert torch.equal(out0, ref0) and torch.equal(out1, ref1)
    assert not torch.equal(ref0, plain0)  # the previous mask was taken somewhere
    # one matrix: prev = rows h .. h+rows-1 of a buffer whose rows 0 .. rows-1
    # are the output
    h = rows // 3
    buf = torch.zeros((rows + h, p0.shape[1]), dtype=torch.int32, device="cuda")
    buf[h:] = p0
    prev_view = buf[h:]
    m, _ = sms.mask(Ws[0], N, M, tau, iters, ls, polish_steps=K, prev_mask=prev_view,
                    out=buf[:rows])
    torch.cuda.synchronize()
    assert torch.equal(m, ref0)


def test_output_buffers_are_checked():
    """Caller-supplied mask / frac buffers of the wrong shape, dtype or layout
    are refused before anything is enqueued."""
    import torch
    W = to_device(np.ones((32, 64), np.float32))
    bad = [torch.empty((32, 1), dtype=torch.int32, device="cuda"),
           torch.empty((32, 2), dtype=torch.int64, device="cuda"),
           torch.empty((2, 32), dtype=torch.int32, device="cuda").t()]
    for out in bad:
        with pytest.raises(ValueError):
            sms.mask(W, 2, 4, 10.0, 5, 1, out=out)
    with pytest.raises(ValueError):
        sms.mask(W, 2, 4, 10.0, 5, 1, frac_out=torch.empty((32, 32), device="cuda"))
    with pytest.raises(ValueError):
        sms.mask_batched([(W, 2, 4)], 10.0, 5, 1, outs=[])


@pytest.mark.parametrize("N,M,rows,cols", [(16, 32, 96, 192), (8, 16, 64, 160), (2, 4, 32, 48)])
def test_generic_scores(N, M, rows, cols):
    """Any non-negative score matrix can stand in for |W| (here Wanda-style
    |W_ij| * ||X_j||): S and masks match the oracle run on the same scores, and
    the local search scores moves with them."""
    import torch
    rng = np.random.default_rng(5 + M)
    W = (0.02 * rng.standard_normal((rows, cols))).astype(np.float32)
    Sc = wl.wanda_scores(W, 17 + M)
    _note("generic scores", N, M)
    Wt = to_device(Sc)
    mask_t, S_t = sms.mask(Wt, N, M, 30.0, 120, 12, return_frac=True)
    torch.cuda.synchronize()
    S = S_t.cpu().numpy()
    S64, _ = oracle.dykstra(Sc, N, M, 30.0, 120)
    assert np.abs(S - S64).max() < S_TOL
    ref, _ = oracle.round_matrix(S, Sc, N, M, 12)
    assert np.array_equal(words(mask_t), ref)
    assert_feasible(words(mask_t), rows, cols, N, M)


@pytest.mark.parametrize("polish", [2, 1000])
@pytest.mark.parametrize("M,nbc,nbr", SMALL)
def test_polish_parity(M, nbc, nbr, polish):
    """Optional 2-opt polish after the fill: masks bit-exact with the oracle's
    rounding (with the same polish) of the GPU's S, every block feasible and
    never below the unpolished objective."""
    import torch
    N = M // 2
    tau, iters, ls = 20.0, 60, 2
    W_np = _small(500 + M, M, nbc, nbr, "student_t", M >= 16)
    rows, cols = W_np.shape
    _note(f"polish {polish} M={M} {rows}x{cols}")
    W = to_device(W_np)
    m1, S_t = sms.mask(W, N, M, tau, iters, ls, return_frac=True, polish_steps=polish)
    m0 = sms.mask(W, N, M, tau, iters, ls)[0]
    torch.cuda.synchronize()
    S = S_t.cpu().numpy()
    Wf = as_f32(W_np)
    ref, st = oracle.round_matrix_ex(S, Wf, N, M, ls, polish)
    assert np.array_equal(words(m1), ref)
    assert_feasible(words(m1), rows, cols, N, M)
    A = np.abs(Wf.astype(np.float64))
    z1 = oracle.unpack_mask(words(m1), cols) * A
    z0 = oracle.unpack_mask(words(m0), cols) * A
    assert z1.sum() >= z0.sum() and st[4] > 0
    print(f"polish {polish} M={M}: swaps {st[4]}, objective +{(z1.sum() / z0.sum() - 1):.3%}",
          flush=True)


@pytest.mark.parametrize("M,nbc,nbr", SMALL)
def test_keep_better_previous_mask(M, nbc, nbr):
    """A previous mask (here a polished one, with some blocks made infeasible)
    is kept exactly where the oracle keeps it; in place (prev = out) gives the
    same result."""
    import torch
    N = M // 2
    tau, iters, ls = 20.0, 60, 2
    W_np = _small(700 + M, M, nbc, nbr, "outlier", M == 8)
    rows, cols = W_np.shape
    _note(f"previous mask M={M} {rows}x{cols}")
    W = to_device(W_np)
    prev, _ = sms.mask(W, N, M, tau, iters, ls, polish_steps=50)
    prev = prev.clone()
    prev[::3, 0] ^= 1  # break row counts of some blocks: those must ignore it
    m, S_t = sms.mask(W, N, M, tau, iters, ls, return_frac=True, prev_mask=prev)
    inplace = prev.clone()
    sms.mask(W, N, M, tau, iters, ls, out=inplace, prev_mask=inplace)
    torch.cuda.synchronize()
    ref, st = oracle.round_matrix_ex(S_t.cpu().numpy(), as_f32(W_np), N, M, ls, 0,
                                     prev_mask=words(prev))
    assert np.array_equal(words(m), ref) and np.array_equal(words(inplace), ref)
    assert_feasible(words(m), rows, cols, N, M)
    assert st[5] > 0


@pytest.mark.parametrize("M,N,nbc,nbr,kind", [
    (4, 2, 70, 3, "student_t"), (8, 3, 45, 2, "outlier"), (16, 8, 37, 2, "student_t"),
    (16, 5, 21, 2, "ties"), (32, 16, 19, 2, "outlier"), (32, 7, 9, 1, "student_t")])
def test_exact_matches_oracle_optimum(M, N, nbc, nbr, kind):
    """tsenor_exact from the method's mask and from the circulant start: every
    block's objective equals the oracle's min-cost-flow optimum (fp64, 1e-9
    relative), the mask is feasible and realises that objective, and it is
    never below the method's mask."""
    import torch
    W_np = _small(900 + M + N, M, nbc, nbr, kind, M >= 16)
    rows, cols = W_np.shape
    _note(f"exact M={M} N={N} {rows}x{cols} {kind}")
    W = to_device(W_np)
    Wf = as_f32(W_np)
    m0, _ = sms.mask(W, N, M, 20.0, 60, 4)
    ids = np.arange((rows // M) * (cols // M))
    opt = oracle.exact_opt_blocks(Wf, N, M, ids)
    A = np.abs(Wf.astype(np.float64))
    for start in (m0, None):
        m, objv = sms.exact(W, N, M, start=start, return_objective=True)
        torch.cuda.synchronize()
        mw = words(m)
        assert_feasible(mw, rows, cols, N, M)
        o = objv.cpu().numpy().ravel()
        assert np.isfinite(o).all()
        assert np.allclose(o, opt, rtol=1e-9, atol=1e-12), np.abs(o - opt).max()
        got = (oracle.block_view(oracle.unpack_mask(mw, cols).astype(np.float64), M)
               * oracle.block_view(A, M)).sum((2, 3)).ravel()
        assert np.allclose(got, opt, rtol=1e-9, atol=1e-12)
    base = (oracle.block_view(oracle.unpack_mask(words(m0), cols).astype(np.float64), M)
            * oracle.block_view(A, M)).sum((2, 3)).ravel()
    assert (opt >= base - 1e-9).all()
    gap = np.where(opt > 0, (opt - base) / np.where(opt > 0, opt, 1.0), 0.0)  # one block is all zero
    print(f"exact M={M} N={N}: method's mean gap {gap.mean():.4%}", flush=True)


def test_exact_cancel_limit():
    """With no cancellations allowed the circulant start is returned where it is
    not already optimal, flagged NaN; the mask stays feasible."""
    import torch
    M, N = 8, 3
    W_np = _small(1234, M, 20, 2, "student_t", False)
    rows, cols = W_np.shape
    W = to_device(W_np)
    m, objv = sms.exact(W, N, M, max_cancel=0, return_objective=True)
    torch.cuda.synchronize()
    assert_feasible(words(m), rows, cols, N, M)
    assert np.isnan(objv.cpu().numpy()).any()


def test_debug_checks_nonfinite(monkeypatch):
    """TSENOR_DEBUG_CHECKS=1: a NaN or Inf anywhere in W (or S for the
    rounding) is reported as status 7 before anything else runs; finite inputs
    give the same masks as without the checks."""
    import torch
    M, N = 16, 8
    W_np = _small(41, M, 9, 2, "student_t", True)
    W = to_device(W_np)
    ref, _ = sms.mask(W, N, M, 20.0, 30, 8)
    monkeypatch.setenv("TSENOR_DEBUG_CHECKS", "1")
    _note("debug checks, finite input")
    got, _ = sms.mask(W, N, M, 20.0, 30, 8)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    for val in (float("nan"), float("inf"), float("-inf")):
        Wb = W.clone()
        Wb[5, 77] = val
        _note(f"debug checks, W holds {val}")
        with pytest.raises(sms.TsenorError) as ei:
            sms.mask(Wb, N, M, 20.0, 30, 8)
        assert ei.value.status == 7
        with pytest.raises(sms.TsenorError) as ei:
            sms.mask_batched([(Wb, N, M)], 20.0, 30, 8)
        assert ei.value.status == 7
    S = torch.rand(W.shape, device="cuda")
    S[3, 3] = float("nan")
    with pytest.raises(sms.TsenorError) as ei:
        sms.round_mask(S, W, N, M, 8)
    assert ei.value.status == 7
    monkeypatch.setenv("TSENOR_DEBUG_CHECKS", "0")
    sms.mask(Wb, N, M, 20.0, 30, 8)  # unchecked: runs (result undefined)
    torch.cuda.synchronize()
