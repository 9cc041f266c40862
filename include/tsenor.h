/*
 * tsenor.h -- C ABI of the MI355X (gfx950) transposable N:M mask-search library.
 *
 * What it computes (pith.science review of "TSENOR: Highly-Efficient Algorithm
 * for Finding Transposable N:M Sparse Masks", arXiv 2505.23949, sections
 * "What carries the argument" and "Core claim"):
 *
 *   The weight matrix W is tiled into aligned M x M blocks.  Each block gets a
 *   0/1 mask with exactly N ones in every row and every column (so W and W^T are
 *   both N:M sparse), chosen to keep as much of |W| as possible:
 *     1. scores What = |W| / max_block |W|  (an all-zero block scores 0);
 *     2. the block LP is solved as capacitated optimal transport with entropy
 *        regularisation: start X = tau * What, Q = 0, then `iters` times
 *        C1 row normalisation (rows of exp(X) sum to N),
 *        C2 column normalisation (columns sum to N),
 *        C3 clip at 1 with its Dykstra correction (Y = X+Q, X = min(Y,0),
 *        Q = Y - X); the fractional result is S = exp(X) in [0,1];
 *     3. rounding: order the entries by (S descending, in-block index i*M+j
 *        ascending) and accept an entry while its row and column both hold
 *        fewer than N ones; then up to `ls_steps` local-search moves, each the
 *        best move over deficient row i, deficient column j and a kept
 *        (i',j') with Z_ij' = Z_i'j = 0, scored in fp32 as
 *        (|W_ij'| + |W_i'j|) - |W_i'j'|, ties to the smallest (i,j,i',j'),
 *        applied only when the score is > 0; finally a feasibility fill that
 *        repeats the same move (first deficient row and column, best (i',j'),
 *        ties to the smallest) with no sign condition until every row and
 *        column holds N ones.
 *
 * Conventions shared by every entry point:
 *   - All data pointers are DEVICE pointers owned by the caller.  The library
 *     never frees them and keeps no reference after the call.
 *   - W is row-major: element (r, c) is at W[r * ld + c]; ld >= cols.
 *     dtype TSENOR_F32 is IEEE fp32, TSENOR_BF16 is bfloat16 (raw 16-bit
 *     patterns); all arithmetic is fp32 (bf16 widens exactly).
 *   - The mask is bit-packed row-major into uint32 words: ceil(cols/32) words
 *     per row, column c is bit (c % 32) of word (c / 32) (LSB = lowest column).
 *     Bits beyond `cols` in a row's last word are written as 0.
 *   - frac_out / S are fp32 [rows][cols] (leading dimension cols, resp. lds).
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream); results are valid after the caller synchronises that stream.
 *   - Argument errors are detected on the host before any HIP call: the call
 *     returns the status and enqueues nothing.  Launch/runtime failures return
 *     TSENOR_ERR_HIP; tsenor_last_error() then gives the HIP message.
 *   - Results are deterministic: the same inputs give bit-identical masks and
 *     S on every run and for every stream.  Non-finite weights give undefined
 *     (but memory-safe) results.
 *   - Debug checks: with the environment variable TSENOR_DEBUG_CHECKS=1 (read
 *     at every call), tsenor_mask, tsenor_mask_ex, tsenor_mask_batched(_ex),
 *     tsenor_round and tsenor_exact first count the non-finite elements of
 *     their W (and S) on the device, wait for the count, and return
 *     TSENOR_ERR_NONFINITE without launching anything else if it is not zero.
 *     The wait synchronises `stream`, so such calls cannot be graph-captured.
 *   - The kernels need no device workspace: every intermediate of the path
 *     lives in registers and LDS.  The library keeps a few cached buffers per
 *     device (the batched descriptor table, a copy of a previous mask that
 *     overlaps an output; allocated on first use, grown on demand, never
 *     freed before process exit).  Calls that can use one of these buffers
 *     -- tsenor_mask_batched(_ex), tsenor_mask_ex with a previous mask that
 *     overlaps its output -- and tsenor_round and tsenor_exact are ordered:
 *     each launch follows the previous ordered one on the device (stream
 *     event), so concurrent such calls from any thread or stream are safe but
 *     do not overlap.  tsenor_mask, tsenor_mask_ex without such a previous
 *     mask, and tsenor_mask_noalloc use no shared buffer and are not ordered:
 *     calls on different streams may overlap in time (their outputs must not
 *     overlap).  The host side is thread-safe.
 */
#ifndef TSENOR_H
#define TSENOR_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { TSENOR_F32 = 0, TSENOR_BF16 = 1 } tsenor_dtype;

typedef enum {
    TSENOR_OK = 0,
    TSENOR_ERR_NULL = 1,  /* a required pointer is NULL                                */
    TSENOR_ERR_SHAPE = 2, /* rows/cols <= 0, rows % M, cols % M, ld < cols, lds < cols   */
    TSENOR_ERR_NM = 3,    /* M not in {4, 8, 16, 32}, or N < 1, or N > M                 */
    TSENOR_ERR_PARAM = 4, /* tau not finite or < 0, iters < 1, ls_steps < 0, count < 0   */
    TSENOR_ERR_DTYPE = 5, /* dtype not a tsenor_dtype                                   */
    TSENOR_ERR_HIP = 6,   /* HIP runtime or launch failure                              */
    TSENOR_ERR_NONFINITE = 7 /* debug checks only: W (or S) holds an Inf or NaN          */
} tsenor_status;

/* Whole method (steps 1-3 above) on one matrix.
 *   W        device, [rows][ld] of dtype; read only.  Only |W| enters the
 *            method, so any other importance measure can be optimised by
 *            passing its (non-negative) score matrix here, e.g. |W_ij|*||X_j||
 *            with activation norms ||X_j||; the mask then keeps the most score.
 *   N, M     pattern: N ones per row and column of every M x M block.
 *   tau      entropy strength (> = 0, finite), applied to block-max-normalised |W|.
 *   iters    Dykstra cycles (C1, C2, C3), >= 1; no convergence test.
 *   ls_steps maximum local-search moves per block, >= 0.
 *   mask_out device, [rows][ceil(cols/32)] uint32, written entirely.
 *   frac_out device, [rows][cols] fp32 fractional S, or NULL to skip.
 *   stream   hipStream_t or NULL.                                              */
int tsenor_mask(const void* W, int dtype, int64_t rows, int64_t cols, int64_t ld, int N, int M,
                float tau, int iters, int ls_steps, uint32_t* mask_out, float* frac_out,
                void* stream);

/* tsenor_mask followed by two optional stages per block (not part of the
 * method as the pages describe it):
 *   polish_steps  >= 0: at most this many 2-opt swaps after the fill.  A swap
 *            takes kept (i, j) and (i', j'), i < i', with Z_ij' = Z_i'j = 0, to
 *            (i, j') and (i', j), keeping every row and column count; its gain
 *            is (|W_ij'| - |W_i'j'|) + (|W_i'j| - |W_ij|) in fp32 (each
 *            difference rounded, then the sum).  The best gain is applied if
 *            > 0, ties to the smallest (i, j, i', j'); 0 turns the stage off.
 *   prev_mask device, same layout as mask_out, or NULL: a previous mask (e.g.
 *            from an earlier pruning step).  A block takes the previous mask
 *            when that has exactly N ones in every row and column and keeps
 *            strictly more score, sum over rows i ascending of the row sums
 *            over j ascending of |W_ij|, both in fp64; so the result is never
 *            worse than the previous mask.  Blocks where the previous mask is
 *            not feasible ignore it.  prev_mask may alias or overlap mask_out
 *            (in-place update): an overlapping previous mask is copied to a
 *            cached device buffer before the solve writes mask_out.
 * Other arguments, errors and conventions as in tsenor_mask (polish_steps < 0
 * is TSENOR_ERR_PARAM).  tsenor_mask(...) equals tsenor_mask_ex(..., 0, NULL, ...). */
int tsenor_mask_ex(const void* W, int dtype, int64_t rows, int64_t cols, int64_t ld, int N, int M,
                   float tau, int iters, int ls_steps, int polish_steps,
                   const uint32_t* prev_mask, uint32_t* mask_out, float* frac_out,
                   void* stream);

/* tsenor_mask for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, result (bit-identical masks and S) and argument errors as
 * tsenor_mask.  It calls no hipMalloc, hipFree or other allocating routine and
 * records or waits on no event.  The path needs no workspace (every
 * intermediate lives in registers and LDS), so no matrix size is beyond it,
 * nothing needs clearing between calls, and calls that overlap in time
 * (different streams, threads without ordering) are independent as long as
 * their outputs do not overlap.  It is not ordered after the other entry
 * points' launches.  TSENOR_DEBUG_CHECKS is ignored here (its check
 * allocates).  The first call on a device also reads the device's
 * launch geometry (CU count, kernel occupancies).                             */
int tsenor_mask_noalloc(const void* W, int dtype, int64_t rows, int64_t cols, int64_t ld,
                        int N, int M, float tau, int iters, int ls_steps, uint32_t* mask_out,
                        float* frac_out, void* stream);

/* Exact optimum of every block: the mask with N ones per row and column that
 * keeps the most |W| (the block LP is a bipartite b-matching, so its optimum
 * is integral).  Not part of the method -- the reference it is measured
 * against (optimality gap, speed-up over an exact solver).  From a feasible
 * start, negative cycles of the block's residual graph are cancelled until a
 * Bellman-Ford pass finds none, which certifies optimality up to 2^-40 of the
 * block's max |W|.
 *   start_mask  device, same layout as mask_out: a feasible start, e.g. the
 *            output of tsenor_mask (blocks whose start is not feasible, and
 *            every block when NULL, start from the circulant mask row i ->
 *            columns i .. i+N-1 mod M).  May alias mask_out.
 *   max_cancel  >= 0, cancellations allowed per block.
 *   mask_out device, written entirely; always feasible.
 *   objective_out  device, fp64 [rows/M][cols/M] per-block objective (sum of
 *            |W| over the mask, rows then columns ascending), NaN where
 *            optimality was not certified within max_cancel; or NULL.
 * Other arguments, errors and conventions as in tsenor_mask.                   */
int tsenor_exact(const void* W, int dtype, int64_t rows, int64_t cols, int64_t ld, int N, int M,
                 const uint32_t* start_mask, int max_cancel, uint32_t* mask_out,
                 double* objective_out, void* stream);

/* ---- 2:4 consumer: one transposable mask serves W and W^T ----------------
 * Not part of the mask search: the payoff the pages measure -- with a 2:4
 * transposable mask (N = 2, M = 4) both the forward product Y = X W^T and the
 * data gradient dX = dY W = dY (W^T)^T reduce over a 2:4-sparse dimension and
 * run on the sparse matrix cores.
 *
 * Compressed operand A [arows][k], 2:4 along k (k a multiple of 32):
 *   values  device bf16 [arows][k/2]: per aligned group of 4 along k, its kept
 *           entries (at most two) in ascending position, unused slots 0;
 *   meta    device uint32 [arows][k/32]: group g of each 32-wide chunk in bits
 *           4g..4g+3, low two bits = position of the first value, high two =
 *           the second's.
 *
 * tsenor_compress24: A = W (transpose 0: arows = rows, k = cols) or A = W^T
 * (transpose 1: arows = cols, k = rows) restricted to `mask` (the layout of
 * tsenor_mask's output).  W is bf16 [rows][ld].  Groups with more than two
 * kept entries keep the first two and are counted into *bad_groups (device
 * int, added to; NULL = no count).  Errors: NULL pointers, bad shapes
 * (k % 32 != 0), transpose not 0/1.
 *
 * tsenor_spmm24: Y = X A^T.  X device bf16 [n][ldx] (16-byte aligned, ldx a
 * multiple of 8), A compressed [m][k], Y device fp32 [n][ldy] (16-byte
 * aligned, ldy a multiple of 4), fp32 accumulation.  n and m multiples of 128,
 * k of 32 (TSENOR_ERR_SHAPE otherwise).  Asynchronous on `stream`.          */
int tsenor_compress24(const void* W, int64_t rows, int64_t cols, int64_t ld,
                      const uint32_t* mask, int transpose, uint16_t* values_out,
                      uint32_t* meta_out, int* bad_groups, void* stream);
int tsenor_spmm24(const void* X, int64_t n, int64_t ldx, const uint16_t* values,
                  const uint32_t* meta, int64_t m, int64_t k, float* Y, int64_t ldy,
                  void* stream);

/* One matrix of a batch.  Field meanings as in tsenor_mask.                    */
typedef struct {
    const void* W;
    int dtype;
    int64_t rows, cols, ld;
    int N, M;
    uint32_t* mask_out;
    float* frac_out; /* NULL = don't write */
} tsenor_matrix;

/* Many matrices (possibly of different shape, dtype and N:M) in one call, one
 * kernel launch per (M, dtype) class present, e.g. every projection of a
 * transformer.  `mats` is a HOST array of `count` descriptors (count >= 0; 0
 * is a no-op); every descriptor is validated as in tsenor_mask before
 * anything is enqueued.  tau, iters and ls_steps apply to all matrices.  The
 * descriptor table is built in one of eight pinned host staging buffers
 * (used in turn) and uploaded on `stream`, so `mats` may be reused as soon
 * as the call returns.  The call does not wait for the device, except when
 * the staging buffer it takes still holds the table of the batched call
 * eight calls earlier whose upload has not yet run.  Each matrix's mask and
 * S are those tsenor_mask gives for it alone.                                */
int tsenor_mask_batched(const tsenor_matrix* mats, int count, float tau, int iters,
                        int ls_steps, void* stream);

/* tsenor_mask_batched with tsenor_mask_ex's optional stages for every matrix:
 * polish_steps >= 0 as in tsenor_mask_ex; prev_masks is NULL or a HOST array
 * of `count` device pointers, entry i a previous mask for matrix i (layout of
 * its mask_out) or NULL.  A previous mask may alias or overlap the mask_out of
 * any matrix of the call: such masks are copied to a cached device buffer
 * before any solve writes.  Each matrix's result equals tsenor_mask_ex's for
 * it alone.  polish_steps < 0 is TSENOR_ERR_PARAM.                           */
int tsenor_mask_batched_ex(const tsenor_matrix* mats, int count, float tau, int iters,
                           int ls_steps, int polish_steps, const uint32_t* const* prev_masks,
                           void* stream);

/* Rounding only (step 3) on a caller-supplied fractional matrix S.
 *   S        device, [rows][lds] fp32, values in [0, 1] (as produced by the
 *            solver; values outside [0,1] give an unspecified order), read only.
 *   W        device, [rows][ld] of dtype; |W| scores the local-search moves.
 * Other arguments as in tsenor_mask.                                           */
int tsenor_round(const float* S, int64_t lds, const void* W, int dtype, int64_t rows,
                 int64_t cols, int64_t ld, int N, int M, int ls_steps, uint32_t* mask_out,
                 void* stream);

/* Static, human-readable name of a status code (never NULL).                   */
const char* tsenor_status_str(int status);

/* Message of the last TSENOR_ERR_HIP on the calling thread ("" if none).       */
const char* tsenor_last_error(void);

/* ABI version: 0x00MMmmpp.                                                     */
int tsenor_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TSENOR_H */
