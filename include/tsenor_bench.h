/*
 * tsenor_bench.h -- measurement-only entry point of libtsenor.so (not part of
 * the mask-search interface in tsenor.h).
 *
 * The fused mask kernel of tsenor_mask reads W once, block by block, and
 * writes one bit per weight; its cost is dominated by the Dykstra cycles, so
 * its own HBM rate says little about how fast that memory work can go.  This
 * entry point runs the same memory work alone, so that the memory side can be
 * measured against the HBM roofline on the machine at hand.
 */
#ifndef TSENOR_BENCH_H
#define TSENOR_BENCH_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads every M x M block of W once (16-byte loads), takes the block max of
 * |W| and writes, for every weight, the bit (2|W| >= block max) into mask_out
 * in tsenor_mask's layout ([rows][ceil(cols/32)] uint32 words, column c is bit
 * c % 32 of word c / 32).  No part of the mask search runs.
 *   W        device, [rows][ld] of dtype (TSENOR_F32 or TSENOR_BF16); W and
 *            every row must be 16-byte aligned (ld * element size % 16 == 0).
 *   M        16 or 32; rows and cols positive multiples of M; ld >= cols.
 *   mask_out device, written entirely.
 *   stream   hipStream_t or NULL.  Asynchronous.
 * Returns a tsenor_status: TSENOR_ERR_NULL, _DTYPE, _NM (M not 16 or 32),
 * _SHAPE (sizes or alignment) before any HIP call, TSENOR_ERR_HIP on a launch
 * failure.                                                                   */
int tsenor_bench_memory_pass(const void* W, int dtype, int64_t rows, int64_t cols, int64_t ld,
                             int M, uint32_t* mask_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TSENOR_BENCH_H */
