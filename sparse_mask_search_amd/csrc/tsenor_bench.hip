// tsenor_bench.hip -- measurement-only kernel: the memory side of the mask
// search on its own.
//
// The fused mask kernel reads W once, block by block, and writes one bit per
// weight.  This kernel does exactly that HBM work and nothing of the method's
// solve or rounding: it reads every M x M block of W with 16-byte loads,
// takes the block max of |W| and writes the packed bits (2|W| >= block max),
// in the mask layout of tsenor_mask.  Its duration against the algorithmic
// bytes (W once + the mask once) is the achievable rate of that memory work,
// the bound the fused kernel's own memory traffic is compared with.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tsenor_internal.h"

namespace tsenor {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// |W| of the 8 bf16 or 4 fp32 values of a 16-byte load, as fp32.
template <bool BF16>
__device__ __forceinline__ void abs_values(const u32x4 v, float (&a)[BF16 ? 8 : 4]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    if constexpr (BF16) {
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            a[2 * h] = __uint_as_float((w[h] & 0x7FFFu) << 16);
            a[2 * h + 1] = __uint_as_float(w[h] & 0x7FFF0000u);
        }
    } else {
#pragma unroll
        for (int h = 0; h < 4; ++h) a[h] = __uint_as_float(w[h] & 0x7FFFFFFFu);
    }
}

// One wave covers one block-row (M rows) by 64 * CPL columns: lane l holds
// columns l*CPL .. l*CPL+CPL-1 of every row (one 16-byte load per row), so a
// block spans M/CPL lanes and a 32-column mask word 32/CPL lanes.
template <int M, bool BF16>
__global__ __launch_bounds__(256) void memory_pass_kernel(const void* __restrict__ W, int64_t rows,
                                                          int64_t cols, int64_t ld,
                                                          uint32_t* __restrict__ mask,
                                                          int64_t wpr) {
    constexpr int CPL = BF16 ? 8 : 4;      // columns per lane (16 bytes)
    constexpr int LPB = M / CPL;           // lanes per block
    constexpr int LPW = 32 / CPL;          // lanes per mask word
    static_assert(M % CPL == 0 && 32 % CPL == 0, "tile");
    const int lane = threadIdx.x % 64;
    const int64_t wave = (int64_t)blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64;
    const int64_t strips = (cols + 64 * CPL - 1) / (64 * CPL);
    const int64_t br = wave / strips;
    if (br >= rows / M) return;
    const int64_t c0 = (wave % strips) * 64 * CPL + (int64_t)lane * CPL;
    const bool valid = c0 < cols;  // cols is a multiple of M, so a lane is all in or all out
    // raw 16-byte rows (M x 4 registers); |W| is formed when used
    u32x4 raw[M];
#pragma unroll
    for (int r = 0; r < M; ++r) {
        const int64_t off = (br * M + r) * ld + c0;
        if (!valid) {
            raw[r] = u32x4{0u, 0u, 0u, 0u};
        } else if constexpr (BF16) {
            raw[r] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(W) + off));
        } else {
            raw[r] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4*>(static_cast<const float*>(W) + off));
        }
    }
    // Empty asm "updates" of the raw rows keep them as loaded: without them the
    // compiler widens every row to fp32 at once (twice the registers, 30%
    // lower bandwidth from the lower occupancy).
#pragma unroll
    for (int r = 0; r < M; ++r) asm volatile("" : "+v"(raw[r]));
    float m = 0.f;
#pragma unroll
    for (int r = 0; r < M; ++r) {
        float a[CPL];
        abs_values<BF16>(raw[r], a);
#pragma unroll
        for (int k = 0; k < CPL; ++k) m = fmaxf(m, a[k]);
    }
#pragma unroll
    for (int s = 1; s < LPB; s <<= 1) m = fmaxf(m, __shfl_xor(m, s));
    const int shift = (lane % LPW) * CPL;
#pragma unroll
    for (int r = 0; r < M; ++r) {
        float a[CPL];
        asm volatile("" : "+v"(raw[r]));
        abs_values<BF16>(raw[r], a);
        uint32_t bits = 0;
#pragma unroll
        for (int k = 0; k < CPL; ++k) bits |= (2.0f * a[k] >= m ? 1u : 0u) << k;
        if (!valid) bits = 0u;  // columns past the matrix (a ragged last word) stay 0
        uint32_t word = bits << shift;
#pragma unroll
        for (int s = 1; s < LPW; s <<= 1) word |= (uint32_t)__shfl_xor((int)word, s);
        if (valid && lane % LPW == 0) mask[(br * M + r) * wpr + (c0 >> 5)] = word;
    }
}

}  // namespace

int launch_memory_pass(const void* W, int bf16, int64_t rows, int64_t cols, int64_t ld, int M,
                       uint32_t* mask, int64_t wpr, void* stream) {
    const int cpl = bf16 ? 8 : 4;
    const int64_t strips = (cols + 64 * cpl - 1) / (64 * cpl);
    const int64_t waves = (rows / M) * strips;
    const int64_t blocks = (waves + 3) / 4;
    const dim3 grid((unsigned)blocks), block(256);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (M == 32 && bf16) hipLaunchKernelGGL((memory_pass_kernel<32, true>), grid, block, 0, s, W, rows, cols, ld, mask, wpr);
    else if (M == 32) hipLaunchKernelGGL((memory_pass_kernel<32, false>), grid, block, 0, s, W, rows, cols, ld, mask, wpr);
    else if (M == 16 && bf16) hipLaunchKernelGGL((memory_pass_kernel<16, true>), grid, block, 0, s, W, rows, cols, ld, mask, wpr);
    else if (M == 16) hipLaunchKernelGGL((memory_pass_kernel<16, false>), grid, block, 0, s, W, rows, cols, ld, mask, wpr);
    else return (int)hipErrorInvalidValue;
    return (int)hipGetLastError();
}

}  // namespace tsenor
