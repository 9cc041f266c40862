// tsenor_spmm.hip -- a consumer of transposable 2:4 masks on gfx950: the
// weight matrix compressed to 2:4 along either of its dimensions, and
// Y = X A^T on the sparse matrix cores (v_smfmac_f32_32x32x32_bf16).
//
// Why transposable masks matter (pith.science review of "TSENOR: Highly-
// Efficient Algorithm for Finding Transposable N:M Sparse Masks", "Core
// claim"): with one mask both W (forward, Y = X W^T) and W^T (data gradient,
// dX = dY W = dY (W^T)^T) are 2:4 along the reduction dimension, so both
// products run on the sparse matrix cores.
//
// Compressed operand A [rows][k] (2:4 along k):
//   values  bf16 [rows][k/2]: for each aligned group of 4 along k, its (at most
//           two) kept entries in ascending position; unused slots are 0.
//   meta    uint32 [rows][k/32]: group g of a 32-wide chunk in bits 4g..4g+3,
//           low two bits = position (0..3) of the first value, high two = the
//           second's.
// smfmac 32x32x32 operand layout (measured on gfx950 with an in-bounds probe):
// lane l holds A row l%32, and for h = l/32 the groups 2h, 2h+1 (k = 8h..8h+7)
// and 4+2h, 5+2h (k = 16+8h..16+8h+7) of the chunk, two slots per group with a
// 2-bit position each in the index operand; B lane l holds column l%32 at
// k = 16h..16h+15; the accumulator is the usual 32x32 layout (lane l: column
// l%32, rows 8*i0 + 4h + i1).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tsenor_internal.h"

namespace tsenor {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x16 __attribute__((ext_vector_type(16)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));

// One thread per (row of A, 32-wide chunk of k): element (r, c) of A is
// W[r][c] (trans = 0) or W[c][r] (trans = 1); mask bit likewise.  Groups with
// more than two kept entries are counted into *bad (their first two are kept).
__global__ void compress24_kernel(const uint16_t* __restrict__ W, int64_t ld,
                                  const uint32_t* __restrict__ mask, int64_t wpr, int64_t rows,
                                  int64_t k, int trans, uint16_t* __restrict__ vals,
                                  uint32_t* __restrict__ meta, int* __restrict__ bad) {
    const int64_t chunks = k / 32;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= rows * chunks) return;
    const int64_t r = t / chunks, ch = t % chunks;
    uint32_t mw = 0u;
    uint16_t v[16];
    int nbad = 0;
#pragma unroll
    for (int g = 0; g < 8; ++g) {
        int cnt = 0;
        uint32_t pos = 0u;
        uint16_t x0 = 0, x1 = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t c = ch * 32 + 4 * g + j;
            const int64_t wr = trans ? c : r, wc = trans ? r : c;
            const bool keep = (mask[wr * wpr + (wc >> 5)] >> (int)(wc & 31)) & 1u;
            if (keep) {
                const uint16_t x = W[wr * ld + wc];
                if (cnt == 0) { x0 = x; pos |= (uint32_t)j; }
                else if (cnt == 1) { x1 = x; pos |= (uint32_t)j << 2; }
                ++cnt;
            }
        }
        if (cnt > 2) ++nbad;
        if (cnt < 2) {  // pad: the unused slot points at a free position, value 0
            const uint32_t p0 = pos & 3u;
            if (cnt == 0) pos = 0u | (1u << 2);
            else pos = p0 | ((p0 == 3u ? 2u : 3u) << 2);
        }
        v[2 * g] = x0;
        v[2 * g + 1] = x1;
        mw |= pos << (4 * g);
    }
    uint16_t* out = vals + r * (k / 2) + ch * 16;
#pragma unroll
    for (int q = 0; q < 16; ++q) out[q] = v[q];
    meta[r * chunks + ch] = mw;
    if (nbad && bad != nullptr) atomicAdd(bad, nbad);
}

// Output tile (tm, tn) of workgroup `bid` in a tiles_m x tiles_n grid.  The
// hardware hands workgroups to the chip's 8 XCDs round robin (workgroup b runs
// on XCD b % 8), and each XCD has its own L2.  When the grid divides by 8, XCD
// x gets the contiguous tile range [x nb/8, (x+1) nb/8) of an order that walks
// groups of up to 8 m-tiles column by column, so the tiles an XCD runs at one
// time form a compact block of the grid: 32 concurrent tiles cover 8 m-tiles
// (rows of A) by 4 n-tiles (rows of X, twice the bytes of an A tile) instead of
// 2 by 16, and share those rows in the XCD's L2.  A bijection on [0, nb).
__device__ __forceinline__ void tile_of_block(int64_t bid, int64_t tiles_m, int64_t tiles_n,
                                              int64_t& tm, int64_t& tn) {
    constexpr int64_t kXcd = 8, kGroupM = 8;
    const int64_t nb = tiles_m * tiles_n;
    const int64_t t = (nb % kXcd == 0) ? (bid % kXcd) * (nb / kXcd) + bid / kXcd : bid;
    const int64_t per_group = kGroupM * tiles_n;
    const int64_t grp = t / per_group, first = grp * kGroupM;
    const int64_t gm = (tiles_m - first < kGroupM) ? tiles_m - first : kGroupM;
    const int64_t r = t - grp * per_group;
    tm = first + r % gm;
    tn = r / gm;
}

// Y [n][m] fp32 (leading dimension ldy) = X [n][k] bf16 (ldx) times A^T, A
// [m][k] compressed as above.  One workgroup of 4 waves per 128 x 128 tile of
// (m, n); each wave owns 64 x 64 = 2 x 2 smfmac tiles and walks k in chunks of
// 32.  m, n multiples of 128 and k of 32 (checked on the host).
__global__ __launch_bounds__(256) void spmm24_kernel(const uint16_t* __restrict__ X, int64_t ldx,
                                                     const uint16_t* __restrict__ vals,
                                                     const uint32_t* __restrict__ meta,
                                                     float* __restrict__ Y, int64_t ldy, int64_t n,
                                                     int64_t m, int64_t k) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int h = lane >> 5, l32 = lane & 31;
    int64_t tm, tn;
    tile_of_block(blockIdx.x, m / 128, n / 128, tm, tn);
    const int64_t m0 = tm * 128 + 64 * (wave >> 1), n0 = tn * 128 + 64 * (wave & 1);
    const int64_t chunks = k / 32;
    f32x16 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int t = 0; t < 16; ++t) acc[a][b][t] = 0.f;
    const uint16_t* arow[2];
    const uint32_t* mrow[2];
    const uint16_t* brow[2];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
        const int64_t r = m0 + 32 * a + l32;
        arow[a] = vals + r * (k / 2) + 4 * h;
        mrow[a] = meta + r * chunks;
    }
#pragma unroll
    for (int b = 0; b < 2; ++b) brow[b] = X + (n0 + 32 * b + l32) * ldx + 16 * h;
    for (int64_t ch = 0; ch < chunks; ++ch) {
        bf16x8 av[2];
        int idx[2];
        bf16x16 bv[2];
#pragma unroll
        for (int a = 0; a < 2; ++a) {
            const u32x2 lo = *reinterpret_cast<const u32x2*>(arow[a] + ch * 16);
            const u32x2 hi = *reinterpret_cast<const u32x2*>(arow[a] + ch * 16 + 8);
            const u32x4 w4 = {lo.x, lo.y, hi.x, hi.y};
            av[a] = __builtin_bit_cast(bf16x8, w4);
            const uint32_t mw = mrow[a][ch];
            idx[a] = (int)(((mw >> (8 * h)) & 0xFFu) | (((mw >> (16 + 8 * h)) & 0xFFu) << 8));
        }
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const u32x4 p = *reinterpret_cast<const u32x4*>(brow[b] + ch * 32);
            const u32x4 q = *reinterpret_cast<const u32x4*>(brow[b] + ch * 32 + 8);
            typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
            const u32x8 w8 = {p.x, p.y, p.z, p.w, q.x, q.y, q.z, q.w};
            bv[b] = __builtin_bit_cast(bf16x16, w8);
        }
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b)
                acc[a][b] = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(av[a], bv[b], acc[a][b], idx[a], 0, 0);
    }
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            float* y = Y + (n0 + 32 * b + l32) * ldy + m0 + 32 * a + 4 * h;
#pragma unroll
            for (int i0 = 0; i0 < 4; ++i0)
                *reinterpret_cast<float4*>(y + 8 * i0) =
                    make_float4(acc[a][b][4 * i0], acc[a][b][4 * i0 + 1], acc[a][b][4 * i0 + 2],
                                acc[a][b][4 * i0 + 3]);
        }
}

// The same product for m and n multiples of 64 WM and 64 WN and k of 64: a
// workgroup of 2 x 2 waves owns a (64 WM) x (64 WN) tile of (m, n), a wave
// WM x WN smfmac tiles (accumulators in AGPRs, one wave per SIMD), so each
// operand read from LDS feeds WN (A) or WM (B) instructions.  Both operands
// reach LDS by direct loads (global_load_lds_dwordx4: lane l's 16 bytes land
// at the instruction's LDS base + 16 l), with no register staging, into a
// ring of three k-step buffers filled two steps ahead.  Swizzles keep the LDS
// reads conflict-free for X (row r keeps its eight 16-byte chunks at
// c ^ ((r >> 1) & 7): the 16 rows of one pass hit 16 bank groups) and at most
// two-way for A (row r keeps its four 16-byte chunks at c ^ ((r >> 2) & 3)).
typedef __attribute__((address_space(3))) void lds_void_t;

// One lane's 16 (or 4) bytes from global memory to LDS at base + 16 l (4 l).
// Written in asm because the compiler cannot tell the ring buffers apart: it
// would wait for every outstanding direct load before each LDS read, which
// serialises the ring.  The kernel waits for them itself (vmcnt) before the
// barrier that publishes a buffer.  No register receives data, so nothing is
// left in flight in a VGPR.  M0 carries the LDS base; nothing else in this
// kernel uses M0 (checked in its ISA), and the clobber tells the compiler.
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
    return (uint32_t)(uintptr_t)(const lds_void_t*)p;
}
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // M0 is a reserved register; see above
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(g), "s"(lds_base) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* g, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
                 :: "v"(g), "s"(lds_base) : "memory", "m0");
}
#pragma clang diagnostic pop

template <int WM, int WN>
__global__ __launch_bounds__(256) void spmm24_dma_kernel(const uint16_t* __restrict__ X, int64_t ldx,
                                                         const uint16_t* __restrict__ vals,
                                                         const uint32_t* __restrict__ meta,
                                                         float* __restrict__ Y, int64_t ldy,
                                                         int64_t n, int64_t m, int64_t k) {
    constexpr int TM = 64 * WM, TN = 64 * WN;
    static_assert(TN % 32 == 0 && TM % 64 == 0, "tile");
    constexpr int QX = TN / 8 / 4;   // 1 KiB X instructions per wave per step (8 rows each)
    constexpr int QA = TM / 16 / 4;  // 1 KiB A instructions per wave (16 rows each)
    constexpr int QM = TM / 32 / 4;  // 256 B position instructions per wave (32 rows each)
    __shared__ u32x4 Xs0[TN * 8], Xs1[TN * 8], Xs2[TN * 8];
    __shared__ u32x2 As0[TM * 8], As1[TM * 8], As2[TM * 8];
    __shared__ u32x2 Ms0[TM], Ms1[TM], Ms2[TM];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int h = lane >> 5, l32 = lane & 31;
    int64_t tm, tn;
    tile_of_block(blockIdx.x, m / TM, n / TN, tm, tn);
    const int64_t m0 = tm * TM, n0 = tn * TN;
    const int64_t kh = k / 2, kw = k / 32;
    const int steps = (int)(k / 64);

    // per-lane global sources of this wave's instructions (step 0)
    const uint16_t* xsrc[QX];
#pragma unroll
    for (int j = 0; j < QX; ++j) {
        const int q = wave * QX + j, row = 8 * q + (lane >> 3), p = lane & 7;
        xsrc[j] = X + (n0 + row) * ldx + 8 * (p ^ ((row >> 1) & 7));
    }
    const uint16_t* asrc[QA];
#pragma unroll
    for (int j = 0; j < QA; ++j) {
        const int q = wave * QA + j, row = 16 * q + (lane >> 2), sl = lane & 3;
        asrc[j] = vals + (m0 + row) * kh + 8 * (sl ^ ((row >> 2) & 3));
    }
    const uint32_t* msrc[QM];
#pragma unroll
    for (int j = 0; j < QM; ++j) {
        const int q = wave * QM + j, row = 32 * q + (lane >> 1);
        msrc[j] = meta + (m0 + row) * kw + (lane & 1);
    }
    f32x16 acc[WM][WN];
#pragma unroll
    for (int a = 0; a < WM; ++a)
#pragma unroll
        for (int b = 0; b < WN; ++b)
#pragma unroll
            for (int t = 0; t < 16; ++t) acc[a][b][t] = 0.f;

    // issue the loads of k-step ST (clamped to the last step: a repeated
    // step lands in a buffer no later step reads) into buffer set XB/AB/MB
#define SPMM_ISSUE(ST, XB, AB, MB)                                                           \
    {                                                                                        \
        const int s_ = (ST) < steps ? (ST) : steps - 1;                                      \
        _Pragma("unroll") for (int j = 0; j < QX; ++j)                                       \
            dma16(xsrc[j] + 64 * s_, lds_offset((XB) + (wave * QX + j) * 64));                 \
        _Pragma("unroll") for (int j = 0; j < QA; ++j)                                       \
            dma16(asrc[j] + 32 * s_, lds_offset((AB) + (wave * QA + j) * 128));                \
        _Pragma("unroll") for (int j = 0; j < QM; ++j)                                       \
            dma4(msrc[j] + 2 * s_, lds_offset((MB) + (wave * QM + j) * 32));                   \
    }
#define SPMM_COMPUTE(XB, AB, MB)                                                             \
    {                                                                                        \
        bf16x16 bv[2][WN];                                                                   \
        bf16x8 avv[2][WM];                                                                   \
        u32x2 mmv[WM];                                                                       \
        _Pragma("unroll") for (int kc = 0; kc < 2; ++kc) {                                   \
            _Pragma("unroll") for (int b = 0; b < WN; ++b) {                                 \
                const int row = 32 * (WN * wn + b) + l32, sw = (row >> 1) & 7;               \
                const int c0 = 4 * kc + 2 * h;                                               \
                const u32x4 p = (XB)[row * 8 + (c0 ^ sw)];                                   \
                const u32x4 q = (XB)[row * 8 + ((c0 + 1) ^ sw)];                             \
                const u32x8 w8 = {p.x, p.y, p.z, p.w, q.x, q.y, q.z, q.w};                   \
                bv[kc][b] = __builtin_bit_cast(bf16x16, w8);                                 \
            }                                                                                \
            _Pragma("unroll") for (int a = 0; a < WM; ++a) {                                 \
                const int row = 32 * (WM * wm + a) + l32, g = (row >> 2) & 3;                \
                const u32x2 lo = (AB)[row * 8 + 2 * ((2 * kc) ^ g) + h];                     \
                const u32x2 hi = (AB)[row * 8 + 2 * ((2 * kc + 1) ^ g) + h];                 \
                const u32x4 w4 = {lo.x, lo.y, hi.x, hi.y};                                   \
                avv[kc][a] = __builtin_bit_cast(bf16x8, w4);                                 \
                if (kc == 0) mmv[a] = (MB)[row];                                             \
            }                                                                                \
        }                                                                                    \
        __builtin_amdgcn_sched_barrier(0);                                                   \
        _Pragma("unroll") for (int kc = 0; kc < 2; ++kc) {                                   \
            _Pragma("unroll") for (int a = 0; a < WM; ++a) {                                 \
                const uint32_t mw = kc ? mmv[a].y : mmv[a].x;                                \
                const int idx =                                                              \
                    (int)(((mw >> (8 * h)) & 0xFFu) | (((mw >> (16 + 8 * h)) & 0xFFu) << 8)); \
                _Pragma("unroll") for (int b = 0; b < WN; ++b) acc[a][b] =                   \
                    __builtin_amdgcn_smfmac_f32_32x32x32_bf16(avv[kc][a], bv[kc][b], acc[a][b], \
                                                              idx, 0, 0);                    \
            }                                                                                \
        }                                                                                    \
    }
    // k-step ST from buffer set 0/1/2: its loads are complete once at most the
    // next step's are outstanding, and every LDS read of the previous step is
    // done; after the barrier every wave's part is visible and the buffer the
    // step after next fills is no longer read by anyone.
#define SPMM_DSTEP(ST, XB, AB, MB, XN, AN, MN)                                               \
    {                                                                                        \
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(QX + QA + QM) : "memory");      \
        __builtin_amdgcn_s_barrier();                                                        \
        asm volatile("" ::: "memory");                                                       \
        __builtin_amdgcn_sched_barrier(0);                                                   \
        SPMM_ISSUE((ST) + 2, XN, AN, MN)                                                     \
        SPMM_COMPUTE(XB, AB, MB)                                                             \
    }

    SPMM_ISSUE(0, Xs0, As0, Ms0)
    SPMM_ISSUE(1, Xs1, As1, Ms1)
    int st = 0;
    for (; st + 3 <= steps; st += 3) {
        SPMM_DSTEP(st, Xs0, As0, Ms0, Xs2, As2, Ms2)
        SPMM_DSTEP(st + 1, Xs1, As1, Ms1, Xs0, As0, Ms0)
        SPMM_DSTEP(st + 2, Xs2, As2, Ms2, Xs1, As1, Ms1)
    }
    if (st < steps) SPMM_DSTEP(st, Xs0, As0, Ms0, Xs2, As2, Ms2)
    if (st + 1 < steps) SPMM_DSTEP(st + 1, Xs1, As1, Ms1, Xs0, As0, Ms0)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#undef SPMM_DSTEP
#undef SPMM_COMPUTE
#undef SPMM_ISSUE
#pragma unroll
    for (int a = 0; a < WM; ++a)
#pragma unroll
        for (int b = 0; b < WN; ++b) {
            float* y = Y + (n0 + 32 * (WN * wn + b) + l32) * ldy + m0 + 32 * (WM * wm + a) + 4 * h;
#pragma unroll
            for (int i0 = 0; i0 < 4; ++i0)
                *reinterpret_cast<float4*>(y + 8 * i0) =
                    make_float4(acc[a][b][4 * i0], acc[a][b][4 * i0 + 1], acc[a][b][4 * i0 + 2],
                                acc[a][b][4 * i0 + 3]);
        }
}

}  // namespace

int launch_compress24(const uint16_t* W, int64_t ld, const uint32_t* mask, int64_t wpr,
                      int64_t rows, int64_t k, int trans, uint16_t* vals, uint32_t* meta, int* bad,
                      void* stream) {
    const int64_t threads = rows * (k / 32);
    const int64_t blocks = (threads + 255) / 256;
    hipLaunchKernelGGL(compress24_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       W, ld, mask, wpr, rows, k, trans, vals, meta, bad);
    return (int)hipGetLastError();
}

int launch_spmm24(const uint16_t* X, int64_t ldx, const uint16_t* vals, const uint32_t* meta,
                  float* Y, int64_t ldy, int64_t n, int64_t m, int64_t k, void* stream) {
    constexpr int WM = 4, WN = 4;
    constexpr int TM = 64 * WM, TN = 64 * WN;
    if (m % TM == 0 && n % TN == 0 && k % 64 == 0 && ldx % 8 == 0 &&
        (reinterpret_cast<uintptr_t>(meta) & 7u) == 0 &&
        (reinterpret_cast<uintptr_t>(vals) & 15u) == 0) {
        const int64_t blocks = (m / TM) * (n / TN);
        hipLaunchKernelGGL((spmm24_dma_kernel<WM, WN>), dim3((unsigned)blocks), dim3(256), 0,
                           (hipStream_t)stream, X, ldx, vals, meta, Y, ldy, n, m, k);
        return (int)hipGetLastError();
    }
    const int64_t blocks = (m / 128) * (n / 128);
    hipLaunchKernelGGL(spmm24_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, X,
                       ldx, vals, meta, Y, ldy, n, m, k);
    return (int)hipGetLastError();
}

}  // namespace tsenor
