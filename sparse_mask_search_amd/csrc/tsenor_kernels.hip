// tsenor_kernels.hip -- gfx950 kernels for transposable N:M mask search.
//
// Method: pith.science review of "TSENOR: Highly-Efficient Algorithm for Finding
// Transposable N:M Sparse Masks" (arXiv 2505.23949), "What carries the argument"
// and "Core claim": entropic capacitated OT per M x M block solved by Dykstra's
// projections (row normalisation C1, column normalisation C2, clip at 1 with its
// correction C3), then rounding by a descending sort, greedy within row/column
// budgets, swap local search and a feasibility fill.
//
// One 64-lane workgroup (one wave) owns a "group" of horizontally adjacent
// blocks of one block-row and runs the whole path for them:
//
//  1. gather   each lane reads R rows of its tile straight from HBM
//              (8/16-byte loads), |W| -> fp32, block max by lane shuffles.
//  2. solve    first Dykstra cycle in log2 space (max-shifted log-sum-exp on
//              rows and columns, robust for any tau); every later cycle in
//              scaling form.  With Y = X + Q the cycle is Y += a_i + b_j and
//              X = min(Y, 0), so keeping P = 2^Y (fixed after cycle 1), a row
//              scale U_i and a column scale V_j, one cycle is
//                 E_ij = min(P_ij V_j U_i, 1)     (= exp(X_ij))          (C3)
//                 a_i  = N / sum_j E_ij,           U_i *= a_i            (C1)
//                 b_j  = N / sum_i E_ij a_i,       V_j *= b_j            (C2)
//              i.e. 4 fp32 VALU ops per element -- mul, mul with the clamp
//              output modifier (the clip), add, fma -- and no transcendental
//              per element.  Rows live in lanes; the column sums of blocks
//              spread over several lanes meet in a DPP butterfly
//              (reduce-scatter, per-owner update of V), and the owners' new
//              V goes back to every lane through LDS.
//  3. export   M >= 8: each block's record -- its log2 row and column offsets
//              with the final scales folded in, and its score scale -- goes
//              to LDS, from which S = min(P V U, 1) = min(2^(scale |W| +
//              row + col), 1) is rebuilt row by row with |W| (read again)
//              by the rounding, which also writes frac_out when asked; S
//              never goes to memory.  M = 4: S itself goes to the LDS
//              staging of the rounding.
//  4. round    blocks are staged in LDS one row and one column per
//              lane.  The greedy over the (S desc, index asc) order is computed
//              as its equivalent fixed point: accepted = {key >= phi_i and
//              key >= theta_j} where phi_i / theta_j is the N-th largest key
//              of row i / column j among entries passing the other side's
//              thresholds.  Alternating the two updates from "everything
//              allowed" climbs monotonically to that unique fixed point (the
//              stable b-matching of the key order), so each step is a
//              per-lane walk over a register-sorted row or column plus a
//              32x32 bit-matrix transpose by lane shuffles.
//  5. repair   local search and fill on the few deficient rows/columns, each
//              move an exact argmax over packed (fp32 score, index) keys.
//  6. pack     row bit masks are OR-combined across the blocks of a word and
//              stored as uint32 words.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tsenor_internal.h"

namespace tsenor {
namespace {

// Solve layout: each lane holds an R x CW tile (R rows, CW = M/H columns) of
// one block, a block spans L = (M/R)*H lanes and a group is BPG = 64/L
// blocks.  Row sums are completed across the H lanes of a row group by DPP
// moves, column sums across the G = M/R row groups by a DPP reduce-scatter.
template <int M> struct Geo;
template <> struct Geo<4> { static constexpr int R = 2, H = 1; };
template <> struct Geo<8> { static constexpr int R = 8, H = 1; };
template <> struct Geo<16> { static constexpr int R = 4, H = 1; };
template <> struct Geo<32> { static constexpr int R = 8, H = 2; };
template <int M> constexpr int kR = Geo<M>::R;
template <int M> constexpr int kH = Geo<M>::H;
template <int M> constexpr int kCW = M / kH<M>;         // columns per lane
template <int M> constexpr int kG = M / kR<M>;           // row groups per block
template <int M> constexpr int kL = kG<M> * kH<M>;       // lanes per block
template <int M> constexpr int kBPG = kWave / kL<M>;     // blocks per group
static_assert(kBPG<32> * 32 % 32 == 0 && kBPG<16> * 16 % 32 == 0, "groups cover whole words");

// Column sums of blocks spread over several lanes (M = 16: 4 lanes per block,
// one row group each; M = 32: 8 lanes per block, 4 row groups x 2 row halves)
// meet by a DPP butterfly in registers (reduce-scatter: each lane ends up
// owning 4 columns), and the owners' new column scales go back to every lane
// through LDS.  Every cross-lane step of the butterfly is one DPP move inside
// an aligned group of 4 or 8 lanes.  M = 32: the two halves of a row pair up
// by one pattern, and the 4 row groups by two further patterns g1, g0 that
// commute with it.  Block lane lb = bits (b2 b1 b0): g1 = b2, g0 = b0^b2,
// h = b1^b2; row halves pair as lane^2 (quad_perm [2,3,0,1]), g1 as lane^7
// (row_half_mirror), g0 as lane^1.  M = 16: g = lb, so g1 = b1 pairs as
// lane^2 and g0 = b0 as lane^1.  Row group g = 2*g1 + g0 holds rows g*R ..
// g*R+R-1, and its CW = 16 columns are stored with the 4-column quads
// permuted: register quad k holds column quad k ^ g.  Two lanes that differ
// only in g1 then hold each other's register quads 0-1 in their quads 2-3,
// and lanes that differ only in g0 hold each other's quad 0 in quad 1, so the
// reduce-scatter of the column sums, and in cycle 1 the all-gather of the
// column maxima and sums, are uniform DPP operations.
template <int M> constexpr bool kBfly = (M == 32 || M == 16);
struct Lanes32 {
    static constexpr int kRow = 0x4E, kG1 = 0x141, kG0 = 0xB1;
    __device__ static int g(int lb) { return 2 * (lb >> 2) + ((lb ^ (lb >> 2)) & 1); }
    __device__ static int h(int lb) { return ((lb >> 1) ^ (lb >> 2)) & 1; }
};
template <int M> constexpr int kCtlG1 = (M == 32) ? Lanes32::kG1 : 0x4E;
template <int M> constexpr int kCtlG0 = Lanes32::kG0;
// The same two pairings as ds_swizzle patterns (bit-mask mode: and 0x1F, or 0,
// xor k within each 32 lanes): g1 is lane^7 at M = 32 (row_half_mirror inside
// an aligned 8-lane group) and lane^2 at M = 16; g0 is lane^1.
template <int M> constexpr int kSwzG1 = 0x1F | (((M == 32) ? 7 : 2) << 10);
constexpr int kSwzG0 = 0x1F | (1 << 10);
static_assert(kCW<32> == 16 && kG<32> == 4 && kH<32> == 2, "the butterfly's tile shape");
static_assert(kCW<16> == 16 && kG<16> == 4 && kH<16> == 1, "the butterfly's tile shape");
// Blocks whose cycle-1 kernel reaches below 2^kDeepLog2 rescale in log2 space.
// fp32 emulation of the iteration against the fp64 oracle: folding in the
// linear domain stays within 5e-6 while the minimum is above ~-115 and fails
// beyond the normal range (-126).
constexpr float kDeepLog2 = -100.0f;

// The butterfly tiles broadcast each cycle's new column scales through LDS:
// one row of M floats per block of the wave.
template <int M> constexpr int dyk_lds_floats() { return kBfly<M> ? kBPG<M> * M : 0; }
static_assert(kL<8> == 1, "blocks of one lane need no column exchange");
// M = 4: the rows of a block are spread over G = 4 / R lanes (all four
// columns each), so a wave holds 64 / G blocks and a 2:4 matrix fills G times
// the waves of one lane per block.  The column totals meet in log2(G)
// exchanges (lane ^ 1, lane ^ 2), after which every lane of the block holds
// the same totals (each level adds a + b in one lane and b + a in its
// partner) and updates all four column scales itself.
template <int M> constexpr bool kPairCols = (M == 4);
static_assert(kH<4> == 1 && kCW<4> == 4 && (kG<4> == 2 || kG<4> == 4), "the layout of M = 4");
// Totals over the G lanes of an M = 4 block for each column.
template <int G, bool MAXOP>
__device__ __forceinline__ void col_pair_allreduce(float (&x)[4]);
// Rounding staging: block q of a pass at q*kStageBlk, row i at i*(M+4); the
// block stride is M (mod 32) apart so that column reads of the blocks that
// share a 32-lane half hit distinct banks.
template <int M> constexpr int kStageRow = (M == 4) ? 4 : M + 4;
template <int M> constexpr int kStageBlk = (M == 4) ? 16 : M * (M + 4) + (M < 32 ? M : 0);
// Blocks the staging area holds: one rounding pass (64 / M blocks), except
// for M = 4, where the solve exports the S of its whole group (32 blocks, two
// passes) straight into LDS; larger M rebuild S pass by pass from per-block
// records (kRec) instead.
template <int M> constexpr bool kStageInLds = (M == 4);
template <int M> constexpr int kStaged = kStageInLds<M> ? kBPG<M> : kWave / M;
// |W| for the local search follows the staging area: block q, row i at
// (q*M + i)*(M+1); then one word per lane for the rows of the current mask.
template <int M> constexpr int rnd_lds_floats() {
    return kStaged<M> * kStageBlk<M> + (kWave / M) * M * (M + 1) + kWave;
}
template <int M> constexpr int solve_round_floats() {
    return dyk_lds_floats<M>() > rnd_lds_floats<M>() ? dyk_lds_floats<M>() : rnd_lds_floats<M>();
}
// M >= 8: the solve leaves a record of each block of the group for the
// rounding, which rebuilds S from it and |W| instead of reading S back from
// memory: the final log2 row offsets (M floats), column offsets (M) and the
// score scale, S_ij = min(2^(scale |W_ij| + row_i + col_j), 1).  The records
// follow the solve's and the rounding's areas and live from the end of the
// solve to the end of the group's rounding.
// Records of M >= 16 are padded to a multiple of 4 floats so that the column
// offsets are read 16 bytes at a time; M = 8 keeps 2M + 1 (its 64 records
// would otherwise push a workgroup's LDS past what four waves per SIMD allow).
template <int M> constexpr int kRec = (M >= 16) ? 2 * M + 4 : 2 * M + 1;
template <int M> constexpr int rec_floats() { return kStageInLds<M> ? 0 : kBPG<M> * kRec<M>; }
template <int M> constexpr int lds_floats() { return solve_round_floats<M>() + rec_floats<M>(); }
static_assert(solve_round_floats<32>() % 4 == 0 && solve_round_floats<16>() % 4 == 0,
              "the records of M >= 16 start 16-byte aligned");

template <int M> constexpr uint32_t kFull = (M == 32) ? 0xFFFFFFFFu : ((1u << M) - 1u);
// Waves per SIMD the solve+round kernels are built for.  The register budget
// of the fused path sits close to these steps (512 / waves registers per
// lane); pinning the target makes the allocator fit it rather than silently
// drop a wave when unrelated code changes.
template <int M> constexpr int kSolveWaves = (M <= 4) ? 8 : (M == 8) ? 4 : (M == 16) ? 3 : 2;

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float lg2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float rcpf(float x) { return __builtin_amdgcn_rcpf(x); }

// ---------------------------------------------------------------- gather
// Native vector types for the 8/16-byte loads of W.  The loads are ordinary
// cached loads: a group's rows are read again by its rounding and, for deep
// blocks, at every fold of the solve, and those reads find part of them in
// L2 (non-temporal loads measured 6.5% slower at tau 200, 1.8% at 4:8 and
// 0.4% at 16:32).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// |W| of M consecutive elements starting at element offset `off`, as fp32.
template <int M, bool BF16>
__device__ __forceinline__ void load_abs_row(const void* W, int64_t off, bool vec, float (&out)[M]) {
    if constexpr (BF16) {
        const uint16_t* p = static_cast<const uint16_t*>(W) + off;
        if (vec) {
            if constexpr (M >= 8) {
#pragma unroll
                for (int q = 0; q < M / 8; ++q) {
                    const u32x4 v = reinterpret_cast<const u32x4*>(p)[q];
                    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int h = 0; h < 4; ++h) {
                        out[8 * q + 2 * h] = __uint_as_float((w[h] & 0x7FFFu) << 16);
                        out[8 * q + 2 * h + 1] = __uint_as_float(w[h] & 0x7FFF0000u);
                    }
                }
            } else {
                const u32x2 v = *reinterpret_cast<const u32x2*>(p);
                out[0] = __uint_as_float((v.x & 0x7FFFu) << 16);
                out[1] = __uint_as_float(v.x & 0x7FFF0000u);
                out[2] = __uint_as_float((v.y & 0x7FFFu) << 16);
                out[3] = __uint_as_float(v.y & 0x7FFF0000u);
            }
        } else {
#pragma unroll
            for (int j = 0; j < M; ++j) out[j] = __uint_as_float((uint32_t)(p[j] & 0x7FFFu) << 16);
        }
    } else {
        const float* p = static_cast<const float*>(W) + off;
        if (vec) {
#pragma unroll
            for (int q = 0; q < M / 4; ++q) {
                const f32x4 v = reinterpret_cast<const f32x4*>(p)[q];
                out[4 * q] = fabsf(v.x);
                out[4 * q + 1] = fabsf(v.y);
                out[4 * q + 2] = fabsf(v.z);
                out[4 * q + 3] = fabsf(v.w);
            }
        } else {
#pragma unroll
            for (int j = 0; j < M; ++j) out[j] = fabsf(p[j]);
        }
    }
}

// In place: quad k of x becomes quad k ^ sw (sw in 0..3), by two conditional
// swaps (the loads stay contiguous; the permutation is lane dependent).
__device__ __forceinline__ void permute_quads(float (&x)[16], int sw) {
    const bool s2 = (sw & 2) != 0, s1 = (sw & 1) != 0;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const float lo = x[c], hi = x[c + 8];
        x[c] = s2 ? hi : lo;
        x[c + 8] = s2 ? lo : hi;
    }
#pragma unroll
    for (int k = 0; k < 16; k += 8)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const float lo = x[k + c], hi = x[k + c + 4];
            x[k + c] = s1 ? hi : lo;
            x[k + c + 4] = s1 ? lo : hi;
        }
}

// M consecutive fp32 values (16-byte loads when `vec`).
template <int M>
__device__ __forceinline__ void load_row_f32(const float* p, bool vec, float (&out)[M]) {
    if (vec) {
#pragma unroll
        for (int q = 0; q < M / 4; ++q) {
            const float4 v = reinterpret_cast<const float4*>(p)[q];
            out[4 * q] = v.x; out[4 * q + 1] = v.y; out[4 * q + 2] = v.z; out[4 * q + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int j = 0; j < M; ++j) out[j] = p[j];
    }
}

template <int M>
__device__ __forceinline__ float tree_sum(const float (&v)[M]) {
    float s[M / 2];
#pragma unroll
    for (int j = 0; j < M / 2; ++j) s[j] = v[2 * j] + v[2 * j + 1];
#pragma unroll
    for (int w = M / 4; w >= 1; w >>= 1) {
#pragma unroll
        for (int j = 0; j < w; ++j) s[j] = s[2 * j] + s[2 * j + 1];
    }
    return s[0];
}

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Totals over the two lanes of a tile row (M = 32) for a pair of slots: the
// partner lane holds the same two rows in the opposite slots, so slot 0 here
// meets the partner's slot 1.
template <bool MAXOP>
__device__ __forceinline__ void row_pair_allreduce(float& x0, float& x1) {
    static_assert(kBfly<32> && kH<32> == 2, "row halves pair by the butterfly layout");
    const float y0 = dpp_mov<Lanes32::kRow>(x1), y1 = dpp_mov<Lanes32::kRow>(x0);
    x0 = MAXOP ? fmaxf(x0, y0) : x0 + y0;
    x1 = MAXOP ? fmaxf(x1, y1) : x1 + y1;
}
// Totals over the H lanes of a tile row for every slot of a lane.
template <int M, bool MAXOP>
__device__ __forceinline__ void row_allreduce_slots(float (&x)[kR<M>]) {
    static_assert(kH<M> == 1 || (kH<M> == 2 && kR<M> % 2 == 0), "H");
    if constexpr (kH<M> == 2) {
#pragma unroll
        for (int r = 0; r < kR<M>; r += 2) row_pair_allreduce<MAXOP>(x[r], x[r + 1]);
    }
}

// Value of x in the partner lane given by a ds_swizzle pattern.  The move
// runs on the LDS crossbar (no LDS memory), so it takes no VALU issue slot;
// the add that consumes it is a plain VALU op.
template <int PAT>
__device__ __forceinline__ float swz(float x) {
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), PAT));
}

// Register-level grouping point for the first K values of x: every write of
// them precedes it and every later read follows it.  Emits no instruction.
// The M = 16 column chain uses it to issue its adds, DPP adds and reciprocals
// as three back-to-back runs: each switch between plain VALU instructions and
// DPP or transcendental ones costs the wave issue time, and left alone the
// scheduler interleaves the three kinds (8:16 -0.7%; at M = 32 it measured
// the same or slower and is not used there).
template <int K>
__device__ __forceinline__ void group_fence(float (&x)[16]) {
    static_assert(K == 4 || K == 8, "group size");
    if constexpr (K == 8)
        asm volatile("" : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]),
                          "+v"(x[5]), "+v"(x[6]), "+v"(x[7]));
    else
        asm volatile("" : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]));
}

// Butterfly (M = 16 and 32): on return x[0..3] of every lane hold the column
// totals (max or sum over the 4 row groups) of those register columns; each
// column is owned by exactly one lane of the block per row half.  The eight
// partner values of the first level are fetched together (ds_swizzle), then
// combined: the same operands and order as a DPP add per column, but the
// moves take no VALU issue slot (2-6% faster in the Dykstra cycle, whose
// serial tail this is).  The second level's four adds are DPP (a further
// 1-4%: one LDS round trip fewer in the tail).
template <int M, bool MAXOP>
__device__ __forceinline__ void col_reduce_scatter(float (&x)[16]) {
    float y[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) y[c] = swz<kSwzG1<M>>(x[c + 8]);
#pragma unroll
    for (int c = 0; c < 8; ++c) x[c] = MAXOP ? fmaxf(x[c], y[c]) : x[c] + y[c];
    if constexpr (M == 16) group_fence<8>(x);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const float z = dpp_mov<kCtlG0<M>>(x[c + 4]);
        x[c] = MAXOP ? fmaxf(x[c], z) : x[c] + z;
    }
    if constexpr (M == 16) group_fence<4>(x);
}
template <int G, bool MAXOP>
__device__ __forceinline__ void col_pair_allreduce(float (&x)[4]) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const float y = dpp_mov<0xB1>(x[c]);  // lane ^ 1
        x[c] = MAXOP ? fmaxf(x[c], y) : x[c] + y;
    }
    if constexpr (G == 4) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const float y = dpp_mov<0x4E>(x[c]);  // lane ^ 2
            x[c] = MAXOP ? fmaxf(x[c], y) : x[c] + y;
        }
    }
}

// Inverse: from the owners' x[0..3], every lane gets x[0..15] for its columns.
template <int M>
__device__ __forceinline__ void col_all_gather(float (&x)[16]) {
#pragma unroll
    for (int c = 0; c < 4; ++c) x[c + 4] = dpp_mov<kCtlG0<M>>(x[c]);
#pragma unroll
    for (int c = 0; c < 8; ++c) x[c + 8] = dpp_mov<kCtlG1<M>>(x[c]);
}

// Register-level ordering point: an empty asm that "reads and writes" a and
// b.  Every later use of a/b waits for it and every earlier write of a/b
// precedes it.  Emits no instruction.
template <int CW>
__device__ __forceinline__ void order_fence(float (&a)[CW], float (&b)[CW]) {
#pragma unroll
    for (int c = 0; c < CW; c += 4)
        asm volatile("" : "+v"(a[c]), "+v"(a[c + 1]), "+v"(a[c + 2]), "+v"(a[c + 3]),
                          "+v"(b[c]), "+v"(b[c + 1]), "+v"(b[c + 2]), "+v"(b[c + 3]));
}

// Orders this wave's LDS accesses at a point, for the compiler only.  Every
// kernel in this file runs one-wave workgroups, and a wave's LDS instructions
// execute in issue order, so a read issued after a write (by any lane of the
// wave) observes it with no barrier and no wait; the empty asm keeps the
// compiler from moving LDS accesses across the point.  Global memory is still
// ordered by __syncthreads().
__device__ __forceinline__ void wave_lds_fence() { asm volatile("" ::: "memory"); }

// Wave priority.  Two waves share a SIMD in the fused kernels, and the VALU
// reaches its full rate only while both issue.  Most of a Dykstra cycle is a
// long run of independent fp32 products that can issue at any time; its row
// and column totals are short serial chains (cross-lane move -> reciprocal ->
// product) whose latency the wave cannot hide by itself.  Raising the
// priority of a wave inside such a chain lets its instructions issue as soon
// as they are ready, and the partner wave's bulk work fills the gaps.  The
// same holds for the rounding (sorts, reductions, branches) against the
// partner's cycles.  Measured on the 16:32 and 8:16 workloads: 12-17% less
// time per launch, results unchanged.
constexpr int kPrioChain = 2;  // serial chains of a cycle
constexpr int kPrioRound = 1;  // rounding and repair
template <int P>
__device__ __forceinline__ void set_prio() { __builtin_amdgcn_s_setprio(P); }
// The rounding's LDS ordering points: the wave-level fence for M <= 8, a
// workgroup barrier for M >= 16 (each measured the faster of the two there).
template <int M>
__device__ __forceinline__ void rnd_sync() {
    if constexpr (M <= 8) wave_lds_fence();
    else __syncthreads();
}

// ---------------------------------------------------------------- solve
// Dykstra for the group's blocks.  M >= 8: leaves each block's record (see
// kRec) in LDS for the rounding, which rebuilds S from it.  M = 4: writes S
// into the rounding's LDS staging, and to job.frac when requested.
template <int M, bool BF16>
__device__ __forceinline__ void dykstra_group(const MatJob& job, const Params& prm, int64_t br,
                                              int64_t bc0, float* __restrict__ lds) {
    constexpr int R = kR<M>, H = kH<M>, CW = kCW<M>, L = kL<M>;
    // M = 32: an opaque lane, so that addresses derived from it are rebuilt
    // per group instead of being hoisted out of the kernel's group loop, where
    // they would stay live (and cost registers) through the whole solve.
    int lane = threadIdx.x;
    if constexpr (M >= 32) asm volatile("" : "+v"(lane));
    const int blk = lane / L, lb = lane % L;
    int g = lb / H, h = lb % H;
    if constexpr (M == 32) { g = Lanes32::g(lb); h = Lanes32::h(lb); }
    const int sw = kBfly<M> ? g : 0;  // register quad k holds column quad k ^ sw
    // Slot k of the lane's tile holds tile row k ^ rsw: the two lanes of a
    // tile row (H = 2) hold each pair of rows in opposite slot order, so one
    // exchange of partial sums and one reciprocal serve two rows.
    const int rsw = (H == 2) ? h : 0;
    const int64_t nbc = job.cols / M;
    const int64_t bc = bc0 + blk;
    const bool valid = bc < nbc;
    const float fN = (float)job.N;
    const float log2N = log2f(fN);
    const bool vec = job.aligned != 0;
    const int64_t row0 = br * M + g * R;      // first matrix row of this lane's tile
    const int64_t col0 = bc * M + h * CW;     // first matrix column of this lane's tile
    // Lane's part of the LDS behind the column-scale exchange (free during
    // the solve): the block's log2 row offsets (R), column offsets (CW) and
    // score scale, entry k of the lane at k * kWave, so that log2 P = scale
    // |W| + row offset + column offset holds through every rescaling below.
    // Kept for every block at M >= 8 (the export's record is made from it),
    // for deep blocks only at M = 4.
    float* offs = lds + dyk_lds_floats<M>() + lane;
    static_assert(dyk_lds_floats<M>() + kWave * (R + CW + 1) <= solve_round_floats<M>(),
                  "the offsets fit the LDS");

    float P[R][CW];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if (valid) {
            load_abs_row<CW, BF16>(job.W, (row0 + (r ^ rsw)) * job.ld + col0, vec, P[r]);
            if constexpr (kBfly<M>) permute_quads(P[r], sw);
        } else {
#pragma unroll
            for (int c = 0; c < CW; ++c) P[r][c] = 0.f;
        }
    }
    // scores What = A / max(A); X = tau * What in log2 units
    float m = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < CW; ++c) m = fmaxf(m, P[r][c]);
#pragma unroll
    for (int s = 1; s < L; s <<= 1) m = fmaxf(m, __shfl_xor(m, s));
    const float scale = (m > 0.f) ? prm.tau_log2e / m : 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < CW; ++c) P[r][c] *= scale;

    bool deep;
    float rho[R];  // cycle 1's log2 row offsets
    // ---- cycle 1 in log2 space (Q = 0, so no clip enters C1/C2) ----
    {  // C1: row max, then row sum of 2^(x - max)
        float mx[R], sm[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            mx[r] = P[r][0];
#pragma unroll
            for (int c = 1; c < CW; ++c) mx[r] = fmaxf(mx[r], P[r][c]);
        }
        row_allreduce_slots<M, true>(mx);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float e[CW];
#pragma unroll
            for (int c = 0; c < CW; ++c) e[c] = ex2(P[r][c] - mx[r]);
            sm[r] = tree_sum<CW>(e);
        }
        row_allreduce_slots<M, false>(sm);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            rho[r] = log2N - mx[r] - lg2(sm[r]);
#pragma unroll
            for (int c = 0; c < CW; ++c) P[r][c] += rho[r];
        }
    }
    {  // C2: column max, then column sum of 2^(x - max)
        float part[CW], cmax[CW], csum[CW];
#pragma unroll
        for (int c = 0; c < CW; ++c) {
            float v = P[0][c];
#pragma unroll
            for (int r = 1; r < R; ++r) v = fmaxf(v, P[r][c]);
            part[c] = v;
        }
        if constexpr (kBfly<M>) {
#pragma unroll
            for (int c = 0; c < CW; ++c) cmax[c] = part[c];
            col_reduce_scatter<M, true>(cmax);
            col_all_gather<M>(cmax);
        } else if constexpr (kPairCols<M>) {
#pragma unroll
            for (int c = 0; c < CW; ++c) cmax[c] = part[c];
            col_pair_allreduce<kG<M>, true>(cmax);
        } else {
#pragma unroll
            for (int c = 0; c < CW; ++c) cmax[c] = part[c];
        }
#pragma unroll
        for (int c = 0; c < CW; ++c) {
            float v = 0.f;
#pragma unroll
            for (int r = 0; r < R; ++r) v += ex2(P[r][c] - cmax[c]);
            part[c] = v;
        }
        if constexpr (kBfly<M>) {
#pragma unroll
            for (int c = 0; c < CW; ++c) csum[c] = part[c];
            col_reduce_scatter<M, false>(csum);
            col_all_gather<M>(csum);
        } else if constexpr (kPairCols<M>) {
#pragma unroll
            for (int c = 0; c < CW; ++c) csum[c] = part[c];
            col_pair_allreduce<kG<M>, false>(csum);
        } else {
#pragma unroll
            for (int c = 0; c < CW; ++c) csum[c] = part[c];
        }
        // C3 of cycle 1 is carried by P = 2^Y: X = min(Y, 0) appears as min(P V U, 1)
        float b[CW];
#pragma unroll
        for (int c = 0; c < CW; ++c) b[c] = log2N - cmax[c] - lg2(csum[c]);
        float ymin = 0.f;
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int c = 0; c < CW; ++c) {
                P[r][c] += b[c];
                ymin = fminf(ymin, P[r][c]);
            }
        // A block is "deep" when its kernel spans more than fp32 can hold
        // next to O(1) values (tau * log2(e) beyond ~100): Y = scale * |W| +
        // row offset + column offset, and the offsets and the scale are kept
        // so that rescaling happens in log2 space.
        int dflag = (ymin < kDeepLog2) ? 1 : 0;
#pragma unroll
        for (int s = 1; s < L; s <<= 1) dflag |= __shfl_xor(dflag, s);
        deep = dflag != 0;
        if (!kStageInLds<M> || deep) {
#pragma unroll
            for (int r = 0; r < R; ++r) offs[r * kWave] = rho[r];
#pragma unroll
            for (int c = 0; c < CW; ++c) offs[(R + c) * kWave] = b[c];
            offs[(R + CW) * kWave] = scale;
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int c = 0; c < CW; ++c) P[r][c] = ex2(P[r][c]);
    }

    // ---- cycles 2..T in scaling form ----
    float V[CW], U[R];
#pragma unroll
    for (int c = 0; c < CW; ++c) V[c] = 1.f;
#pragma unroll
    for (int r = 0; r < R; ++r) U[r] = 1.f;
    // Per cycle: row r's total s_r gives the row factor a_r = N / s_r (U_r <-
    // U_r a_r) and the column totals of E a_r give the column factors.  With
    // H = 1 the factor enters as (U_r N) (1 / s_r) and the column totals as
    // sums of E / s_r, i.e. divided by N, so that each column factor is one
    // reciprocal (V <- V / cacc); the M = 32 tile keeps a_r = N (1 / s_r),
    // which measured faster there.
    for (int it = 1; it < prm.iters; ++it) {
        float cacc[CW];
        if constexpr (H == 1) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                float e[CW], acc[4];
#pragma unroll
                for (int c = 0; c < CW; ++c) {
                    // E = min(P V U, 1): the clamp folds into the second multiply
                    e[c] = __builtin_amdgcn_fmed3f((P[r][c] * V[c]) * U[r], 0.0f, 1.0f);
                    acc[c & 3] = (c < 4) ? e[c] : acc[c & 3] + e[c];
                }
                set_prio<kPrioChain>();
                const float a = rcpf((acc[0] + acc[1]) + (acc[2] + acc[3]));
                set_prio<0>();
                U[r] = (U[r] * fN) * a;
#pragma unroll
                for (int c = 0; c < CW; ++c) cacc[c] = (r == 0) ? e[c] * a : fmaf(e[c], a, cacc[c]);
                // Keep one row's temporaries live at a time: left alone, the
                // instruction selector hoists every row's products and spills
                // the tile.  The empty asm claims to update cacc and V, so this
                // row's column updates complete before, and the next row's
                // products start after, this point.  No instruction is emitted.
                order_fence<CW>(cacc, V);
            }
        } else {
            // Two slots at a time (see rsw): slot r here and slot r + 1 of the
            // partner lane hold the same row, so the row total of slot r is one
            // exchange away, and the factor of slot r + 1 is the partner's.
#pragma unroll
            for (int r = 0; r < R; r += 2) {
                float e0[CW], e1[CW], acc0[4], acc1[4];
#pragma unroll
                for (int c = 0; c < CW; ++c) {
                    e0[c] = __builtin_amdgcn_fmed3f((P[r][c] * V[c]) * U[r], 0.0f, 1.0f);
                    acc0[c & 3] = (c < 4) ? e0[c] : acc0[c & 3] + e0[c];
                }
#pragma unroll
                for (int c = 0; c < CW; ++c) {
                    e1[c] = __builtin_amdgcn_fmed3f((P[r + 1][c] * V[c]) * U[r + 1], 0.0f, 1.0f);
                    acc1[c & 3] = (c < 4) ? e1[c] : acc1[c & 3] + e1[c];
                }
                set_prio<kPrioChain>();
                const float rs = ((acc0[0] + acc0[1]) + (acc0[2] + acc0[3])) +
                                 dpp_mov<Lanes32::kRow>((acc1[0] + acc1[1]) + (acc1[2] + acc1[3]));
                // The partner's factor is formed from its reciprocal moved here:
                // N * dpp(r) is one DPP multiply, where dpp(N * r) was a multiply,
                // a DPP move and a wait state (same value; 16:32 -0.5%, tau 200
                // -1.3%).
                const float r0 = rcpf(rs);
                const float a0 = fN * r0, a1 = fN * dpp_mov<Lanes32::kRow>(r0);
                set_prio<0>();
                U[r] *= a0;
                U[r + 1] *= a1;
                // Columns in the order k ^ 7 (each column's update stands
                // alone, so no result changes): with it the allocation puts
                // no v_fmac of these updates with its three operands (total,
                // E, factor) in one VGPR bank (register number mod 4).  Such
                // an instruction issues at 0.57x the rate of one with spread
                // operands; the ascending order gave 11-13 of them per cycle,
                // 1-2% of a whole 16:32 launch.
#pragma unroll
                for (int k = 0; k < CW; ++k) {
                    const int c = k ^ 7;
                    cacc[c] = (r == 0) ? e0[c] * a0 : fmaf(e0[c], a0, cacc[c]);
                    cacc[c] = fmaf(e1[c], a1, cacc[c]);
                }
                order_fence<CW>(cacc, V);  // as above, per pair of slots
            }
        }
        // Scale guard.  After cycle 1 every row/column factor lies in
        // [1/M, M], so checking every 4th cycle against 2^+-40 keeps P V U,
        // U and V far inside the fp32 range.
        bool bad = false;
        if constexpr (L == 1 || kPairCols<M>) {
            if constexpr (kPairCols<M>) {  // both lanes of the block get the column totals
                set_prio<kPrioChain>();
                col_pair_allreduce<kG<M>, false>(cacc);
                set_prio<0>();
            }
#pragma unroll
            for (int c = 0; c < CW; ++c) V[c] = V[c] * rcpf(cacc[c]);
            if ((it & 3) == 0) {
                float lo = V[0], hi = V[0];
#pragma unroll
                for (int c = 1; c < CW; ++c) { lo = fminf(lo, V[c]); hi = fmaxf(hi, V[c]); }
                bad = !(lo >= 0x1p-40f && hi <= 0x1p40f);
            }
        } else {
            static_assert(kBfly<M>, "blocks of several lanes use the butterfly");
            // column totals by butterfly; each owner rescales its 4 columns
            // (column quad g of its half) and the new scales are gathered back
            // (a serial chain to the end of the cycle: raised priority)
            set_prio<kPrioChain>();
            col_reduce_scatter<M, false>(cacc);
            float rc[16];
#pragma unroll
            for (int c = 0; c < 4; ++c) rc[c] = rcpf(cacc[c]);
            if constexpr (M == 16) group_fence<4>(rc);  // the 4 reciprocals back to back
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                if constexpr (H == 1) V[c] = V[c] * rc[c];
                else V[c] = V[c] * (fN * rc[c]);
            }
            if ((it & 3) == 0) {
                if constexpr (M == 32) {
                    // one range test of the extremes instead of one per scale
                    // (-1% at 16:32; at M = 16 the per-scale tests measured
                    // 2.7% faster and stay)
                    float vlo = V[0], vhi = V[0];
#pragma unroll
                    for (int c = 1; c < 4; ++c) { vlo = fminf(vlo, V[c]); vhi = fmaxf(vhi, V[c]); }
                    bad = !(vlo >= 0x1p-40f && vhi <= 0x1p40f);
                } else {
#pragma unroll
                    for (int c = 0; c < 4; ++c) bad |= !(V[c] >= 0x1p-40f && V[c] <= 0x1p40f);
                }
            }
            {
                // The new scales reach the other lanes through LDS (one 16-byte
                // write per owner, three reads per lane) rather than by 12 DPP
                // moves: each DPP operation costs the SIMD far more issue time
                // than its one slot, while LDS traffic leaves the VALU free.
                float* vb = lds + blk * M + h * CW;
                *reinterpret_cast<float4*>(vb + 4 * g) = make_float4(V[0], V[1], V[2], V[3]);
                wave_lds_fence();
#pragma unroll
                for (int k = 1; k < 4; ++k) {
                    const float4 v = *reinterpret_cast<const float4*>(vb + 4 * (k ^ sw));
                    V[4 * k] = v.x; V[4 * k + 1] = v.y; V[4 * k + 2] = v.z; V[4 * k + 3] = v.w;
                }
                set_prio<0>();
            }
        }
        if ((it & 3) != 0) continue;
        if constexpr (M == 32 || M == 8) {  // (4:8 -0.2%)
            float ulo = U[0], uhi = U[0];
#pragma unroll
            for (int r = 1; r < R; ++r) { ulo = fminf(ulo, U[r]); uhi = fmaxf(uhi, U[r]); }
            bad |= !(ulo >= 0x1p-40f && uhi <= 0x1p40f);
        } else {
#pragma unroll
            for (int r = 0; r < R; ++r) bad |= !(U[r] >= 0x1p-40f && U[r] <= 0x1p40f);
        }
        bad = bad && valid;
        if (__builtin_expect(__ballot(bad) != 0ull, 0)) {
            // Rare: fold the scales into the kernel (scales <- 1), so that
            // P U V is unchanged but the scales stay far from the fp32 range
            // limits.  Deep blocks fold in log2 space (row offsets += log2 U,
            // column offsets += log2 V) and rebuild P = 2^Y from |W|, which
            // is read again: folding into P itself would lose the entries of
            // P that underflow, which can still grow to O(1) later.  A block
            // folds only when one of its lanes is valid, and then all are.
            int f = bad ? 1 : 0;
#pragma unroll
            for (int s = 1; s < L; s <<= 1) f |= __shfl_xor(f, s);
            if (f && deep) {
                // The tile's origin is rebuilt here from an opaque lane id, so
                // that its addresses are not held in registers through the
                // solve; the offsets stay in LDS and are read where used.
                int ln = threadIdx.x;
                asm volatile("" : "+v"(ln));
                const int lbf = ln % L;
                int gf = lbf / H, hf = lbf % H;
                if constexpr (M == 32) { gf = Lanes32::g(lbf); hf = Lanes32::h(lbf); }
                const int swf = kBfly<M> ? gf : 0, rswf = (H == 2) ? hf : 0;
                const int64_t r0 = br * M + gf * R, c0 = (bc0 + ln / L) * M + hf * CW;
                float* of = lds + dyk_lds_floats<M>() + ln;
                const float sc = of[(R + CW) * kWave];
#pragma unroll
                for (int c = 0; c < CW; ++c) of[(R + c) * kWave] += lg2(V[c]);
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const float ro = of[r * kWave] + lg2(U[r]);
                    of[r * kWave] = ro;
                    load_abs_row<CW, BF16>(job.W, (r0 + (r ^ rswf)) * job.ld + c0, vec, P[r]);
                    if constexpr (kBfly<M>) permute_quads(P[r], swf);
#pragma unroll
                    for (int c = 0; c < CW; ++c)
                        P[r][c] = ex2(fmaf(P[r][c], sc, ro) + of[(R + c) * kWave]);
                }
            } else if (f) {
                if constexpr (!kStageInLds<M>) {  // the offsets follow the fold
                    int ln = threadIdx.x;
                    asm volatile("" : "+v"(ln));
                    float* of = lds + dyk_lds_floats<M>() + ln;
#pragma unroll
                    for (int c = 0; c < CW; ++c) of[(R + c) * kWave] += lg2(V[c]);
#pragma unroll
                    for (int r = 0; r < R; ++r) of[r * kWave] += lg2(U[r]);
                }
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int c = 0; c < CW; ++c) P[r][c] = (P[r][c] * V[c]) * U[r];
            }
            if (f) {
#pragma unroll
                for (int c = 0; c < CW; ++c) V[c] = 1.f;
#pragma unroll
                for (int r = 0; r < R; ++r) U[r] = 1.f;
            }
        }
    }

    if constexpr (kStageInLds<M>) {
        // ---- export S = exp(X) = min(P U V, 1) into the rounding's staging ----
        const bool fvec = ((reinterpret_cast<uintptr_t>(job.frac) & 15u) == 0);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float s[CW];
#pragma unroll
            for (int c = 0; c < CW; ++c) s[c] = __builtin_amdgcn_fmed3f((P[r][c] * V[c]) * U[r], 0.0f, 1.0f);
            float* srow = lds + blk * kStageBlk<M> + (g * R + (r ^ rsw)) * kStageRow<M> + h * CW;
#pragma unroll
            for (int q = 0; q < CW / 4; ++q)
                *reinterpret_cast<float4*>(srow + 4 * (q ^ sw)) =
                    make_float4(s[4 * q], s[4 * q + 1], s[4 * q + 2], s[4 * q + 3]);
            if (job.frac != nullptr && valid) {
                float* frow = job.frac + (row0 + (r ^ rsw)) * job.cols + col0;
                if (fvec) {
#pragma unroll
                    for (int q = 0; q < CW / 4; ++q)
                        *reinterpret_cast<float4*>(frow + 4 * (q ^ sw)) =
                            make_float4(s[4 * q], s[4 * q + 1], s[4 * q + 2], s[4 * q + 3]);
                } else {
#pragma unroll
                    for (int c = 0; c < CW; ++c) frow[(c & 3) + 4 * ((c >> 2) ^ sw)] = s[c];
                }
            }
        }
    } else {
        // ---- the block's record: offsets with the final scales folded in ----
        // S = min(P U V, 1) = min(2^(scale |W| + row + col), 1), rebuilt by the
        // rounding.  Each row is written by the lanes of its h = 0 column half,
        // each column by the lanes of row group 0, the scale by lane 0.
        float* rb = lds + solve_round_floats<M>() + blk * kRec<M>;
        if (H == 1 || h == 0) {
#pragma unroll
            for (int r = 0; r < R; ++r) rb[g * R + (r ^ rsw)] = offs[r * kWave] + lg2(U[r]);
        }
        if (g == 0) {
#pragma unroll
            for (int c = 0; c < CW; ++c)
                rb[M + h * CW + 4 * ((c >> 2) ^ sw) + (c & 3)] = offs[(R + c) * kWave] + lg2(V[c]);
        }
        if (lb == 0) rb[2 * M] = offs[(R + CW) * kWave];
    }
}

// ---------------------------------------------------------------- round
// Sort key of the entry at position `pos` of a row (pos = column j) or of a
// column (pos = row r) with fractional value s.  High word: the fp32 bits of
// s plus one in the double's exponent field, so for s >= 0 the key is a
// positive normal double ordered like s; low word: M-1-pos.  In a row, idx =
// i*M + j ascends with j, and in a column idx = r*M + i ascends with r, so a
// larger key comes earlier in the (s descending, idx ascending) order.
template <int M>
__device__ __forceinline__ double make_key(float s, int pos, int zero) {
    const uint32_t hi = __float_as_uint(s + 0.0f) + 0x00100000u;  // -0 -> +0
    return __hiloint2double((int)hi, M - 1 - pos + zero);
}
// One-hot bit (1 << pos) of the entry a key was made from.
template <int M>
__device__ __forceinline__ uint32_t key_bit(double key) {
    return (1u << (M - 1)) >> ((uint32_t)__double2loint(key) & (uint32_t)(M - 1));
}

// Batcher's odd-even merge sort network (descending) on registers: 191
// compare-exchanges for 32 keys (bitonic needs 240).  Every index is a
// compile-time constant after unrolling.
template <int M>
__device__ __forceinline__ void sort_desc(double (&a)[M]) {
#pragma unroll
    for (int p = 1; p < M; p <<= 1)
#pragma unroll
        for (int k = p; k >= 1; k >>= 1)
#pragma unroll
            for (int j = k % p; j + k < M; j += 2 * k)
#pragma unroll
                for (int i = 0; i < k; ++i) {
                    const int x = i + j, y = i + j + k;
                    if (y < M && x / (2 * p) == y / (2 * p)) {
                        const double hi = fmax(a[x], a[y]), lo = fmin(a[x], a[y]);
                        a[x] = hi;
                        a[y] = lo;
                    }
                }
}

// Walk a sorted row (or column); pb[k] = bit of the entry at sorted position
// k.  Returns the bits of the entries at positions up to and including the
// N-th entry whose bit is set in `allowed` -- i.e. every entry whose key is
// >= the N-th largest allowed key -- or all entries if fewer than N are
// allowed (threshold "minus infinity").  c = (allowed entries seen) - N is
// negative exactly while the walk is inside the prefix, so its sign bit is
// the inclusion mask: no compares, selects or condition registers.
template <int M>
__device__ __forceinline__ uint32_t walk(const uint32_t (&pb)[M], uint32_t allowed, int N) {
    int c = -N;
    uint32_t m = 0u;
#pragma unroll
    for (int k = 0; k < M; ++k) {
        m |= pb[k] & (uint32_t)(c >> 31);
        c += __popc(allowed & pb[k]);
    }
    return m | ((uint32_t)(c >> 31) & kFull<M>);
}

// Same walk for a compile-time N: the first N positions always lie inside
// the prefix (fewer than N allowed entries precede any of them), so their
// bits are pre-ORed into `head` and only positions N..M-1 are walked.
template <int M, int N>
__device__ __forceinline__ uint32_t walk_tail(uint32_t head, const uint32_t (&tail)[M - N],
                                              uint32_t allowed) {
    int c = __popc(allowed & head) - N;
    uint32_t m = head;
#pragma unroll
    for (int k = 0; k < M - N; ++k) {
        m |= tail[k] & (uint32_t)(c >> 31);
        c += __popc(allowed & tail[k]);
    }
    return m | ((uint32_t)(c >> 31) & kFull<M>);
}

__device__ __forceinline__ constexpr uint32_t lowmask(int s) {
    return s == 16 ? 0x0000FFFFu
         : s == 8  ? 0x00FF00FFu
         : s == 4  ? 0x0F0F0F0Fu
         : s == 2  ? 0x33333333u
                   : 0x55555555u;
}

// Value of x in lane (lane ^ S), by DPP / permlane (no LDS traffic).
template <int S>
__device__ __forceinline__ uint32_t xor_lane(uint32_t x) {
    if constexpr (S == 1) return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, true);
    if constexpr (S == 2) return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, true);
    if constexpr (S == 4)  // row_half_mirror then quad_perm [3,2,1,0]
        return (uint32_t)__builtin_amdgcn_mov_dpp(
            __builtin_amdgcn_mov_dpp((int)x, 0x141, 0xF, 0xF, true), 0x1B, 0xF, 0xF, true);
    if constexpr (S == 8) return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x128, 0xF, 0xF, true);  // row_ror:8
    if constexpr (S == 16) {
        // permlane16_swap(x, x): result[0] holds lanes 0-15's x in lanes 16-31,
        // result[1] holds lanes 16-31's x in lanes 0-15.
        const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
        return (threadIdx.x & 16u) ? r[0] : r[1];
    }
    static_assert(S == 1 || S == 2 || S == 4 || S == 8 || S == 16, "xor distance");
    return x;
}

// Transpose of the M x M bit matrix held by each aligned group of M lanes
// (lane i: row i, bit j = column j) -> lane j gets column j (bit i = row i).
// Level s swaps the off-diagonal s x s sub-blocks between lanes i and i^s:
// the lower lane keeps its bits with (pos & s) == 0 and takes the partner's
// low-half bits rotated up by s; the upper lane the mirror image.  A rotation
// by s moves exactly those bits into place (no bit wraps into a kept
// position), so each level is one cross-lane move, one alignbit and one bfi.
template <int M, int S>
__device__ __forceinline__ uint32_t transpose_level(uint32_t x, uint32_t lane) {
    const uint32_t up = 0u - ((lane >> __builtin_ctz(S)) & 1u);
    const uint32_t keep = (lowmask(S) ^ up);            // own bits that stay
    const uint32_t y = xor_lane<S>(x);
    const uint32_t rot = __builtin_amdgcn_alignbit(y, y, up ? S : 32 - S);  // rotr(y, .)
    return (keep & x) | (~keep & rot & kFull<M>);
}

template <int M>
__device__ __forceinline__ uint32_t transpose_bits(uint32_t x, uint32_t lane) {
    if constexpr (M >= 32) x = transpose_level<M, 16>(x, lane);
    if constexpr (M >= 16) x = transpose_level<M, 8>(x, lane);
    if constexpr (M >= 8) x = transpose_level<M, 4>(x, lane);
    if constexpr (M >= 4) x = transpose_level<M, 2>(x, lane);
    return transpose_level<M, 1>(x, lane);
}

__device__ __forceinline__ uint32_t float_to_ord(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float ord_to_float(uint32_t o) {
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}
// Maximum / sum over each aligned group of M lanes, one DPP or permlane move
// per step (no LDS round trip).  All 64 lanes must be active.
template <int S, int M>
__device__ __forceinline__ uint64_t max_u64_step(uint64_t v) {
    if constexpr (S >= M) {
        return v;
    } else {
        const uint32_t lo = xor_lane<S>((uint32_t)v), hi = xor_lane<S>((uint32_t)(v >> 32));
        const uint64_t o = ((uint64_t)hi << 32) | lo;
        return max_u64_step<2 * S, M>(o > v ? o : v);
    }
}
template <int M>
__device__ __forceinline__ uint64_t group_max_u64(uint64_t v) { return max_u64_step<1, M>(v); }
template <int S, int M>
__device__ __forceinline__ int sum_step(int v) {
    if constexpr (S >= M) return v;
    else return sum_step<2 * S, M>(v + (int)xor_lane<S>((uint32_t)v));
}
template <int M>
__device__ __forceinline__ int group_sum(int v) { return sum_step<1, M>(v); }
template <int S, int M, bool MAX>
__device__ __forceinline__ uint32_t ext_u32_step(uint32_t v) {
    if constexpr (S >= M) {
        return v;
    } else {
        const uint32_t o = xor_lane<S>(v);
        return ext_u32_step<2 * S, M, MAX>(MAX ? (o > v ? o : v) : (o < v ? o : v));
    }
}
template <int M>
__device__ __forceinline__ uint32_t group_max_u32(uint32_t v) { return ext_u32_step<1, M, true>(v); }
template <int M>
__device__ __forceinline__ uint32_t group_min_u32(uint32_t v) { return ext_u32_step<1, M, false>(v); }

// Greedy over the (S desc, index asc) order, as the fixed point of the row
// and column thresholds; returns row i of the accepted mask.
// Row step: Rmask_i = {j : key_ij >= phi_i}, phi_i = N-th largest key of row i
// among j in Amask_i.  Column step: Cmask_j = {i : key_ij >= theta_j}, theta_j
// = N-th largest key of column j among i with key_ij >= phi_i.  Amask_i =
// {j : key_ij >= theta_j}.  Accepted = Rmask & Amask at the fixed point.  The
// theta sequence rises monotonically from "minus infinity" and can change at
// most M*M + M times, so the loop bound is never the exit in exact terms.
// NS > 0: N is the compile-time NS (walks skip the first NS positions).
template <int M, int NS>
__device__ __forceinline__ uint32_t greedy_rows(const uint32_t (&rpb)[M], const uint32_t (&cpb)[M],
                                                int N, uint32_t lane) {
    uint32_t Amask = kFull<M>, Rmask = kFull<M>, Cmask = 0u;
    if constexpr (NS > 0) {
        uint32_t rh = 0u, ch = 0u, rt[M - NS], ct[M - NS];
#pragma unroll
        for (int k = 0; k < NS; ++k) { rh |= rpb[k]; ch |= cpb[k]; }
#pragma unroll
        for (int k = 0; k < M - NS; ++k) { rt[k] = rpb[NS + k]; ct[k] = cpb[NS + k]; }
        for (int round = 0; round <= M * M + M + 2; ++round) {
            Rmask = walk_tail<M, NS>(rh, rt, Amask);
            const uint32_t Cnew = walk_tail<M, NS>(ch, ct, transpose_bits<M>(Rmask, lane));
            const bool changed = Cnew != Cmask;
            Cmask = Cnew;
            Amask = transpose_bits<M>(Cmask, lane);
            if (__ballot(changed) == 0ull) break;
        }
    } else {
        for (int round = 0; round <= M * M + M + 2; ++round) {
            Rmask = walk<M>(rpb, Amask, N);
            const uint32_t Cnew = walk<M>(cpb, transpose_bits<M>(Rmask, lane), N);
            const bool changed = Cnew != Cmask;
            Cmask = Cnew;
            Amask = transpose_bits<M>(Cmask, lane);
            if (__ballot(changed) == 0ull) break;
        }
    }
    return Rmask & Amask;
}

// ---------------------------------------------------------------- optional stages
// The 2-opt polish keeps per block a triangular table of the best swap gain
// of every row pair (4-byte keys); the keep-better sums reuse its area.
template <int M> constexpr int kPairs = M * (M - 1) / 2;
template <int M>
__device__ __forceinline__ int tri(int a, int b) { return a * M - a * (a + 1) / 2 + (b - a - 1); }
template <int M> constexpr int ref_tab_floats() {
    constexpr int tabs = (kWave / M) * kPairs<M>, sums = 2 * 2 * kWave;
    return tabs > sums ? tabs : sums;
}

// The optional stages R4 (2-opt polish, at most polish_steps swaps) and R5
// (keep the caller's previous mask where it is feasible and better) on the
// finished mask row Z of lane (q, i) = block q, row i of a pass of 64/M
// blocks: |W| rows staged in As ([G][M][M+1]), mask rows in Zs ([G][M]), and
// tab_area an 8-byte aligned LDS area of ref_tab_floats<M>() floats that
// nothing else uses meanwhile.  Returns the lane's final mask row.
template <int M>
__device__ __forceinline__ uint32_t refine_block(uint32_t Z, const MatJob& job, int64_t br,
                                                 int64_t bc, bool valid, int polish_steps,
                                                 const float* __restrict__ As,
                                                 uint32_t* __restrict__ Zs,
                                                 uint64_t* __restrict__ tab_area, int lane) {
    constexpr uint32_t FULL = kFull<M>;
    const int q = lane / M, i = lane % M;
    const int N = job.N;
    // ---- R4: 2-opt polish (optional) ----
    // A swap takes kept (i, j), (i', j'), i < i', with Z_ij' = Z_i'j = 0, to
    // (i, j'), (i', j); gain fl(fl(A_ij' - A_i'j') + fl(A_i'j - A_ij)).  Per row
    // pair the gain is monotone in each rounded difference, so the best gain
    // is fl(T1 + T2) with T1 = max over j' of the first difference and T2 =
    // max over j of the second; the smallest j and then j' attaining it give
    // the lexicographic tie-break.
    if (polish_steps > 0) {
        // Gain table: for every row pair {a < b} of the block, the ordered key
        // of its best swap gain (0 = no improving swap), triangular, pair at
        // tri<M>(a, b), so row a's pairs are contiguous.  Filled once; after a
        // swap of rows r1, r2 only the pairs touching r1 or r2 change, and lane
        // p re-evaluates {p, r1} and {p, r2} -- two pairs per lane per step.
        // Which (j, j') attains a pair's gain matters only for the pairs tied
        // at a step's best gain, so it is found then, for those pairs alone.
        uint32_t* tab = reinterpret_cast<uint32_t*>(tab_area) + q * kPairs<M>;
        float ai[M];
        {
            const float* Ai = As + (q * M + i) * (M + 1);
#pragma unroll
            for (int c = 0; c < M; ++c) ai[c] = Ai[c];
        }
        Zs[q * M + i] = Z;
        __syncthreads();
        // The pair {i, p} (p != i), row p's mask Zp: with a = min(i, p), b =
        // max(i, p), d_c = fl(A_ac - A_bc) = +-fl(A_ic - A_pc), the second
        // difference is fl(A_bj - A_aj) = -d_j exactly, so the best gain is
        // fl(T1 - min over j of d_j), T1 = max over j' of d_j'.
        auto pair_gain = [&](int p, uint32_t Zp, float& T1) -> float {
            const bool lo = i < p;
            const uint32_t Za = lo ? Z : Zp, Zb = lo ? Zp : Z;
            const uint32_t dj = Za & ~Zb;   // j:  Z_aj = 1, Z_bj = 0
            const uint32_t dk = Zb & ~Za;   // j': Z_bj' = 1, Z_aj' = 0
            const float* Ap = As + (q * M + p) * (M + 1);
            float Dmin = __builtin_inff();
            T1 = -__builtin_inff();
#pragma unroll
            for (int c = 0; c < M; ++c) {
                const float x = __fsub_rn(ai[c], Ap[c]);
                const float d = lo ? x : -x;
                if ((dk >> c) & 1u) T1 = fmaxf(T1, d);
                if ((dj >> c) & 1u) Dmin = fminf(Dmin, d);
            }
            return dj == 0u ? -__builtin_inff() : __fadd_rn(T1, -Dmin);
        };
        auto gain_key = [&](int p, uint32_t Zp) -> uint32_t {
            float T1;
            const float G = pair_gain(p, Zp, T1);
            return G > 0.f ? float_to_ord(G) : 0u;
        };
        // Fill: lane i takes the partners i+1 .. i+M/2 (mod M), the last one only
        // for i < M/2 -- every pair exactly once, about M/2 pairs per lane.
        for (int k = 1; k <= M / 2; ++k) {
            const int p = (i + k) % M;
            if (k < M / 2 || i < M / 2) {
                const int a = i < p ? i : p, b = i < p ? p : i;
                tab[tri<M>(a, b)] = valid ? gain_key(p, Zs[q * M + p]) : 0u;
            }
        }
        __syncthreads();
        bool active = valid;
        for (int step = 0; step < polish_steps && __ballot(active) != 0ull; ++step) {
            // the best gain of the block: lane i scans the pairs it fills
            // (the same circulant share, about M/2 independent reads)
            uint32_t g = 0u;
#pragma unroll
            for (int k = 1; k <= M / 2; ++k) {
                const int p = (i + k) % M;
                const int a = i < p ? i : p, b = i < p ? p : i;
                const uint32_t v = (k < M / 2 || i < M / 2) ? tab[tri<M>(a, b)] : 0u;
                g = v > g ? v : g;
            }
            if (!active) g = 0u;
            const uint32_t gmax = group_max_u32<M>(g);
            if (active && gmax == 0u) active = false;  // no improving swap left
            // The lexicographically smallest swap among the pairs at that gain.
            // lex grows with a first, so only the tied pairs of the smallest a
            // matter; they are taken one at a time in (a, b) order, each by the
            // whole block (lane c: column c) -- the same arithmetic as a scan
            // of the pair's columns, as two group reductions and two ballots.
            const float G = ord_to_float(gmax);
            uint32_t tied = 0u;  // bit k - 1: pair k of this lane's share ties
            if (active) {
                for (int k = 1; k <= M / 2; ++k) {
                    const int p = (i + k) % M;
                    const int a = i < p ? i : p, b = i < p ? p : i;
                    if ((k < M / 2 || i < M / 2) && tab[tri<M>(a, b)] == gmax) tied |= 1u << (k - 1);
                }
            }
            uint32_t lex = 0xFFFFFFFFu;
            int amin = M;
            for (;;) {
                // smallest remaining tied pair of the block, as a * M + b
                uint32_t key = 0xFFFFFFFFu;
                for (uint32_t t = tied; t; t &= t - 1u) {
                    const int p = (i + __ffs(t)) % M;
                    const uint32_t ab = i < p ? (uint32_t)(i * M + p) : (uint32_t)(p * M + i);
                    key = ab < key ? ab : key;
                }
                const uint32_t kmin = group_min_u32<M>(key);
                const bool more = kmin != 0xFFFFFFFFu && (int)(kmin / M) <= amin;
                if (__ballot(more) == 0ull) break;
                for (uint32_t t = tied; t; t &= t - 1u) {  // the owner drops it
                    const int k = __ffs(t), p = (i + k) % M;
                    const uint32_t ab = i < p ? (uint32_t)(i * M + p) : (uint32_t)(p * M + i);
                    if (ab == kmin) tied &= ~(1u << (k - 1));
                }
                const int a = more ? (int)(kmin / M) : 0, b = more ? (int)(kmin % M) : 1;
                const float* Aa = As + (q * M + a) * (M + 1);
                const float* Ab = As + (q * M + b) * (M + 1);
                const uint32_t Za = Zs[q * M + a], Zb = Zs[q * M + b];
                const float d = __fsub_rn(Aa[i], Ab[i]);  // d_c = fl(A_ac - A_bc), c = i
                const bool inJ = ((Za & ~Zb) >> i) & 1u, inK = ((Zb & ~Za) >> i) & 1u;
                const float T1 = ord_to_float(group_max_u32<M>(inK ? float_to_ord(d) : 0u));
                const uint32_t hj =
                    (uint32_t)(__ballot(inJ && __fadd_rn(T1, -d) == G) >> (q * M)) & FULL;
                const int jb = hj ? __ffs(hj) - 1 : 0;
                const float t2 = -__fsub_rn(Aa[jb], Ab[jb]);
                const uint32_t hk =
                    (uint32_t)(__ballot(inK && __fadd_rn(d, t2) == G) >> (q * M)) & FULL;
                const int jpb = hk ? __ffs(hk) - 1 : 0;
                if (more) {
                    amin = a;
                    const uint32_t l = (uint32_t)(((a * M + jb) * M + b) * M + jpb);
                    lex = l < lex ? l : lex;
                }
            }
            __syncthreads();
            int r1 = -1, r2 = -1;
            if (active) {
                const int jp = (int)(lex % M), ip = (int)((lex / M) % M);
                const int j = (int)((lex / (M * M)) % M), ii = (int)(lex / (M * M * M));
                if (i == ii) Z = (Z & ~(1u << j)) | (1u << jp);
                if (i == ip) Z = (Z & ~(1u << jp)) | (1u << j);
                Zs[q * M + i] = Z;
                r1 = ii;
                r2 = ip;
            }
            __syncthreads();
            if (r1 >= 0) {
                // lane i refreshes {i, r1} and {i, r2}; lane r1 refreshes {r1, r2}
                const int pa = (i == r1) ? r2 : r1;
                const int pb = (i == r1 || i == r2) ? -1 : r2;
                {
                    const int lo2 = i < pa ? i : pa, hi2 = i < pa ? pa : i;
                    if (i != r2 || pa != r1) tab[tri<M>(lo2, hi2)] = gain_key(pa, Zs[q * M + pa]);
                }
                if (pb >= 0) {
                    const int lo2 = i < pb ? i : pb, hi2 = i < pb ? pb : i;
                    tab[tri<M>(lo2, hi2)] = gain_key(pb, Zs[q * M + pb]);
                }
            }
            __syncthreads();
        }
    }

    // ---- R5: keep the caller's previous mask where it is feasible and better ----
    // Objective of a block: row sums over j ascending, then over rows i
    // ascending, both in fp64 (every lane forms the same total from LDS).
    if (job.prev != nullptr) {
        const float* Ai = As + (q * M + i) * (M + 1);
        uint32_t Zp = 0u;
        if (valid) {
            const int64_t c0 = bc * M;
            Zp = (job.prev[(br * M + i) * job.wpr + (c0 >> 5)] >> (int)(c0 & 31)) & FULL;
        }
        const bool rows_ok = __popc(Zp) == N;
        const bool cols_ok = __popc(transpose_bits<M>(Zp, (uint32_t)lane)) == N;
        const uint64_t okb = __ballot(rows_ok && cols_ok);
        const bool feasible = ((uint32_t)(okb >> (q * M)) & FULL) == FULL;
        double rz = 0.0, rp = 0.0;
#pragma unroll
        for (int j = 0; j < M; ++j) {
            const double a = (double)Ai[j];
            if ((Z >> j) & 1u) rz += a;
            if ((Zp >> j) & 1u) rp += a;
        }
        double* sums = reinterpret_cast<double*>(tab_area);  // [G][M][2]; tables are done
        sums[2 * (q * M + i)] = rz;
        sums[2 * (q * M + i) + 1] = rp;
        __syncthreads();
        double tz = 0.0, tp = 0.0;
        for (int k = 0; k < M; ++k) {
            tz += sums[2 * (q * M + k)];
            tp += sums[2 * (q * M + k) + 1];
        }
        __syncthreads();
        if (valid && feasible && tp > tz) Z = Zp;
    }

    return Z;
}

// Rounding of the 64/M blocks handled by this pass: lane (q, i) = block q,
// row i (and column i).  Sb points at the lane's block (row stride sld).
// Row i of a rounding pass's block for one lane: S (from Sb, row stride sld;
// Sb must be a readable address even for a block past the matrix) and |W|
// (block column bc of block-row br); zeros for a block past the matrix.
template <int M, bool BF16>
__device__ __forceinline__ void load_pass_rows(const float* __restrict__ Sb, int64_t sld,
                                               const MatJob& job, int64_t br, int64_t bc,
                                               bool valid, int i, float (&v)[M], float (&a)[M]) {
    load_row_f32<M>(Sb + i * sld, (reinterpret_cast<uintptr_t>(Sb) & 15u) == 0 && (sld & 3) == 0,
                    v);
    if (valid) {
        load_abs_row<M, BF16>(job.W, (br * M + i) * job.ld + bc * M, job.aligned != 0, a);
    } else {
#pragma unroll
        for (int j = 0; j < M; ++j) { v[j] = 0.f; a[j] = 0.f; }
    }
}

// Row i of |W| of a rounding pass's block (block column bc of block-row br);
// zeros for a block past the matrix.
template <int M, bool BF16>
__device__ __forceinline__ void load_abs_pass_row(const MatJob& job, int64_t br, int64_t bc,
                                                  bool valid, int i, float (&a)[M]) {
    if (valid) {
        load_abs_row<M, BF16>(job.W, (br * M + i) * job.ld + bc * M, job.aligned != 0, a);
    } else {
#pragma unroll
        for (int j = 0; j < M; ++j) a[j] = 0.f;
    }
}

// Row i of S of a rounding pass's block rebuilt from the block's record rb
// (see kRec) and its row of |W|: S_ij = min(2^(scale |W_ij| + row_i +
// col_j), 1), zeros for a block past the matrix.  The row is also the S
// output when one is requested.
template <int M>
__device__ __forceinline__ void rebuild_row(const float* __restrict__ rb, const MatJob& job,
                                            int64_t br, int64_t bc, bool valid, int i,
                                            const float (&a)[M], float (&v)[M]) {
    // Every record holds finite values (a block past the matrix solves a
    // zero block), so the row is computed for every lane and then zeroed
    // with one multiply: a conditional here became a branch per element.
    float col[M];
    if constexpr (kRec<M> % 4 == 0) {
#pragma unroll
        for (int q = 0; q < M / 4; ++q) {
            const float4 c4 = *reinterpret_cast<const float4*>(rb + M + 4 * q);
            col[4 * q] = c4.x; col[4 * q + 1] = c4.y; col[4 * q + 2] = c4.z; col[4 * q + 3] = c4.w;
        }
    } else {
#pragma unroll
        for (int j = 0; j < M; ++j) col[j] = rb[M + j];
    }
    const float sc = rb[2 * M], ro = rb[i];
    const float keep = valid ? 1.0f : 0.0f;
#pragma unroll
    for (int j = 0; j < M; ++j)
        v[j] = __builtin_amdgcn_fmed3f(ex2(fmaf(a[j], sc, ro) + col[j]), 0.0f, 1.0f) * keep;
    if (job.frac != nullptr && valid) {
        float* frow = job.frac + (br * M + i) * job.cols + bc * M;
        if ((reinterpret_cast<uintptr_t>(frow) & 15u) == 0) {
#pragma unroll
            for (int q = 0; q < M / 4; ++q)
                *reinterpret_cast<float4*>(frow + 4 * q) =
                    make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
        } else {
#pragma unroll
            for (int j = 0; j < M; ++j) frow[j] = v[j];
        }
    }
}

// The next pass whose |W| rows round_pass loads ahead (after its own rows are
// staged), so that their memory latency overlaps this pass's sorts and greedy.
// Used at M = 8 (eight passes per group; 1-3% faster at 4:8 and 8:16 in A/B
// runs); at M = 32 the registers it holds through the rounding made the 16:32
// launch 2% slower, and at M = 16 it measured the same as none.
template <int M> constexpr bool kPrefetch = (M == 8);
struct NextPass {
    int64_t bc;
    bool valid, any;
};

// How a rounding pass gets its rows: loaded here from Sb (row stride sld) and
// W; given by the caller (v = S, a = |W|), optionally loading the next pass's
// |W| rows ahead into an; or S already in the LDS staging at Ss and a given.
enum RowSource { kRowsLoad = 0, kRowsGiven = 1, kRowsStaged = 2 };

// Rounding of the 64/M blocks of one pass; lane (q, i) = block q, row i.
// POLISH: the optional stages (refine_block) run on the finished rows before
// the pack, with the pass's S staging (free by then) as their table area.
template <int M, bool BF16, int SRC, bool POLISH = false>
__device__ __forceinline__ void round_pass(const float* __restrict__ Sb, int64_t sld,
                                           const float (&v)[M], const float (&a)[M],
                                           const MatJob& job, int64_t br, int64_t bc, bool valid,
                                           int ls_steps, float* __restrict__ Ss,
                                           float* __restrict__ lds, const NextPass& nx,
                                           float (&an)[M],
                                           int polish_steps = 0) {
    constexpr int G = kWave / M;
    constexpr uint32_t FULL = kFull<M>;
    int lane = threadIdx.x;
    // Opaque to the optimiser: nothing derived from the lane (per-entry key
    // bits, LDS addresses) is hoisted out of the surrounding loops, where it
    // would stay live -- and cost registers -- through the solve.
    asm volatile("" : "+v"(lane));
    const int q = lane / M, i = lane % M;
    const int N = job.N;

    // Stage the pass's blocks in LDS, then sort row i and column i by key and
    // keep only the bit of each sorted entry.  Row i of |W| is fetched in the
    // same round trip as row i of S: most blocks need it for the local search.
    // Ss [G][M][kStageRow] (S), As [G][M][M+1] (|W|), Zs [G][M] (mask rows)
    float* As = lds + kStaged<M> * kStageBlk<M>;
    uint32_t* Zs = reinterpret_cast<uint32_t*>(As + G * M * (M + 1));
    auto stage = [&](const float (&vs)[M], const float (&as)[M]) {
        if constexpr (SRC != kRowsStaged) {
            float* dst = Ss + q * kStageBlk<M> + i * kStageRow<M>;
#pragma unroll
            for (int k4 = 0; k4 < M / 4; ++k4)
                *reinterpret_cast<float4*>(dst + 4 * k4) =
                    make_float4(vs[4 * k4], vs[4 * k4 + 1], vs[4 * k4 + 2], vs[4 * k4 + 3]);
        }
        float* Ai = As + (q * M + i) * (M + 1);
#pragma unroll
        for (int j = 0; j < M; ++j) Ai[j] = as[j];
    };
    if constexpr (SRC == kRowsLoad) {
        float vl[M], al[M];
        load_pass_rows<M, BF16>(Sb, sld, job, br, bc, valid, i, vl, al);
        stage(vl, al);
    } else {
        stage(v, a);
    }
    rnd_sync<M>();
    if constexpr (SRC == kRowsGiven) {
        if (nx.any) load_abs_pass_row<M, BF16>(job, br, nx.bc, nx.valid, i, an);
    }
    uint32_t rpb[M], cpb[M];
    // An opaque zero in the keys' low words: with compile-time constants there
    // the scheduler interleaves both sorts and runs out of registers.
    int kzero = 0;
    asm volatile("" : "+v"(kzero));
    {
        double key[M];
        const float* src = Ss + q * kStageBlk<M> + i * kStageRow<M>;
#pragma unroll
        for (int j = 0; j < M; ++j) key[j] = make_key<M>(src[j], j, kzero);
        sort_desc<M>(key);
#pragma unroll
        for (int k = 0; k < M; ++k) {
            rpb[k] = key_bit<M>(key[k]);
            asm volatile("" : "+v"(rpb[k]));  // keep only the bit, not the index
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    {
        double key[M];
        const float* src = Ss + q * kStageBlk<M> + i;
#pragma unroll
        for (int r = 0; r < M; ++r) key[r] = make_key<M>(src[r * kStageRow<M>], r, kzero);
        sort_desc<M>(key);
#pragma unroll
        for (int k = 0; k < M; ++k) {
            cpb[k] = key_bit<M>(key[k]);
            asm volatile("" : "+v"(cpb[k]));
        }
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- greedy as the fixed point of the row / column thresholds ----
    const uint32_t ulane = (uint32_t)lane;
    const uint32_t Z0 = (N == M / 2) ? greedy_rows<M, M / 2>(rpb, cpb, N, ulane)
                                     : greedy_rows<M, 0>(rpb, cpb, N, ulane);
    uint32_t Z = Z0;  // row i of the greedy mask
    int r = __popc(Z);
    int c = __popc(transpose_bits<M>(Z, ulane));  // column i count
    const int shift = q * M;
    uint32_t DR = (uint32_t)(__ballot(r < N) >> shift) & FULL;
    uint32_t DC = (uint32_t)(__ballot(c < N) >> shift) & FULL;
    int D = group_sum<M>(N - r);

    // ---- local search (R2) and fill (R3) ----
    const bool need = valid && D > 0;
    if (__ballot(need) != 0ull) {
        const float* Ai = As + (q * M + i) * (M + 1);
        Zs[q * M + i] = Z;
        rnd_sync<M>();

        int moves = 0;
        bool active = need && ls_steps > 0;
        // R2: at most ls_steps moves, each the best (i, j, i', j') with a
        // positive score, ties to the smallest in lexicographic order.
        if constexpr (M <= 8) {
            // Small blocks: a direct scan of every candidate, one packed
            // (score, ~lexicographic index) maximum per step.
            while (__ballot(active) != 0ull) {
                uint64_t best = 0;
                if (active) {
                    for (uint32_t dr = DR; dr; dr &= dr - 1u) {
                        const int ii = __ffs(dr) - 1;
                        const uint32_t cand0 = Z & ~Zs[q * M + ii];
                        if (!cand0) continue;
                        const float* Aii = As + (q * M + ii) * (M + 1);
                        for (uint32_t dc = DC; dc; dc &= dc - 1u) {
                            const int jj = __ffs(dc) - 1;
                            if ((Z >> jj) & 1u) continue;
                            const float a2 = Ai[jj];
                            for (uint32_t cs = cand0; cs; cs &= cs - 1u) {
                                const int jp = __ffs(cs) - 1;
                                const float sc = __fsub_rn(__fadd_rn(Aii[jp], a2), Ai[jp]);
                                const uint32_t lex = (uint32_t)(((ii * M + jj) * M + i) * M + jp);
                                const uint64_t key =
                                    ((uint64_t)float_to_ord(sc) << 32) | (uint64_t)(0xFFFFFFFFu - lex);
                                best = key > best ? key : best;
                            }
                        }
                    }
                }
                best = group_max_u64<M>(best);
                rnd_sync<M>();
                if (active) {
                    const float sc = ord_to_float((uint32_t)(best >> 32));
                    if (best == 0ull || !(sc > 0.f)) {
                        active = false;
                    } else {
                        const uint32_t lex = 0xFFFFFFFFu - (uint32_t)best;
                        const int jp = (int)(lex % M), ip = (int)((lex / M) % M);
                        const int jj = (int)((lex / (M * M)) % M), ii = (int)(lex / (M * M * M));
                        if (i == ii) { Z |= 1u << jp; r += 1; }
                        if (i == ip) Z = (Z | (1u << jj)) & ~(1u << jp);
                        if (i == jj) c += 1;
                        Zs[q * M + i] = Z;
                        ++moves;
                        --D;
                        if (D == 0 || moves >= ls_steps) active = false;
                    }
                }
                rnd_sync<M>();
                DR = (uint32_t)(__ballot(r < N) >> shift) & FULL;
                DC = (uint32_t)(__ballot(c < N) >> shift) & FULL;
            }
        } else {
            float* Cm = Ss + q * M;  // column maxima of block q (the staging area is free now)
            // The score fl(fl(A_ij' + A_i'j) - A_i'j') is monotone in A_ij' and
            // in A_i'j, and the admissibility of i (deficient, Z_ij' = 0) does not
            // involve j, nor that of j (deficient, Z_i'j = 0) i.  So for a fixed
            // (i', j') the best score takes the largest admissible A_ij' of column
            // j' and the largest admissible A_i'j of row i'.  Lane i acts as column
            // j' = i for the first maximum and as row i' = i for the second and for
            // its best score.  The smallest (i, j, i', j') attaining the block's best
            // score G is then found one coordinate at a time, each stage keeping
            // only the candidates that can still reach G.
            while (__ballot(active) != 0ull) {
                float cmax = 0.f, rmax = 0.f;
                bool hc = false, hr = false;
                if (active) {
                    for (uint32_t dr = DR; dr; dr &= dr - 1u) {
                        const int ii = __ffs(dr) - 1;
                        if ((Zs[q * M + ii] >> i) & 1u) continue;
                        const float a = As[(q * M + ii) * (M + 1) + i];
                        cmax = (!hc || a > cmax) ? a : cmax;
                        hc = true;
                    }
                    for (uint32_t dc = DC & ~Z; dc; dc &= dc - 1u) {
                        const float a = Ai[__ffs(dc) - 1];
                        rmax = (!hr || a > rmax) ? a : rmax;
                        hr = true;
                    }
                    Cm[i] = cmax;
                }
                const uint32_t CM = (uint32_t)(__ballot(hc) >> shift) & FULL;
                rnd_sync<M>();
                uint32_t sk = 0u;  // ordered key of the lane's best score, 0 = no candidate
                uint32_t J = 0u;   // the columns j' attaining it
                if (active && hr) {
                    auto consider = [&](int jp, float cmj, float aij) {
                        const uint32_t k = float_to_ord(__fsub_rn(__fadd_rn(cmj, rmax), aij));
                        J = (k > sk) ? (1u << jp) : (k == sk ? (J | (1u << jp)) : J);
                        sk = k > sk ? k : sk;
                    };
                    if constexpr (M == 32) {
                        // two columns per iteration, in ascending order, so that
                        // their four LDS reads are in flight together (16:32
                        // -0.6%; at M = 16 +0.5%, so one column there)
                        for (uint32_t cs = Z & CM; cs;) {
                            const int jp0 = __ffs(cs) - 1;
                            cs &= cs - 1u;
                            const bool two = cs != 0u;
                            const int jp1 = two ? __ffs(cs) - 1 : jp0;
                            cs &= cs - 1u;
                            const float c0 = Cm[jp0], a0 = Ai[jp0], c1 = Cm[jp1], a1 = Ai[jp1];
                            consider(jp0, c0, a0);
                            if (two) consider(jp1, c1, a1);
                        }
                    } else {
                        for (uint32_t cs = Z & CM; cs; cs &= cs - 1u) {
                            const int jp = __ffs(cs) - 1;
                            consider(jp, Cm[jp], Ai[jp]);
                        }
                    }
                }
                const uint32_t gk = group_max_u32<M>(sk);
                const float Gs = ord_to_float(gk);
                if (active && (gk == 0u || !(Gs > 0.f))) active = false;
                if (sk != gk || !active) J = 0u;
                // stage 1: smallest deficient row i
                uint32_t t = M;
                if (J) {
                    for (uint32_t dr = DR; dr && t == (uint32_t)M; dr &= dr - 1u) {
                        const int ii = __ffs(dr) - 1;
                        const float* Aii = As + (q * M + ii) * (M + 1);
                        for (uint32_t cs = J & ~Zs[q * M + ii]; cs; cs &= cs - 1u) {
                            const int jp = __ffs(cs) - 1;
                            if (__fsub_rn(__fadd_rn(Aii[jp], rmax), Ai[jp]) == Gs) {
                                t = (uint32_t)ii;
                                break;
                            }
                        }
                    }
                }
                const int bi = (int)group_min_u32<M>(t);
                // stage 2: smallest deficient column j for that row
                uint32_t Jw = 0u;
                t = M;
                if (J && bi < M) {
                    const float* Abi = As + (q * M + bi) * (M + 1);
                    for (uint32_t cs = J & ~Zs[q * M + bi]; cs; cs &= cs - 1u) {
                        const int jp = __ffs(cs) - 1;
                        if (__fsub_rn(__fadd_rn(Abi[jp], rmax), Ai[jp]) == Gs) Jw |= 1u << jp;
                    }
                    for (uint32_t dc = DC & ~Z; dc && Jw && t == (uint32_t)M; dc &= dc - 1u) {
                        const int jj = __ffs(dc) - 1;
                        const float a2 = Ai[jj];
                        for (uint32_t cs = Jw; cs; cs &= cs - 1u) {
                            const int jp = __ffs(cs) - 1;
                            if (__fsub_rn(__fadd_rn(Abi[jp], a2), Ai[jp]) == Gs) {
                                t = (uint32_t)jj;
                                break;
                            }
                        }
                    }
                }
                const int bj = (int)group_min_u32<M>(t);
                // stage 3: smallest row i', then its smallest column j'
                uint32_t Jf = 0u;
                if (Jw && bj < M && !((Z >> bj) & 1u)) {
                    const float* Abi = As + (q * M + bi) * (M + 1);
                    const float a2 = Ai[bj];
                    for (uint32_t cs = Jw; cs; cs &= cs - 1u) {
                        const int jp = __ffs(cs) - 1;
                        if (__fsub_rn(__fadd_rn(Abi[jp], a2), Ai[jp]) == Gs) Jf |= 1u << jp;
                    }
                }
                const uint32_t IP = (uint32_t)(__ballot(Jf != 0u) >> shift) & FULL;
                const int bip = IP ? __ffs(IP) - 1 : M;
                const int bjp = (int)group_max_u32<M>(i == bip ? (uint32_t)(__ffs(Jf) - 1) : 0u);
                rnd_sync<M>();
                if (active) {
                    if (bip >= M) {
                        active = false;  // unreachable: G is attained by construction
                    } else {
                        if (i == bi) { Z |= 1u << bjp; r += 1; }
                        if (i == bip) Z = (Z | (1u << bj)) & ~(1u << bjp);
                        if (i == bj) c += 1;
                        Zs[q * M + i] = Z;
                        ++moves;
                        --D;
                        if (D == 0 || moves >= ls_steps) active = false;
                    }
                }
                rnd_sync<M>();
                DR = (uint32_t)(__ballot(r < N) >> shift) & FULL;
                DC = (uint32_t)(__ballot(c < N) >> shift) & FULL;
            }
        }
        active = valid && D > 0;
        while (__ballot(active) != 0ull) {  // R3
            uint64_t best = 0;
            if (active) {
                const int ii = __ffs(DR) - 1, jj = __ffs(DC) - 1;
                if (!((Z >> jj) & 1u)) {
                    const float* Aii = As + (q * M + ii) * (M + 1);
                    const float a2 = Ai[jj];
                    for (uint32_t cs = Z & ~Zs[q * M + ii]; cs; cs &= cs - 1u) {
                        const int jp = __ffs(cs) - 1;
                        const float sc = __fsub_rn(__fadd_rn(Aii[jp], a2), Ai[jp]);
                        const uint32_t lex = (uint32_t)(i * M + jp);
                        const uint64_t key =
                            ((uint64_t)float_to_ord(sc) << 32) | (uint64_t)(0xFFFFFFFFu - lex);
                        best = key > best ? key : best;
                    }
                }
            }
            best = group_max_u64<M>(best);
            rnd_sync<M>();
            if (active) {
                if (best == 0ull) {
                    active = false;  // unreachable while the invariant holds
                } else {
                    const int ii = __ffs(DR) - 1, jj = __ffs(DC) - 1;
                    const uint32_t lex = 0xFFFFFFFFu - (uint32_t)best;
                    const int jp = (int)(lex % M), ip = (int)(lex / M);
                    if (i == ii) { Z |= 1u << jp; r += 1; }
                    if (i == ip) Z = (Z | (1u << jj)) & ~(1u << jp);
                    if (i == jj) c += 1;
                    Zs[q * M + i] = Z;
                    --D;
                    if (D == 0) active = false;
                }
            }
            rnd_sync<M>();
            DR = (uint32_t)(__ballot(r < N) >> shift) & FULL;
            DC = (uint32_t)(__ballot(c < N) >> shift) & FULL;
        }
    }

    if constexpr (POLISH) {
        static_assert(kStageInLds<M> ? (kWave / M) * kStageBlk<M> >= ref_tab_floats<M>()
                                     : kStaged<M> * kStageBlk<M> >= ref_tab_floats<M>(),
                      "the optional stages' table fits the pass's S staging");
        rnd_sync<M>();  // every lane is done with the staged S
        Z = refine_block<M>(Z, job, br, bc, valid, polish_steps, As, Zs,
                            reinterpret_cast<uint64_t*>(Ss), lane);
    }

    // ---- pack: OR the blocks of one 32-column word together, one store ----
    const int bit0 = (int)((bc * M) & 31);
    uint32_t w = valid ? (Z << bit0) : 0u;
    if constexpr (M <= 4) w |= xor_lane<4>(w);
    if constexpr (M <= 8) w |= xor_lane<8>(w);
    if constexpr (M <= 16) w |= xor_lane<16>(w);
    if (valid && bit0 == 0) job.mask[(br * M + i) * job.wpr + ((bc * M) >> 5)] = w;
}

// ---------------------------------------------------------------- exact
// Optimal mask of every block (the block LP -- rows and columns summing to N,
// 0 <= S <= 1 -- is a bipartite b-matching, hence integral).  Starting from a
// feasible mask, a mask is optimal iff the residual graph has no negative
// cycle: row i -> column j for Z_ij = 0 at cost -|W_ij|, column j -> row i for
// Z_ij = 1 at cost +|W_ij|.  Each round of Bellman-Ford from a virtual source
// (all distances 0) relaxes every node's incoming arcs at once (one lane per
// row or column node, fp64 distances); a change in round 2M proves a negative
// cycle, which is found by following predecessors and cancelled (Z flips along
// it, every row and column count is kept, the objective rises by -cost).  A
// block is done when a Bellman-Ford pass settles; `tol` = 2^-40 * max|W| of the
// block ignores cycles within rounding.  One wave handles one 32-column word
// of one block-row (32/M blocks of 2M lanes).
template <int M> __device__ __forceinline__ uint32_t circulant_row(int i, int N) {
    uint32_t z = 0u;
    for (int k = 0; k < N; ++k) z |= 1u << ((i + k) % M);
    return z;
}

template <int M, bool BF16>
__global__ __launch_bounds__(kWave) void exact_kernel(MatJob job, const uint32_t* __restrict__ start,
                                                      double* __restrict__ obj, int max_cancel) {
    constexpr int V = 2 * M, NB = kWave / V;
    constexpr uint32_t FULL = kFull<M>;
    static_assert(NB * M == 32, "one wave covers one 32-column word");
    __shared__ double dist_s[kWave];
    __shared__ int pred_s[kWave];
    __shared__ uint32_t z_s[kWave];
    __shared__ int cyc_s[NB][V + 1];
    __shared__ double sum_s[kWave];
    __shared__ float a_s[NB][M][M];  // the blocks' scores, for the cycle costs
    constexpr uint64_t kBlkLanes = (V == 64) ? ~0ull : ((1ull << V) - 1ull);
    const int lane = threadIdx.x;
    const int b = lane / V, v = lane % V;
    const bool isrow = v < M;
    const int idx = isrow ? v : v - M;
    const int N = job.N;
    const int64_t nbc = job.cols / M, nbr = job.rows / M;
    const int64_t units = nbr * job.wpr;
    for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {
        const int64_t br = u / job.wpr, w = u % job.wpr;
        const int64_t bc = w * NB + b;
        const bool valid = bc < nbc;
        const int64_t r0 = br * M, c0 = bc * M;
        // |W| along this node's row (row node) or column (column node)
        double a[M];
        double amax = 0.0;
#pragma unroll
        for (int k = 0; k < M; ++k) {
            float x = 0.f;
            if (valid) {
                const int64_t off = isrow ? (r0 + idx) * job.ld + c0 + k : (r0 + k) * job.ld + c0 + idx;
                if constexpr (BF16)
                    x = __uint_as_float((uint32_t)(static_cast<const uint16_t*>(job.W)[off] & 0x7FFFu) << 16);
                else
                    x = fabsf(static_cast<const float*>(job.W)[off]);
            }
            a[k] = (double)x;
            amax = fmax(amax, a[k]);
        }
        // start mask (row nodes read it; an infeasible start block falls back
        // to the circulant mask row i -> columns i .. i+N-1 mod M)
        uint32_t zr = 0u;
        if (isrow && valid)
            zr = start ? (start[(r0 + idx) * job.wpr + (c0 >> 5)] >> (int)(c0 & 31)) & FULL
                       : circulant_row<M>(idx, N);
        z_s[lane] = zr;
        sum_s[lane] = amax;
        __syncthreads();
        uint32_t zc = 0u;  // column nodes: bit i = Z_i,idx
#pragma unroll
        for (int k = 0; k < M; ++k) zc |= ((z_s[b * V + k] >> idx) & 1u) << k;
        double bmax = 0.0;
#pragma unroll
        for (int k = 0; k < V; ++k) bmax = fmax(bmax, sum_s[b * V + k]);
        const double tol = bmax * 0x1p-40;
        const bool cnt_ok = __popc(isrow ? zr : zc) == N;
        const uint64_t okb = __ballot(cnt_ok);
        const bool feasible = ((okb >> (b * V)) & kBlkLanes) == kBlkLanes;
        __syncthreads();
        if (!feasible) {
            zr = (isrow && valid) ? circulant_row<M>(idx, N) : 0u;
            z_s[lane] = zr;
            __syncthreads();
            zc = 0u;
#pragma unroll
            for (int k = 0; k < M; ++k) zc |= ((z_s[b * V + k] >> idx) & 1u) << k;
            __syncthreads();
        }
        uint32_t z = isrow ? zr : zc;
        if (isrow) {
#pragma unroll
            for (int k = 0; k < M; ++k) a_s[b][idx][k] = (float)a[k];
        }
        bool done = !valid;
        bool failed = false;
        for (int cancel = 0; cancel <= max_cancel && __ballot(!done) != 0ull; ++cancel) {
            double d = 0.0;
            int pred = -1;
            bool settled = done, neg = false, last = false;
            for (int round = 0; round <= V && __ballot(!settled) != 0ull; ++round) {
                dist_s[lane] = d;
                __syncthreads();
                double best = d;
                int bp = -1;
                if (!settled) {
#pragma unroll
                    for (int k = 0; k < M; ++k) {
                        // row node: arcs column k -> row idx for Z_idx,k = 1 (cost +A);
                        // column node: arcs row k -> column idx for Z_k,idx = 0 (cost -A)
                        const bool arc = isrow ? ((z >> k) & 1u) != 0u : ((z >> k) & 1u) == 0u;
                        const double c = isrow ? dist_s[b * V + M + k] + a[k] : dist_s[b * V + k] - a[k];
                        if (arc && c < best - tol) {
                            best = c;
                            bp = isrow ? M + k : k;
                        }
                    }
                }
                __syncthreads();
                const bool ch = bp >= 0;
                if (ch) { d = best; pred = bp; }
                const uint64_t chb = __ballot(ch);
                const bool blk_ch = ((chb >> (b * V)) & kBlkLanes) != 0ull;
                if (!settled && !blk_ch) settled = true;
                if (!settled && round == V) {
                    neg = true;
                    settled = true;
                    last = ch;  // changed in the last round: its predecessors lead into a cycle
                }
            }
            pred_s[lane] = pred;
            z_s[lane] = last ? 1u : 0u;
            __syncthreads();
            if (neg && v == 0) {
                // walk the predecessors onto the cycle, list it (cyc_s[b][0] =
                // length, then the nodes; pred(x) follows x) and check its cost
                int x = -1;
                for (int k = 0; k < V; ++k)
                    if (z_s[b * V + k] != 0u) { x = k; break; }
                bool ok = x >= 0;
                for (int t = 0; t < V && ok; ++t) {
                    x = pred_s[b * V + x];
                    ok = x >= 0;
                }
                int n = 0;
                double cost = 0.0;
                if (ok) {
                    const int s0 = x;
                    do {
                        const int y = pred_s[b * V + x];
                        cyc_s[b][1 + n] = x;
                        ++n;
                        if (y < 0) break;
                        cost += (y < M) ? -(double)a_s[b][y][x - M] : (double)a_s[b][x][y - M];
                        x = y;
                    } while (x != s0 && n < V);
                    ok = x == s0 && (n & 1) == 0 && cost < -tol;
                }
                cyc_s[b][0] = ok ? n : -1;
            }
            __syncthreads();
            if (neg) {
                const int n = cyc_s[b][0];
                if (n < 0) {
                    done = true;  // no usable cycle (rounding): keep the current mask
                    failed = true;
                } else {
                    for (int t = 0; t < n; ++t) {  // arc y -> x with y = pred(x)
                        const int x = cyc_s[b][1 + t];
                        const int y = cyc_s[b][1 + (t + 1) % n];
                        if (y < M && x >= M) {  // row y -> column x: Z_y,x 0 -> 1
                            if (isrow && idx == y) z |= 1u << (x - M);
                            if (!isrow && idx == x - M) z |= 1u << y;
                        } else if (y >= M && x < M) {  // column y -> row x: Z_x,y 1 -> 0
                            if (isrow && idx == x) z &= ~(1u << (y - M));
                            if (!isrow && idx == y - M) z &= ~(1u << x);
                        }
                    }
                    if (cancel == max_cancel) { done = true; failed = true; }
                }
            } else {
                done = true;  // no negative cycle: optimal
            }
            __syncthreads();
        }
        // store: row lanes OR their blocks' bits into the word of their row
        z_s[lane] = (isrow && valid) ? (z << (b * M)) : 0u;
        double rs = 0.0;
        if (isrow) {
#pragma unroll
            for (int k = 0; k < M; ++k)
                if ((z >> k) & 1u) rs += a[k];
        }
        sum_s[lane] = rs;
        __syncthreads();
        if (b == 0 && isrow) {
            uint32_t word = 0u;
#pragma unroll
            for (int q = 0; q < NB; ++q) word |= z_s[q * V + idx];
            if (br * M + idx < job.rows && w < job.wpr) job.mask[(r0 + idx) * job.wpr + w] = word;
        }
        if (obj != nullptr && valid && v == 0) {
            double tot = 0.0;
            for (int k = 0; k < M; ++k) tot += sum_s[b * V + k];
            obj[br * nbc + bc] = failed ? __builtin_nan("") : tot;
        }
        __syncthreads();
    }
}

// Whole path for group gl (block-row br, first block column bc0) of one matrix.
template <int M, bool BF16, bool POLISH>
__device__ __forceinline__ void process_group(const MatJob& job, const Params& prm, int64_t gl,
                                              float* lds) {
    constexpr int BPG = kBPG<M>, G = kWave / M;
    const int64_t nbc = job.cols / M;
    const int64_t gpr = (nbc + BPG - 1) / BPG;
    const int64_t br = gl / gpr, bc0 = (gl % gpr) * BPG;
    constexpr int PASSES = BPG / G;
    // M = 4: the |W| rows the rounding passes use are loaded before the solve
    // (their latency is then hidden by it), and the solve exports S into the
    // LDS staging area of both passes.
    float apre[kStageInLds<M> ? PASSES : 1][M];
    if constexpr (kStageInLds<M>) {
        const int q = (int)threadIdx.x / M, i = (int)threadIdx.x % M;
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
            const int64_t bc = bc0 + p * G + q;
            if (bc < nbc) {
                load_abs_row<M, BF16>(job.W, (br * M + i) * job.ld + bc * M, job.aligned != 0,
                                      apre[p]);
            } else {
#pragma unroll
                for (int j = 0; j < M; ++j) apre[p][j] = 0.f;
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < M; ++j) apre[0][j] = 0.f;
    }
    dykstra_group<M, BF16>(job, prm, br, bc0, lds);
    __syncthreads();  // S or the records visible to every lane; LDS free for rounding
    set_prio<kPrioRound>();
    const NextPass none{0, false, false};
    if constexpr (kStageInLds<M>) {
        float unused[M];
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
            const int64_t bc = bc0 + p * G + (int)threadIdx.x / M;
            round_pass<M, BF16, kRowsStaged, POLISH>(nullptr, 0, apre[p], apre[p], job, br, bc,
                                                     bc < nbc, prm.ls_steps,
                                                     lds + p * G * kStageBlk<M>, lds, none,
                                                     unused, prm.polish_steps);
            __syncthreads();
        }
    } else {
        // Each pass's rows of S are rebuilt from the blocks' records and |W|.
        // kPrefetch: pass p + 1's |W| rows are loaded during pass p (in
        // round_pass, after staging).  An opaque lane keeps the row addresses
        // from being hoisted out of the kernel's group loop (and held through
        // the solve).
        const float* rec = lds + solve_round_floats<M>();
        float v[M], a[M], an[M];
        int lane = (int)threadIdx.x;
        asm volatile("" : "+v"(lane));
        const int q = lane / M, i = lane % M;
        if constexpr (kPrefetch<M>) {
            load_abs_pass_row<M, BF16>(job, br, bc0 + q, bc0 + q < nbc, i, a);
#pragma unroll 1
            for (int p = 0; p < PASSES; ++p) {
                const int64_t bc = bc0 + p * G + q, bcn = bc + G;
                rebuild_row<M>(rec + (p * G + q) * kRec<M>, job, br, bc, bc < nbc, i, a, v);
                const NextPass nx{bcn, bcn < nbc, p + 1 < PASSES};
                round_pass<M, BF16, kRowsGiven, POLISH>(nullptr, 0, v, a, job, br, bc, bc < nbc,
                                                        prm.ls_steps, lds, lds, nx, an,
                                                        prm.polish_steps);
                __syncthreads();
#pragma unroll
                for (int j = 0; j < M; ++j) a[j] = an[j];
            }
        } else {
#pragma unroll 1
            for (int p = 0; p < PASSES; ++p) {
                const int lb = p * G + q;
                const int64_t bc = bc0 + lb;
                load_abs_pass_row<M, BF16>(job, br, bc, bc < nbc, i, a);
                rebuild_row<M>(rec + lb * kRec<M>, job, br, bc, bc < nbc, i, a, v);
                round_pass<M, BF16, kRowsGiven, POLISH>(nullptr, 0, v, a, job, br, bc, bc < nbc,
                                                        prm.ls_steps, lds, lds, none, an,
                                                        prm.polish_steps);
                __syncthreads();
            }
        }
    }
    set_prio<0>();
}

template <int M, bool BF16, bool POLISH>
__global__ __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(kSolveWaves<M>)))
void mask_kernel(MatJob job, Params prm) {
    __shared__ __attribute__((aligned(16))) float lds[lds_floats<M>()];
    constexpr int BPG = kBPG<M>;
    const int64_t nbc = job.cols / M;
    const int64_t ngroups = (job.rows / M) * ((nbc + BPG - 1) / BPG);
    for (int64_t g = blockIdx.x; g < ngroups; g += gridDim.x)
        process_group<M, BF16, POLISH>(job, prm, g, lds);
}

template <int M, bool BF16>
__global__ __launch_bounds__(kWave) void round_kernel(MatJob job, const float* __restrict__ S,
                                                      int64_t sld, int ls_steps) {
    __shared__ __attribute__((aligned(16))) float lds[rnd_lds_floats<M>()];
    constexpr int G = kWave / M;
    const int64_t nbc = job.cols / M;
    const int64_t gpr = (nbc + G - 1) / G;
    const int64_t ngroups = (job.rows / M) * gpr;
    const NextPass none{0, false, false};
    float unused[M];
    for (int64_t g = blockIdx.x; g < ngroups; g += gridDim.x) {
        const int64_t br = g / gpr;
        const int64_t bc = (g % gpr) * G + threadIdx.x / M;
        const bool valid = bc < nbc;
        const float* Sb = S + br * M * sld + (valid ? bc : 0) * M;
        round_pass<M, BF16, kRowsLoad>(Sb, sld, unused, unused, job, br, bc, valid, ls_steps, lds,
                                       lds, none, unused);
        __syncthreads();
    }
}

// Many matrices of one (M, dtype) class in one launch: `jobs` lists the
// class's matrices with group_begin = prefix sum of their group counts; the
// grid walks the concatenated group range.  One kernel per class keeps the
// register allocation of each path as tight as in mask_kernel.
template <int M, bool BF16, bool POLISH>
__global__ __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(kSolveWaves<M>)))
void batched_kernel(const MatJob* __restrict__ jobs, int count, int64_t total_groups, Params prm) {
    __shared__ __attribute__((aligned(16))) float lds[lds_floats<M>()];
    for (int64_t g = blockIdx.x; g < total_groups; g += gridDim.x) {
        int lo = 0, hi = count - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (jobs[mid].group_begin <= g) lo = mid; else hi = mid - 1;
        }
        const MatJob job = jobs[lo];
        process_group<M, BF16, POLISH>(job, prm, g - job.group_begin, lds);
    }
}

// ---------------------------------------------------------------- debug check
// Counts the non-finite elements of a row-major [rows][cols] matrix (leading
// dimension ld), fp32 or bf16: those with an all-ones exponent field.
__global__ __launch_bounds__(64) void zero_count_kernel(int* count) { *count = 0; }

__global__ __launch_bounds__(256) void nonfinite_kernel(const void* __restrict__ p, int bf16,
                                                        int64_t rows, int64_t cols, int64_t ld,
                                                        int* __restrict__ count) {
    const int64_t n = rows * cols;
    int bad = 0;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < n;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = t / cols, c = t % cols;
        if (bf16) {
            const uint16_t u = static_cast<const uint16_t*>(p)[r * ld + c];
            bad += (u & 0x7F80u) == 0x7F80u;
        } else {
            const uint32_t u = __float_as_uint(static_cast<const float*>(p)[r * ld + c]);
            bad += (u & 0x7F800000u) == 0x7F800000u;
        }
    }
    if (bad) atomicAdd(count, bad);
}

}  // namespace

// ---------------------------------------------------------------- host side
#define TSENOR_DISPATCH(M_, BF, CALL)                                   \
    do {                                                                \
        switch ((M_) * 2 + ((BF) ? 1 : 0)) {                            \
            case 8: { constexpr int MM = 4; constexpr bool B = false; CALL; } break;  \
            case 9: { constexpr int MM = 4; constexpr bool B = true; CALL; } break;   \
            case 16: { constexpr int MM = 8; constexpr bool B = false; CALL; } break; \
            case 17: { constexpr int MM = 8; constexpr bool B = true; CALL; } break;  \
            case 32: { constexpr int MM = 16; constexpr bool B = false; CALL; } break; \
            case 33: { constexpr int MM = 16; constexpr bool B = true; CALL; } break;  \
            case 64: { constexpr int MM = 32; constexpr bool B = false; CALL; } break; \
            case 65: { constexpr int MM = 32; constexpr bool B = true; CALL; } break;  \
            default: return (int)hipErrorInvalidValue;                  \
        }                                                               \
    } while (0)

int blocks_per_group(int M) {
    switch (M) {
        case 4: return kBPG<4>;
        case 8: return kBPG<8>;
        case 16: return kBPG<16>;
        case 32: return kBPG<32>;
        default: return 0;
    }
}

int launch_mask(const MatJob& job, const Params& prm, int grid, void* stream) {
    if (prm.polish_steps > 0 || job.prev != nullptr) {
        TSENOR_DISPATCH(job.M, job.bf16,
                        hipLaunchKernelGGL((mask_kernel<MM, B, true>), dim3(grid), dim3(kWave), 0,
                                           (hipStream_t)stream, job, prm));
    } else {
        TSENOR_DISPATCH(job.M, job.bf16,
                        hipLaunchKernelGGL((mask_kernel<MM, B, false>), dim3(grid), dim3(kWave),
                                           0, (hipStream_t)stream, job, prm));
    }
    return (int)hipGetLastError();
}

int launch_round(const MatJob& job, const float* S, int64_t lds, int ls_steps, int grid,
                 void* stream) {
    TSENOR_DISPATCH(job.M, job.bf16,
                    hipLaunchKernelGGL((round_kernel<MM, B>), dim3(grid), dim3(kWave), 0,
                                       (hipStream_t)stream, job, S, lds, ls_steps));
    return (int)hipGetLastError();
}

int launch_batched(const MatJob* jobs_dev, int count, int64_t total_groups, int M, int bf16,
                   const Params& prm, bool optional_stages, int grid, void* stream) {
    if (optional_stages) {
        TSENOR_DISPATCH(M, bf16,
                        hipLaunchKernelGGL((batched_kernel<MM, B, true>), dim3(grid), dim3(kWave),
                                           0, (hipStream_t)stream, jobs_dev, count, total_groups,
                                           prm));
    } else {
        TSENOR_DISPATCH(M, bf16,
                        hipLaunchKernelGGL((batched_kernel<MM, B, false>), dim3(grid),
                                           dim3(kWave), 0, (hipStream_t)stream, jobs_dev, count,
                                           total_groups, prm));
    }
    return (int)hipGetLastError();
}

int occupancy_mask(int M, int bf16, bool optional_stages) {
    int n = 0;
    if (optional_stages) {
        TSENOR_DISPATCH(M, bf16,
                        (void)hipOccupancyMaxActiveBlocksPerMultiprocessor(
                            &n, mask_kernel<MM, B, true>, kWave, 0));
    } else {
        TSENOR_DISPATCH(M, bf16,
                        (void)hipOccupancyMaxActiveBlocksPerMultiprocessor(
                            &n, mask_kernel<MM, B, false>, kWave, 0));
    }
    return n;
}

int occupancy_round(int M, int bf16) {
    int n = 0;
    TSENOR_DISPATCH(M, bf16,
                    (void)hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, round_kernel<MM, B>,
                                                                       kWave, 0));
    return n;
}

int launch_exact(const MatJob& job, const uint32_t* start, double* obj, int max_cancel, int grid,
                 void* stream) {
    TSENOR_DISPATCH(job.M, job.bf16,
                    hipLaunchKernelGGL((exact_kernel<MM, B>), dim3(grid), dim3(kWave), 0,
                                       (hipStream_t)stream, job, start, obj, max_cancel));
    return (int)hipGetLastError();
}

int occupancy_exact(int M, int bf16) {
    int n = 0;
    TSENOR_DISPATCH(M, bf16,
                    (void)hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, exact_kernel<MM, B>,
                                                                       kWave, 0));
    return n;
}

int occupancy_batched(int M, int bf16, bool optional_stages) {
    int n = 0;
    if (optional_stages) {
        TSENOR_DISPATCH(M, bf16,
                        (void)hipOccupancyMaxActiveBlocksPerMultiprocessor(
                            &n, batched_kernel<MM, B, true>, kWave, 0));
    } else {
        TSENOR_DISPATCH(M, bf16,
                        (void)hipOccupancyMaxActiveBlocksPerMultiprocessor(
                            &n, batched_kernel<MM, B, false>, kWave, 0));
    }
    return n;
}

int launch_count_nonfinite(const void* p, int bf16, int64_t rows, int64_t cols, int64_t ld,
                           int* count, int grid, void* stream) {
    hipLaunchKernelGGL(zero_count_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, count);
    hipLaunchKernelGGL(nonfinite_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, p, bf16,
                       rows, cols, ld, count);
    return (int)hipGetLastError();
}

}  // namespace tsenor
