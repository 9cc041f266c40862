// tsenor_internal.h -- shared between the host ABI layer and the HIP kernels.
// Not installed; the public interface is include/tsenor.h.
#pragma once
#include <stdint.h>

namespace tsenor {

// One matrix as the kernels see it.
struct MatJob {
    const void* W;      // device, [rows][ld]
    uint32_t* mask;     // device, [rows][wpr]
    float* frac;        // device, [rows][cols] or nullptr
    const uint32_t* prev;  // device, [rows][wpr] previous mask for the keep-better stage, or nullptr
    int64_t rows, cols, ld, wpr;
    int64_t group_begin;  // batched launch: first group id of this matrix within its (M, dtype) class
    int32_t N, M;
    int32_t bf16;       // 1 = bfloat16 weights, 0 = fp32
    int32_t aligned;    // 1 = W rows may be read with 16-byte vector loads
};

// Scalars shared by every matrix of a launch.
struct Params {
    float tau_log2e;    // tau * log2(e): the Gibbs exponent in base 2
    int32_t iters;
    int32_t ls_steps;
    int32_t polish_steps;  // optional 2-opt swaps per block (0: none)
};

// Work decomposition: one workgroup = one wave (64 lanes) processes a "group"
// of horizontally adjacent blocks of one block-row; see blocks_per_group().
constexpr int kWave = 64;

// Blocks per group of the fused kernel for pattern size M (the solve layout
// is fixed per M in tsenor_kernels.hip).
int blocks_per_group(int M);

// Host-side launchers (tsenor_kernels.hip).  They return a hipError_t value.
// The fused kernel runs the optional stages -- at most prm.polish_steps 2-opt
// swaps per block, then keeping job.prev where it is feasible and better (if
// non-null) -- in a separate instance, chosen when either is asked for.
int launch_mask(const MatJob& job, const Params& prm, int grid, void* stream);
int launch_round(const MatJob& job, const float* S, int64_t lds, int ls_steps, int grid,
                 void* stream);
// Exact optimum of every block by negative-cycle canceling from `start` (a
// feasible mask, or nullptr for a circulant start) into job.mask; per-block
// objectives (fp64, NaN if not proven within max_cancel cancellations) to obj
// when non-null.  One workgroup per (block-row, 32-column word).
int launch_exact(const MatJob& job, const uint32_t* start, double* obj, int max_cancel, int grid,
                 void* stream);
int launch_batched(const MatJob* jobs_dev, int count, int64_t total_groups, int M, int bf16,
                   const Params& prm, bool optional_stages, int grid, void* stream);
// Number of 64-lane workgroups of each kernel that fit on one CU at once.
int occupancy_mask(int M, int bf16, bool optional_stages);
int occupancy_round(int M, int bf16);
int occupancy_batched(int M, int bf16, bool optional_stages);
int occupancy_exact(int M, int bf16);
// Writes to *count (device) the number of non-finite elements of a row-major
// fp32 / bf16 matrix; two launches on `stream`.
int launch_count_nonfinite(const void* p, int bf16, int64_t rows, int64_t cols, int64_t ld,
                           int* count, int grid, void* stream);

// Measurement only (tsenor_bench.hip): the memory side of the mask search
// alone -- W read once by M x M blocks (M = 16 or 32; 16-byte aligned rows),
// block max of |W|, one bit per weight (2|W| >= block max) into `mask`
// ([rows][wpr] words).
int launch_memory_pass(const void* W, int bf16, int64_t rows, int64_t cols, int64_t ld, int M,
                       uint32_t* mask, int64_t wpr, void* stream);

// 2:4 consumer (tsenor_spmm.hip).
int launch_compress24(const uint16_t* W, int64_t ld, const uint32_t* mask, int64_t wpr,
                      int64_t rows, int64_t k, int trans, uint16_t* vals, uint32_t* meta, int* bad,
                      void* stream);
int launch_spmm24(const uint16_t* X, int64_t ldx, const uint16_t* vals, const uint32_t* meta,
                  float* Y, int64_t ldy, int64_t n, int64_t m, int64_t k, void* stream);

}  // namespace tsenor
