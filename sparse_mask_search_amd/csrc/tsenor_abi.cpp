// tsenor_abi.cpp -- the extern "C" boundary declared in include/tsenor.h.
//
// Host-side only: argument validation (before any HIP call), the per-device
// cached buffers (batched descriptor table, previous-mask copy), launch
// geometry, and the stream ordering that makes the shared buffers safe.  The arithmetic of the method lives entirely in the
// kernels (tsenor_kernels.hip).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "tsenor.h"
#include "tsenor_bench.h"
#include "tsenor_internal.h"

using tsenor::MatJob;
using tsenor::Params;

namespace {

thread_local char g_last_error[256] = "";

int hip_fail(hipError_t e, const char* where) {
    std::snprintf(g_last_error, sizeof g_last_error, "%s: %s", where, hipGetErrorString(e));
    return TSENOR_ERR_HIP;
}

constexpr int kMaxDevices = 64;
// Pinned staging buffers for the batched descriptor table, used in turn: a
// call waits on the host only while the upload from its buffer, issued
// kStageRing calls earlier, is still queued behind unfinished work.
constexpr int kStageRing = 8;

struct DeviceState {
    std::mutex mu;
    bool init = false;              // num_cu and the occupancy tables
    bool ordered = false;           // `last` exists
    int num_cu = 0;
    hipEvent_t last = nullptr;      // completion of the newest launch that used this state
    MatJob* jobs_dev = nullptr;     // batched descriptor table (device)
    MatJob* jobs_host[kStageRing] = {};   // pinned staging copies, used in turn
    hipEvent_t jobs_up[kStageRing] = {};  // completion of the upload from each
    int jobs_next = 0;
    size_t jobs_cap = 0;
    int occ_mask[2][33] = {};      // the fused kernel without / with the optional stages
    int occ_mask_opt[2][33] = {};
    int occ_round[2][33] = {};
    int occ_batched[2][33] = {};
    int occ_batched_opt[2][33] = {};
    int occ_exact[2][33] = {};
    uint32_t* prev_copy = nullptr;  // copy of a previous mask that aliases the output
    size_t prev_cap = 0;            // words
    int* dbg_count = nullptr;       // debug checks: device counter and its pinned host copy
    int* dbg_host = nullptr;
};
DeviceState g_dev[kMaxDevices];

bool valid_m(int M) { return M == 4 || M == 8 || M == 16 || M == 32; }

int check_matrix(const void* W, int dtype, int64_t rows, int64_t cols, int64_t ld, int N, int M,
                 const void* mask) {
    if (W == nullptr || mask == nullptr) return TSENOR_ERR_NULL;
    if (dtype != TSENOR_F32 && dtype != TSENOR_BF16) return TSENOR_ERR_DTYPE;
    if (!valid_m(M) || N < 1 || N > M) return TSENOR_ERR_NM;
    if (rows <= 0 || cols <= 0 || rows % M != 0 || cols % M != 0 || ld < cols)
        return TSENOR_ERR_SHAPE;
    // keep every element offset inside int64 comfortably
    if (rows > (int64_t(1) << 40) / ld) return TSENOR_ERR_SHAPE;
    return TSENOR_OK;
}

int check_params(float tau, int iters, int ls_steps) {
    if (!std::isfinite(tau) || tau < 0.0f || iters < 1 || ls_steps < 0) return TSENOR_ERR_PARAM;
    return TSENOR_OK;
}

MatJob make_job(const void* W, int dtype, int64_t rows, int64_t cols, int64_t ld, int N, int M,
                uint32_t* mask, float* frac) {
    MatJob j;
    j.W = W;
    j.mask = mask;
    j.frac = frac;
    j.prev = nullptr;
    j.rows = rows;
    j.cols = cols;
    j.ld = ld;
    j.wpr = (cols + 31) / 32;
    j.group_begin = 0;
    j.N = N;
    j.M = M;
    j.bf16 = dtype == TSENOR_BF16 ? 1 : 0;
    const int64_t es = j.bf16 ? 2 : 4;
    j.aligned = ((reinterpret_cast<uintptr_t>(W) & 15u) == 0 && (ld * es) % 16 == 0) ? 1 : 0;
    return j;
}

int64_t groups_of(const MatJob& j) {
    const int64_t bpg = tsenor::blocks_per_group(j.M);
    const int64_t nbc = j.cols / j.M;
    return (j.rows / j.M) * ((nbc + bpg - 1) / bpg);
}

// Lock the current device's state and fill in its launch geometry (CU count,
// occupancy of every kernel).  Creates no HIP object and allocates nothing.
int acquire_geometry(DeviceState** out, std::unique_lock<std::mutex>* lk) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return hip_fail(hipErrorInvalidDevice, "device index");
    DeviceState& st = g_dev[dev];
    *lk = std::unique_lock<std::mutex>(st.mu);
    if (!st.init) {
        e = hipDeviceGetAttribute(&st.num_cu, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
        for (int b = 0; b < 2; ++b)
            for (int M : {4, 8, 16, 32}) {
                st.occ_mask[b][M] = tsenor::occupancy_mask(M, b, false);
                st.occ_mask_opt[b][M] = tsenor::occupancy_mask(M, b, true);
                st.occ_round[b][M] = tsenor::occupancy_round(M, b);
                st.occ_batched[b][M] = tsenor::occupancy_batched(M, b, false);
                st.occ_batched_opt[b][M] = tsenor::occupancy_batched(M, b, true);
                st.occ_exact[b][M] = tsenor::occupancy_exact(M, b);
            }
        st.init = true;
    }
    *out = &st;
    return TSENOR_OK;
}

// Flags of the library's internal events.  They only order work on one
// device (launches sharing the cached buffers, uploads from a staging buffer)
// and let the host wait for completion before reusing or freeing a buffer;
// nothing reads device memory through them, so they skip the system-scope
// cache writeback and invalidation that a default event performs at every
// record (measured: 5 us per 2:4 call, 29 us per 4:8 call that had left 64 MB
// of dirty lines).
constexpr unsigned kEventFlags = hipEventDisableTiming | hipEventDisableSystemFence;

// acquire_geometry, plus the event that orders the launches sharing the
// cached buffers.
int acquire(DeviceState** out, std::unique_lock<std::mutex>* lk) {
    int code = acquire_geometry(out, lk);
    if (code != TSENOR_OK) return code;
    DeviceState& st = **out;
    if (!st.ordered) {
        hipError_t e = hipEventCreateWithFlags(&st.last, kEventFlags);
        if (e != hipSuccess) return hip_fail(e, "hipEventCreate");
        st.ordered = true;
    }
    return TSENOR_OK;
}

// Ensure the cached copy buffer for previous masks holds `words` words.
// Growing waits for every earlier launch that may still read the old buffer.
int ensure_prev_copy(DeviceState& st, size_t words) {
    if (st.prev_cap >= words) return TSENOR_OK;
    hipError_t e;
    if (st.prev_copy != nullptr) {
        e = hipEventSynchronize(st.last);
        if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
        (void)hipFree(st.prev_copy);
        st.prev_copy = nullptr;
        st.prev_cap = 0;
    }
    e = hipMalloc(&st.prev_copy, words * sizeof(uint32_t));
    if (e != hipSuccess) {
        st.prev_copy = nullptr;
        return hip_fail(e, "hipMalloc(previous mask copy)");
    }
    st.prev_cap = words;
    return TSENOR_OK;
}

// True when the byte ranges [a, a + an) and [b, b + bn) share a byte.
bool overlaps(const void* a, size_t an, const void* b, size_t bn) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return an > 0 && bn > 0 && x < y + bn && y < x + an;
}

size_t mask_words(int64_t rows, int64_t cols) { return (size_t)rows * (size_t)((cols + 31) / 32); }

int64_t clamp_grid(int64_t groups, int num_cu, int occ) {
    int64_t cap = (int64_t)num_cu * (occ > 0 ? occ : 1);
    return groups < cap ? groups : cap;
}

int order_and_record_begin(DeviceState& st, hipStream_t s) {
    hipError_t e = hipStreamWaitEvent(s, st.last, 0);
    return e == hipSuccess ? TSENOR_OK : hip_fail(e, "hipStreamWaitEvent");
}

int record_end(DeviceState& st, hipStream_t s) {
    hipError_t e = hipEventRecord(st.last, s);
    return e == hipSuccess ? TSENOR_OK : hip_fail(e, "hipEventRecord");
}

// TSENOR_DEBUG_CHECKS=1 (read at every call): inputs are scanned for
// non-finite values on the device before anything else is launched, and the
// call waits for the answer (so it cannot be captured into a graph).
bool debug_checks() {
    const char* v = std::getenv("TSENOR_DEBUG_CHECKS");
    return v != nullptr && v[0] == '1' && v[1] == '\0';
}

int check_finite(DeviceState& st, hipStream_t s, const void* p, int bf16, int64_t rows,
                 int64_t cols, int64_t ld) {
    hipError_t e;
    if (st.dbg_count == nullptr) {
        e = hipMalloc(&st.dbg_count, sizeof(int));
        if (e != hipSuccess) {
            st.dbg_count = nullptr;
            return hip_fail(e, "hipMalloc(debug counter)");
        }
    }
    if (st.dbg_host == nullptr) {
        e = hipHostMalloc(reinterpret_cast<void**>(&st.dbg_host), sizeof(int), hipHostMallocDefault);
        if (e != hipSuccess) {
            st.dbg_host = nullptr;
            return hip_fail(e, "hipHostMalloc(debug counter)");
        }
    }
    const int64_t n = rows * cols;
    const int64_t cap = (int64_t)st.num_cu * 8;
    const int64_t grid = (n + 255) / 256 < cap ? (n + 255) / 256 : cap;
    e = (hipError_t)tsenor::launch_count_nonfinite(p, bf16, rows, cols, ld, st.dbg_count, (int)grid, s);
    if (e != hipSuccess) return hip_fail(e, "debug check launch");
    e = hipMemcpyAsync(st.dbg_host, st.dbg_count, sizeof(int), hipMemcpyDeviceToHost, s);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(debug counter)");
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize(debug check)");
    return *st.dbg_host != 0 ? TSENOR_ERR_NONFINITE : TSENOR_OK;
}

}  // namespace

extern "C" {

int tsenor_mask(const void* W, int dtype, int64_t rows, int64_t cols, int64_t ld, int N, int M,
                float tau, int iters, int ls_steps, uint32_t* mask_out, float* frac_out,
                void* stream) {
    return tsenor_mask_ex(W, dtype, rows, cols, ld, N, M, tau, iters, ls_steps, 0, nullptr,
                          mask_out, frac_out, stream);
}

int tsenor_mask_ex(const void* W, int dtype, int64_t rows, int64_t cols, int64_t ld, int N,
                   int M, float tau, int iters, int ls_steps, int polish_steps,
                   const uint32_t* prev_mask, uint32_t* mask_out, float* frac_out,
                   void* stream) {
    int st_code = check_matrix(W, dtype, rows, cols, ld, N, M, mask_out);
    if (st_code != TSENOR_OK) return st_code;
    st_code = check_params(tau, iters, ls_steps);
    if (st_code != TSENOR_OK) return st_code;
    if (polish_steps < 0) return TSENOR_ERR_PARAM;

    DeviceState* st = nullptr;
    std::unique_lock<std::mutex> lk;
    if ((st_code = acquire(&st, &lk)) != TSENOR_OK) return st_code;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (debug_checks() &&
        (st_code = check_finite(*st, s, W, dtype == TSENOR_BF16, rows, cols, ld)) != TSENOR_OK)
        return st_code;
    MatJob job = make_job(W, dtype, rows, cols, ld, N, M, mask_out, frac_out);
    job.prev = prev_mask;
    // the optional stages run inside the fused kernel, in its second instance
    const bool optional = polish_steps > 0 || prev_mask != nullptr;
    const int64_t grid = clamp_grid(
        groups_of(job), st->num_cu,
        optional ? st->occ_mask_opt[job.bf16][M] : st->occ_mask[job.bf16][M]);
    Params prm;
    prm.tau_log2e = (float)((double)tau * 1.4426950408889634);
    prm.iters = iters;
    prm.ls_steps = ls_steps;
    prm.polish_steps = polish_steps;
    const size_t words = (size_t)rows * (size_t)job.wpr;
    // a previous mask that the solve overwrites (any overlap with the output)
    // is copied first
    const bool prev_alias = prev_mask != nullptr &&
                            overlaps(prev_mask, words * 4, mask_out, words * 4);
    if (!prev_alias) {
        // No cached buffer is involved (the kernel needs no workspace), so the
        // launch is not ordered after the device's other calls: the stream
        // wait and event record that ordering takes cost ~1 us per call
        // (6.5% of a 2:4 launch on a 1024 x 1024 matrix).
        const hipError_t e = (hipError_t)tsenor::launch_mask(job, prm, (int)grid, stream);
        return e == hipSuccess ? TSENOR_OK : hip_fail(e, "mask kernel launch");
    }
    if ((st_code = ensure_prev_copy(*st, words)) != TSENOR_OK) return st_code;
    if ((st_code = order_and_record_begin(*st, s)) != TSENOR_OK) return st_code;
    hipError_t e = hipMemcpyAsync(st->prev_copy, prev_mask, words * sizeof(uint32_t),
                                  hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) {
        (void)record_end(*st, s);
        return hip_fail(e, "hipMemcpyAsync(previous mask)");
    }
    job.prev = st->prev_copy;
    e = (hipError_t)tsenor::launch_mask(job, prm, (int)grid, stream);
    if (e != hipSuccess) {
        (void)record_end(*st, s);
        return hip_fail(e, "mask kernel launch");
    }
    return record_end(*st, s);
}

int tsenor_mask_noalloc(const void* W, int dtype, int64_t rows, int64_t cols, int64_t ld,
                        int N, int M, float tau, int iters, int ls_steps, uint32_t* mask_out,
                        float* frac_out, void* stream) {
    int st_code = check_matrix(W, dtype, rows, cols, ld, N, M, mask_out);
    if (st_code != TSENOR_OK) return st_code;
    st_code = check_params(tau, iters, ls_steps);
    if (st_code != TSENOR_OK) return st_code;
    DeviceState* st = nullptr;
    std::unique_lock<std::mutex> lk;
    if ((st_code = acquire_geometry(&st, &lk)) != TSENOR_OK) return st_code;
    MatJob job = make_job(W, dtype, rows, cols, ld, N, M, mask_out, frac_out);
    const int64_t grid = clamp_grid(groups_of(job), st->num_cu, st->occ_mask[job.bf16][M]);
    Params prm;
    prm.tau_log2e = (float)((double)tau * 1.4426950408889634);
    prm.iters = iters;
    prm.ls_steps = ls_steps;
    prm.polish_steps = 0;
    hipError_t e = (hipError_t)tsenor::launch_mask(job, prm, (int)grid, stream);
    return e == hipSuccess ? TSENOR_OK : hip_fail(e, "mask kernel launch");
}

int tsenor_exact(const void* W, int dtype, int64_t rows, int64_t cols, int64_t ld, int N, int M,
                 const uint32_t* start_mask, int max_cancel, uint32_t* mask_out,
                 double* objective_out, void* stream) {
    int st_code = check_matrix(W, dtype, rows, cols, ld, N, M, mask_out);
    if (st_code != TSENOR_OK) return st_code;
    if (max_cancel < 0) return TSENOR_ERR_PARAM;
    DeviceState* st = nullptr;
    std::unique_lock<std::mutex> lk;
    if ((st_code = acquire(&st, &lk)) != TSENOR_OK) return st_code;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (debug_checks() &&
        (st_code = check_finite(*st, s, W, dtype == TSENOR_BF16, rows, cols, ld)) != TSENOR_OK)
        return st_code;
    MatJob job = make_job(W, dtype, rows, cols, ld, N, M, mask_out, nullptr);
    const int64_t units = (rows / M) * job.wpr;
    const int64_t grid = clamp_grid(units, st->num_cu, st->occ_exact[job.bf16][M]);
    if ((st_code = order_and_record_begin(*st, s)) != TSENOR_OK) return st_code;
    hipError_t e = (hipError_t)tsenor::launch_exact(job, start_mask, objective_out, max_cancel,
                                                    (int)grid, stream);
    if (e != hipSuccess) {
        (void)record_end(*st, s);
        return hip_fail(e, "exact kernel launch");
    }
    return record_end(*st, s);
}

int tsenor_compress24(const void* W, int64_t rows, int64_t cols, int64_t ld,
                      const uint32_t* mask, int transpose, uint16_t* values_out,
                      uint32_t* meta_out, int* bad_groups, void* stream) {
    if (W == nullptr || mask == nullptr || values_out == nullptr || meta_out == nullptr)
        return TSENOR_ERR_NULL;
    if (transpose != 0 && transpose != 1) return TSENOR_ERR_PARAM;
    if (rows <= 0 || cols <= 0 || ld < cols || rows > (int64_t(1) << 40) / ld) return TSENOR_ERR_SHAPE;
    const int64_t arows = transpose ? cols : rows, k = transpose ? rows : cols;
    if (k % 32 != 0) return TSENOR_ERR_SHAPE;
    const int64_t wpr = (cols + 31) / 32;
    hipError_t e = (hipError_t)tsenor::launch_compress24(
        static_cast<const uint16_t*>(W), ld, mask, wpr, arows, k, transpose, values_out, meta_out,
        bad_groups, stream);
    return e == hipSuccess ? TSENOR_OK : hip_fail(e, "compress24 kernel launch");
}

int tsenor_spmm24(const void* X, int64_t n, int64_t ldx, const uint16_t* values,
                  const uint32_t* meta, int64_t m, int64_t k, float* Y, int64_t ldy,
                  void* stream) {
    if (X == nullptr || values == nullptr || meta == nullptr || Y == nullptr) return TSENOR_ERR_NULL;
    if (n <= 0 || m <= 0 || k <= 0 || n % 128 != 0 || m % 128 != 0 || k % 32 != 0 || ldx < k ||
        ldy < m || ldx % 8 != 0 || ldy % 4 != 0)
        return TSENOR_ERR_SHAPE;
    if ((reinterpret_cast<uintptr_t>(X) & 15u) != 0 || (reinterpret_cast<uintptr_t>(Y) & 15u) != 0 ||
        (reinterpret_cast<uintptr_t>(values) & 7u) != 0 || (reinterpret_cast<uintptr_t>(meta) & 3u) != 0)
        return TSENOR_ERR_SHAPE;
    hipError_t e = (hipError_t)tsenor::launch_spmm24(static_cast<const uint16_t*>(X), ldx, values,
                                                     meta, Y, ldy, n, m, k, stream);
    return e == hipSuccess ? TSENOR_OK : hip_fail(e, "spmm24 kernel launch");
}

int tsenor_round(const float* S, int64_t lds, const void* W, int dtype, int64_t rows,
                 int64_t cols, int64_t ld, int N, int M, int ls_steps, uint32_t* mask_out,
                 void* stream) {
    if (S == nullptr) return TSENOR_ERR_NULL;
    int st_code = check_matrix(W, dtype, rows, cols, ld, N, M, mask_out);
    if (st_code != TSENOR_OK) return st_code;
    if (lds < cols) return TSENOR_ERR_SHAPE;
    if (ls_steps < 0) return TSENOR_ERR_PARAM;

    DeviceState* st = nullptr;
    std::unique_lock<std::mutex> lk;
    if ((st_code = acquire(&st, &lk)) != TSENOR_OK) return st_code;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (debug_checks() &&
        ((st_code = check_finite(*st, s, W, dtype == TSENOR_BF16, rows, cols, ld)) != TSENOR_OK ||
         (st_code = check_finite(*st, s, S, 0, rows, cols, lds)) != TSENOR_OK))
        return st_code;
    MatJob job = make_job(W, dtype, rows, cols, ld, N, M, mask_out, nullptr);
    const int64_t per_pass = tsenor::kWave / M;
    const int64_t nbc = cols / M;
    const int64_t groups = (rows / M) * ((nbc + per_pass - 1) / per_pass);
    const int64_t grid = clamp_grid(groups, st->num_cu, st->occ_round[job.bf16][M]);
    if ((st_code = order_and_record_begin(*st, s)) != TSENOR_OK) return st_code;
    hipError_t e = (hipError_t)tsenor::launch_round(job, S, lds, ls_steps, (int)grid, stream);
    if (e != hipSuccess) {
        (void)record_end(*st, s);
        return hip_fail(e, "round kernel launch");
    }
    return record_end(*st, s);
}

int tsenor_mask_batched(const tsenor_matrix* mats, int count, float tau, int iters, int ls_steps,
                        void* stream) {
    return tsenor_mask_batched_ex(mats, count, tau, iters, ls_steps, 0, nullptr, stream);
}

int tsenor_mask_batched_ex(const tsenor_matrix* mats, int count, float tau, int iters,
                           int ls_steps, int polish_steps, const uint32_t* const* prev_masks,
                           void* stream) {
    if (count < 0 || polish_steps < 0) return TSENOR_ERR_PARAM;
    if (count > 0 && mats == nullptr) return TSENOR_ERR_NULL;
    int st_code = check_params(tau, iters, ls_steps);
    if (st_code != TSENOR_OK) return st_code;
    for (int i = 0; i < count; ++i) {
        const tsenor_matrix& m = mats[i];
        st_code = check_matrix(m.W, m.dtype, m.rows, m.cols, m.ld, m.N, m.M, m.mask_out);
        if (st_code != TSENOR_OK) return st_code;
    }
    if (count == 0) return TSENOR_OK;

    DeviceState* st = nullptr;
    std::unique_lock<std::mutex> lk;
    if ((st_code = acquire(&st, &lk)) != TSENOR_OK) return st_code;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (debug_checks())
        for (int i = 0; i < count; ++i) {
            const tsenor_matrix& m = mats[i];
            st_code = check_finite(*st, s, m.W, m.dtype == TSENOR_BF16, m.rows, m.cols, m.ld);
            if (st_code != TSENOR_OK) return st_code;
        }
    hipError_t e;
    if (st->jobs_cap < (size_t)count) {
        // Growing (rare): wait for every launch that may read the device table
        // and every upload that may read a staging buffer, then reallocate.
        if (st->jobs_dev != nullptr) {
            e = hipEventSynchronize(st->last);
            if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
            (void)hipFree(st->jobs_dev);
            st->jobs_dev = nullptr;
        }
        for (int k = 0; k < kStageRing; ++k) {
            if (st->jobs_up[k] != nullptr) {
                e = hipEventSynchronize(st->jobs_up[k]);
                if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
            } else {
                e = hipEventCreateWithFlags(&st->jobs_up[k], kEventFlags);
                if (e != hipSuccess) return hip_fail(e, "hipEventCreate");
            }
            if (st->jobs_host[k] != nullptr) (void)hipHostFree(st->jobs_host[k]);
            st->jobs_host[k] = nullptr;
        }
        st->jobs_cap = 0;
        e = hipMalloc(&st->jobs_dev, sizeof(MatJob) * (size_t)count);
        if (e != hipSuccess) return hip_fail(e, "hipMalloc(descriptors)");
        for (int k = 0; k < kStageRing; ++k) {
            e = hipHostMalloc(reinterpret_cast<void**>(&st->jobs_host[k]),
                              sizeof(MatJob) * (size_t)count, hipHostMallocDefault);
            if (e != hipSuccess) return hip_fail(e, "hipHostMalloc(descriptors)");
        }
        st->jobs_cap = (size_t)count;
    }
    // This call's staging buffer: free once the upload that last read it has
    // run (normally long ago; the host blocks only when kStageRing batched
    // calls are queued behind unfinished work).
    const int ring = st->jobs_next;
    st->jobs_next = (ring + 1) % kStageRing;
    e = hipEventSynchronize(st->jobs_up[ring]);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize(staging)");
    MatJob* const table = st->jobs_host[ring];
    // Previous masks that any of the call's outputs overlaps are copied first,
    // back to back (the solve of one matrix may overwrite another's previous
    // mask before its optional stages read it); prev_eff[i] is what matrix i's
    // descriptor reads.
    const bool optional = polish_steps > 0 || prev_masks != nullptr;
    size_t alias_words = 0;
    std::vector<char> alias(count, 0);
    if (prev_masks != nullptr)
        for (int i = 0; i < count; ++i) {
            if (prev_masks[i] == nullptr) continue;
            const size_t words = mask_words(mats[i].rows, mats[i].cols);
            for (int j = 0; j < count && !alias[i]; ++j)
                alias[i] = overlaps(prev_masks[i], words * 4, mats[j].mask_out,
                                    mask_words(mats[j].rows, mats[j].cols) * 4);
            if (alias[i]) alias_words += words;
        }
    if (alias_words > 0 && (st_code = ensure_prev_copy(*st, alias_words)) != TSENOR_OK)
        return st_code;
    std::vector<const uint32_t*> prev_eff(count, nullptr);
    if (prev_masks != nullptr) {
        size_t off = 0;
        for (int i = 0; i < count; ++i) {
            prev_eff[i] = prev_masks[i];
            if (!alias[i]) continue;
            prev_eff[i] = st->prev_copy + off;
            off += mask_words(mats[i].rows, mats[i].cols);
        }
    }
    // One launch per (M, dtype) class present; the class's descriptors are
    // contiguous in the table, in call order, with group ids counted from 0.
    struct Class { int M, bf16, first, n; int64_t groups, grid; };
    Class cls[8];
    int ncls = 0, filled = 0;
    for (int M : {32, 16, 8, 4})
        for (int b = 0; b < 2; ++b) {
            Class c{M, b, filled, 0, 0, 0};
            for (int i = 0; i < count; ++i) {
                const tsenor_matrix& m = mats[i];
                if (m.M != M || (m.dtype == TSENOR_BF16 ? 1 : 0) != b) continue;
                MatJob j = make_job(m.W, m.dtype, m.rows, m.cols, m.ld, m.N, m.M, m.mask_out,
                                    m.frac_out);
                j.prev = prev_eff[i];
                j.group_begin = c.groups;
                c.groups += groups_of(j);
                table[filled++] = j;
                ++c.n;
            }
            if (c.n == 0) continue;
            c.grid = clamp_grid(c.groups, st->num_cu,
                                optional ? st->occ_batched_opt[b][M] : st->occ_batched[b][M]);
            cls[ncls++] = c;
        }
    Params prm;
    prm.tau_log2e = (float)((double)tau * 1.4426950408889634);
    prm.iters = iters;
    prm.ls_steps = ls_steps;
    prm.polish_steps = polish_steps;
    if ((st_code = order_and_record_begin(*st, s)) != TSENOR_OK) return st_code;
    e = hipMemcpyAsync(st->jobs_dev, table, sizeof(MatJob) * (size_t)count,
                       hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(descriptors)");
    e = hipEventRecord(st->jobs_up[ring], s);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord(staging)");
    for (int i = 0; i < count; ++i) {
        if (!alias[i]) continue;
        e = hipMemcpyAsync(const_cast<uint32_t*>(prev_eff[i]), prev_masks[i],
                           mask_words(mats[i].rows, mats[i].cols) * sizeof(uint32_t),
                           hipMemcpyDeviceToDevice, s);
        if (e != hipSuccess) {
            (void)record_end(*st, s);
            return hip_fail(e, "hipMemcpyAsync(previous mask)");
        }
    }
    // The launches run in stream order after the descriptor upload.
    for (int k = 0; k < ncls; ++k) {
        const Class& c = cls[k];
        e = (hipError_t)tsenor::launch_batched(st->jobs_dev + c.first, c.n, c.groups, c.M, c.bf16,
                                               prm, optional, (int)c.grid, stream);
        if (e != hipSuccess) {
            // earlier classes may be in flight: keep the ordering
            (void)record_end(*st, s);
            return hip_fail(e, "batched kernel launch");
        }
    }
    return record_end(*st, s);
}

int tsenor_bench_memory_pass(const void* W, int dtype, int64_t rows, int64_t cols, int64_t ld,
                             int M, uint32_t* mask_out, void* stream) {
    if (W == nullptr || mask_out == nullptr) return TSENOR_ERR_NULL;
    if (dtype != TSENOR_F32 && dtype != TSENOR_BF16) return TSENOR_ERR_DTYPE;
    if (M != 16 && M != 32) return TSENOR_ERR_NM;
    const int64_t es = dtype == TSENOR_BF16 ? 2 : 4;
    if (rows <= 0 || cols <= 0 || rows % M != 0 || cols % M != 0 || ld < cols ||
        rows > (int64_t(1) << 40) / ld || (reinterpret_cast<uintptr_t>(W) & 15u) != 0 ||
        (ld * es) % 16 != 0)
        return TSENOR_ERR_SHAPE;
    hipError_t e = (hipError_t)tsenor::launch_memory_pass(W, dtype == TSENOR_BF16, rows, cols, ld,
                                                          M, mask_out, (cols + 31) / 32, stream);
    return e == hipSuccess ? TSENOR_OK : hip_fail(e, "memory pass kernel launch");
}

const char* tsenor_status_str(int status) {
    switch (status) {
        case TSENOR_OK: return "ok";
        case TSENOR_ERR_NULL: return "required pointer is NULL";
        case TSENOR_ERR_SHAPE: return "bad shape (rows/cols must be positive multiples of M, ld >= cols)";
        case TSENOR_ERR_NM: return "bad N:M (M in {4,8,16,32}, 1 <= N <= M)";
        case TSENOR_ERR_PARAM: return "bad parameter (tau finite >= 0, iters >= 1, ls_steps >= 0)";
        case TSENOR_ERR_DTYPE: return "bad dtype (TSENOR_F32 or TSENOR_BF16)";
        case TSENOR_ERR_HIP: return "HIP runtime error (see tsenor_last_error)";
        case TSENOR_ERR_NONFINITE: return "input holds a non-finite value (TSENOR_DEBUG_CHECKS=1)";
        default: return "unknown status";
    }
}

const char* tsenor_last_error(void) { return g_last_error; }

int tsenor_version(void) { return 0x000100; }

}  // extern "C"
