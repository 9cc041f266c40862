/* Test driver (test infrastructure): runs every exported routine of the CPU
 * oracle on small seeded inputs, so that a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_oracle_sanitize.py) reports any
 * out-of-bounds access, use of uninitialised stack or undefined arithmetic.
 * Prints a checksum line; exit status 0 when every call returned 0.        */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_dykstra(const float* W, int64_t rows, int64_t cols, int64_t ld, int N, int M,
                   double tau, int iters, double* S64, float* S32, int nthreads);
int oracle_dykstra_blocks_f32(const float* W, int64_t rows, int64_t cols, int64_t ld, int N,
                              int M, float tau, int iters, const int64_t* block_ids,
                              int64_t nblocks, float* S, int nthreads);
int oracle_round(const float* S32, int64_t lds, const float* W, int64_t ld, int64_t rows,
                 int64_t cols, int N, int M, int ls_steps, uint32_t* mask, int64_t* stats,
                 int nthreads);
int oracle_round_ex(const float* S32, int64_t lds, const float* W, int64_t ld, int64_t rows,
                    int64_t cols, int N, int M, int ls_steps, int polish_steps,
                    const uint32_t* prev_mask, uint32_t* mask, int64_t* stats, int nthreads);
int oracle_round_block(const float* S32, const float* A, int N, int M, int ls_steps,
                       uint8_t* Z, int* info, uint8_t* Zgreedy, float* move_scores,
                       int* move_ijs);
int oracle_exact_opt_blocks(const float* W, int64_t rows, int64_t cols, int64_t ld, int N,
                            int M, const int64_t* block_ids, int64_t nblocks, double* opt,
                            int nthreads);

static uint64_t state = 0x9E3779B97F4A7C15ull;
static double uniform(void) { /* splitmix64 */
    uint64_t z = (state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return (double)(z >> 11) * 0x1.0p-53;
}

int main(void) {
    int failures = 0;
    double checksum = 0.0;
    const int Ms[4] = {4, 8, 16, 32};
    for (int t = 0; t < 4; ++t) {
        const int M = Ms[t], N = M / 2;
        const int64_t rows = 2 * M, cols = 3 * M, nb = 6, wpr = (cols + 31) / 32;
        float* W = malloc(sizeof(float) * rows * cols);
        double* S64 = malloc(sizeof(double) * rows * cols);
        float* S32 = malloc(sizeof(float) * rows * cols);
        float* Sf = malloc(sizeof(float) * nb * M * M);
        uint32_t* mask = calloc((size_t)(rows * wpr), sizeof(uint32_t));
        uint32_t* mask2 = calloc((size_t)(rows * wpr), sizeof(uint32_t));
        double opt[6];
        int64_t ids[6] = {0, 1, 2, 3, 4, 5}, stats[6] = {0};
        for (int64_t k = 0; k < rows * cols; ++k)
            W[k] = (float)((uniform() - 0.5) * (uniform() < 0.01 ? 40.0 : 1.0));
        for (int k = 0; k < M; ++k) W[k * cols + k] = 0.0f; /* a few exact zeros */
        failures += oracle_dykstra(W, rows, cols, cols, N, M, 30.0, 40, S64, S32, 1) != 0;
        failures += oracle_dykstra_blocks_f32(W, rows, cols, cols, N, M, 30.0f, 40, ids, nb, Sf,
                                              1) != 0;
        failures += oracle_round(S32, cols, W, cols, rows, cols, N, M, M, mask, stats, 1) != 0;
        failures += oracle_round_ex(S32, cols, W, cols, rows, cols, N, M, 2, 6, mask, mask2,
                                    stats, 1) != 0;
        failures += oracle_exact_opt_blocks(W, rows, cols, cols, N, M, ids, nb, opt, 1) != 0;
        {
            float A[1024], S[1024], sc[1024];
            uint8_t Z[1024], Zg[1024];
            int info[3], ijs[4096];
            for (int i = 0; i < M; ++i)
                for (int j = 0; j < M; ++j) {
                    A[i * M + j] = fabsf(W[i * cols + j]);
                    S[i * M + j] = S32[i * cols + j];
                }
            failures += oracle_round_block(S, A, N, M, M, Z, info, Zg, sc, ijs) != 0;
            checksum += info[0] + info[1] + info[2];
        }
        for (int64_t k = 0; k < rows * cols; ++k) checksum += S64[k];
        for (int k = 0; k < nb * M * M; ++k) checksum += Sf[k];
        for (int64_t k = 0; k < rows * wpr; ++k) checksum += (double)(mask[k] & 0xFFu) + (mask2[k] >> 24);
        for (int k = 0; k < nb; ++k) checksum += opt[k];
        free(W); free(S64); free(S32); free(Sf); free(mask); free(mask2);
    }
    printf("checksum %.6f failures %d\n", checksum, failures);
    return failures != 0;
}
