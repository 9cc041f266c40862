/*
 * tsenor_oracle.c -- plain, slow, obviously-correct CPU oracle for transposable
 * N:M mask search (TSENOR-style).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or load
 * this code: only the test-suite, the smoke check and the CPU-baseline leg of the
 * benchmark do.  It shares no source, header, table or helper with the HIP
 * library; the two meet only through the seeded input generators.
 *
 * Source of the method: the pith.science review of "TSENOR: Highly-Efficient
 * Algorithm for Finding Transposable N:M Sparse Masks" (Meng, Makni, Mazumder,
 * arXiv 2505.23949) -- sections "What carries the argument" and "Extended
 * reading notes / Core claim".  Where that page leaves a step open, the reading
 * taken is stated next to the step.
 *
 * Precision: every Dykstra quantity is fp64 with natural logarithms; the
 * rounding stage consumes the fp32 fractional matrix S32 and scores moves in
 * fp32 exactly as (a + b) - c, round-to-nearest, no contraction.
 *
 * Build: gcc -O2 -fopenmp -fPIC -shared -ffp-contract=off (no fast-math).
 */
#define _GNU_SOURCE
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <float.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_OK 0
#define OR_ERR_ARG 1
#define OR_ERR_NONFINITE 2
#define OR_ERR_INVARIANT 3

/* ------------------------------------------------------------------------ */
/* Block gather (problem (1)/(2) of the review's "Core claim"): a block is the
 * M x M sub-matrix rows [bi*M, bi*M+M) x cols [bj*M, bj*M+M); its scores are
 * A = |W| (fp32, exact).                                                    */
static void gather_abs(const float* W, int64_t ld, int64_t bi, int64_t bj, int M,
                       float* A) {
    for (int i = 0; i < M; ++i)
        for (int j = 0; j < M; ++j)
            A[i * M + j] = fabsf(W[(bi * M + i) * ld + (bj * M + j)]);
}

/* ------------------------------------------------------------------------ */
/* Entropic capacitated OT by Dykstra's alternating KL projections, log space
 * ("What carries the argument"; "Core claim"):
 *   scores  What = A / max(A)  (max over the block -- the page leaves the
 *           normalisation open; an all-zero block gives What = 0)
 *   start   X = tau * What, Q = 0   (the Gibbs kernel exp(tau*What); tau
 *           multiplies the normalised scores)
 *   repeat T times, in this order (one cycle = C1, C2, C3; exactly T cycles,
 *   no stopping test)
 *     C1  row normalisation:    X_ij += ln N - LSE_j' X_ij'
 *     C2  column normalisation: X_ij += ln N - LSE_i' X_i'j
 *     C3  clip at 1 with the Dykstra correction:
 *         Y = X + Q;  X = min(Y, 0);  Q = Y - X
 *   return S = exp(X) in [0, 1].
 * Only the clip carries a correction term: C1/C2 corrections are row/column
 * constants that the next C1/C2 removes, so the iterates are the same.      */
static double lse(const double* x, int n, int stride) {
    double mx = -INFINITY;
    for (int k = 0; k < n; ++k)
        if (x[k * stride] > mx) mx = x[k * stride];
    double s = 0.0;
    for (int k = 0; k < n; ++k) s += exp(x[k * stride] - mx);
    return mx + log(s);
}

static int dykstra_block(const float* A, int N, int M, double tau, int iters,
                         double* X, double* Q) {
    const int n = M * M;
    double m = 0.0;
    for (int k = 0; k < n; ++k) {
        if (!isfinite(A[k])) return OR_ERR_NONFINITE;
        if ((double)A[k] > m) m = (double)A[k];
    }
    for (int k = 0; k < n; ++k) {
        double what = (m > 0.0) ? (double)A[k] / m : 0.0;
        X[k] = tau * what;
        Q[k] = 0.0;
    }
    const double lnN = log((double)N);
    for (int t = 0; t < iters; ++t) {
        for (int i = 0; i < M; ++i) { /* C1 */
            double a = lnN - lse(X + i * M, M, 1);
            for (int j = 0; j < M; ++j) X[i * M + j] += a;
        }
        for (int j = 0; j < M; ++j) { /* C2 */
            double b = lnN - lse(X + j, M, M);
            for (int i = 0; i < M; ++i) X[i * M + j] += b;
        }
        for (int k = 0; k < n; ++k) { /* C3 */
            double y = X[k] + Q[k];
            double x = (y < 0.0) ? y : 0.0;
            Q[k] = y - x;
            X[k] = x;
        }
    }
    for (int k = 0; k < n; ++k) X[k] = exp(X[k]); /* S, overwrites X */
    return OR_OK;
}

/* The same steps in fp32 (single-precision values, expf/logf, natural log):
 * the method's own sensitivity to fp32 arithmetic.  Comparing its S with the
 * fp64 S above bounds how far any fp32 implementation of these steps may
 * drift from the fp64 result for reasons that lie in the iteration itself
 * rather than in an implementation.                                        */
static float lse_f32(const float* x, int n, int stride) {
    float mx = -INFINITY;
    for (int k = 0; k < n; ++k)
        if (x[k * stride] > mx) mx = x[k * stride];
    float s = 0.0f;
    for (int k = 0; k < n; ++k) s += expf(x[k * stride] - mx);
    return mx + logf(s);
}

static int dykstra_block_f32(const float* A, int N, int M, float tau, int iters, float* X,
                             float* Q) {
    const int n = M * M;
    float m = 0.0f;
    for (int k = 0; k < n; ++k) {
        if (!isfinite(A[k])) return OR_ERR_NONFINITE;
        if (A[k] > m) m = A[k];
    }
    for (int k = 0; k < n; ++k) {
        float what = (m > 0.0f) ? A[k] / m : 0.0f;
        X[k] = tau * what;
        Q[k] = 0.0f;
    }
    const float lnN = logf((float)N);
    for (int t = 0; t < iters; ++t) {
        for (int i = 0; i < M; ++i) { /* C1 */
            float a = lnN - lse_f32(X + i * M, M, 1);
            for (int j = 0; j < M; ++j) X[i * M + j] += a;
        }
        for (int j = 0; j < M; ++j) { /* C2 */
            float b = lnN - lse_f32(X + j, M, M);
            for (int i = 0; i < M; ++i) X[i * M + j] += b;
        }
        for (int k = 0; k < n; ++k) { /* C3 */
            float y = X[k] + Q[k];
            float x = (y < 0.0f) ? y : 0.0f;
            Q[k] = y - x;
            X[k] = x;
        }
    }
    for (int k = 0; k < n; ++k) X[k] = expf(X[k]);
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Rounding ("What carries the argument": sort descending, greedy within the
 * row/column budgets, then a local search on the swap score).
 *
 * R1 greedy   order all M^2 entries by (S32 descending, i*M+j ascending: the
 *             page gives no tie rule); accept (i,j) iff r_i < N and c_j < N.
 * R2 search   (<= L moves; one move per step, the best over all deficient
 *             pairs -- the page fixes neither): over every deficient row i, deficient
 *             column j and (i',j') with Z_i'j' = 1, Z_ij' = 0, Z_i'j = 0,
 *             score = fl32(fl32(A_ij' + A_i'j) - A_i'j') on raw |W|; take the
 *             maximum, ties to the smallest (i, j, i', j'); apply the move
 *             (set Z_ij' = Z_i'j = 1, clear Z_i'j') only if score > 0, else
 *             stop.
 * R3 fill     (not on the page; it runs after the search, which only has
 *             work while a shortfall remains) while a shortfall remains:
 *             i = smallest deficient row,
 *             j = smallest deficient column; best (i',j') by the same score,
 *             ties to the smallest (i', j'); apply with no sign condition.
 * Invariant I (checked): Z_ij = 1 for every deficient row i and deficient
 * column j, after R1 and after every move.                                   */
typedef struct {
    const float* s;
} sort_ctx_t;

static int cmp_order(const void* pa, const void* pb, void* vctx) {
    const sort_ctx_t* ctx = (const sort_ctx_t*)vctx;
    int a = *(const int*)pa, b = *(const int*)pb;
    float sa = ctx->s[a], sb = ctx->s[b];
    if (sa > sb) return -1;
    if (sa < sb) return 1;
    return (a < b) ? -1 : (a > b) ? 1 : 0;
}

static int invariant_I(const uint8_t* Z, const int* r, const int* c, int N, int M) {
    for (int i = 0; i < M; ++i)
        if (r[i] < N)
            for (int j = 0; j < M; ++j)
                if (c[j] < N && !Z[i * M + j]) return 0;
    return 1;
}

/* info[0] = shortfall D after R1, info[1] = R2 moves, info[2] = R3 moves.
 * Optional traces, in the order the moves are applied: move_scores[k] the
 * fp32 score of move k, move_ijs[4k..4k+3] its (i, j, i', j').             */
static int round_block(const float* S, const float* A, int N, int M, int L,
                       uint8_t* Z, int* order, int* info, uint8_t* Zgreedy,
                       float* move_scores, int* move_ijs) {
    const int n = M * M;
    for (int k = 0; k < n; ++k) {
        if (!isfinite(S[k])) return OR_ERR_NONFINITE;
        order[k] = k;
        Z[k] = 0;
    }
    sort_ctx_t ctx = {S};
    qsort_r(order, (size_t)n, sizeof(int), cmp_order, &ctx);

    int r[64], c[64];
    for (int i = 0; i < M; ++i) r[i] = c[i] = 0;
    int ones = 0;
    for (int k = 0; k < n; ++k) { /* R1 */
        int i = order[k] / M, j = order[k] % M;
        if (r[i] < N && c[j] < N) {
            Z[order[k]] = 1;
            ++r[i];
            ++c[j];
            ++ones;
        }
    }
    int D = N * M - ones;
    info[0] = D;
    if (Zgreedy) memcpy(Zgreedy, Z, (size_t)n);
    info[1] = info[2] = 0;
    if (!invariant_I(Z, r, c, N, M)) return OR_ERR_INVARIANT;

    int moves = 0;
    while (D > 0 && moves < L) { /* R2 */
        int found = 0, bi = 0, bj = 0, bip = 0, bjp = 0;
        float best = 0.0f;
        for (int i = 0; i < M; ++i) {
            if (r[i] >= N) continue;
            for (int j = 0; j < M; ++j) {
                if (c[j] >= N) continue;
                for (int ip = 0; ip < M; ++ip)
                    for (int jp = 0; jp < M; ++jp) {
                        if (!Z[ip * M + jp] || Z[i * M + jp] || Z[ip * M + j]) continue;
                        volatile float sum = A[i * M + jp] + A[ip * M + j];
                        float s = sum - A[ip * M + jp];
                        if (!found || s > best) {
                            found = 1;
                            best = s;
                            bi = i; bj = j; bip = ip; bjp = jp;
                        }
                    }
            }
        }
        if (!found || !(best > 0.0f)) break;
        if (move_scores) move_scores[moves] = best;
        if (move_ijs) {
            move_ijs[4 * moves] = bi;
            move_ijs[4 * moves + 1] = bj;
            move_ijs[4 * moves + 2] = bip;
            move_ijs[4 * moves + 3] = bjp;
        }
        Z[bi * M + bjp] = 1;
        Z[bip * M + bj] = 1;
        Z[bip * M + bjp] = 0;
        ++r[bi];
        ++c[bj];
        --D;
        ++moves;
        if (!invariant_I(Z, r, c, N, M)) return OR_ERR_INVARIANT;
    }
    info[1] = moves;

    while (D > 0) { /* R3 */
        int i = 0, j = 0;
        while (r[i] >= N) ++i;
        while (c[j] >= N) ++j;
        int found = 0, bip = 0, bjp = 0;
        float best = 0.0f;
        for (int ip = 0; ip < M; ++ip)
            for (int jp = 0; jp < M; ++jp) {
                if (!Z[ip * M + jp] || Z[i * M + jp] || Z[ip * M + j]) continue;
                volatile float sum = A[i * M + jp] + A[ip * M + j];
                float s = sum - A[ip * M + jp];
                if (!found || s > best) {
                    found = 1;
                    best = s;
                    bip = ip; bjp = jp;
                }
            }
        if (!found) return OR_ERR_INVARIANT; /* cannot happen while I holds */
        if (move_scores) move_scores[info[1] + info[2]] = best;
        if (move_ijs) {
            const int k = info[1] + info[2];
            move_ijs[4 * k] = i;
            move_ijs[4 * k + 1] = j;
            move_ijs[4 * k + 2] = bip;
            move_ijs[4 * k + 3] = bjp;
        }
        Z[i * M + bjp] = 1;
        Z[bip * M + j] = 1;
        Z[bip * M + bjp] = 0;
        ++r[i];
        ++c[j];
        --D;
        ++info[2];
        if (!invariant_I(Z, r, c, N, M)) return OR_ERR_INVARIANT;
    }
    for (int i = 0; i < M; ++i)
        if (r[i] != N || c[i] != N) return OR_ERR_INVARIANT;
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Optional stages after R3 (the pages describe no such step; the readings
 * below are this oracle's own):
 *
 * R4 2-opt polish, at most K swaps.  A swap takes kept (i, j) and (i', j'),
 *    i < i', with Z_ij' = Z_i'j = 0, to (i, j') and (i', j); every row and
 *    column keeps its count.  Its gain is evaluated in fp32 as
 *    (A_ij' - A_i'j') + (A_i'j - A_ij), each difference rounded, then the sum.
 *    The best gain is taken, ties to the smallest (i, j, i', j'); it is applied
 *    only when > 0, else R4 ends.
 * R5 keep-better safeguard against a caller's previous mask P: if P has N
 *    ones in every row and column of the block and obj(P) > obj(Z), the block
 *    takes P.  obj(Z) = sum over rows i ascending of (sum over j ascending of
 *    A_ij Z_ij), both sums in fp64.                                          */
static int polish_block(const float* A, int M, int K, uint8_t* Z, float* gains) {
    int swaps = 0;
    while (swaps < K) {
        int found = 0, bi = 0, bj = 0, bip = 0, bjp = 0;
        float best = 0.0f;
        for (int i = 0; i < M; ++i)
            for (int j = 0; j < M; ++j) {
                if (!Z[i * M + j]) continue;
                for (int ip = i + 1; ip < M; ++ip) {
                    if (Z[ip * M + j]) continue;
                    for (int jp = 0; jp < M; ++jp) {
                        if (!Z[ip * M + jp] || Z[i * M + jp]) continue;
                        volatile float t1 = A[i * M + jp] - A[ip * M + jp];
                        volatile float t2 = A[ip * M + j] - A[i * M + j];
                        float g = t1 + t2;
                        if (!found || g > best) {
                            found = 1;
                            best = g;
                            bi = i; bj = j; bip = ip; bjp = jp;
                        }
                    }
                }
            }
        if (!found || !(best > 0.0f)) break;
        if (gains) gains[swaps] = best;
        Z[bi * M + bj] = 0;
        Z[bi * M + bjp] = 1;
        Z[bip * M + bjp] = 0;
        Z[bip * M + bj] = 1;
        ++swaps;
    }
    return swaps;
}

static double block_objective(const float* A, const uint8_t* Z, int M) {
    double total = 0.0;
    for (int i = 0; i < M; ++i) {
        double row = 0.0;
        for (int j = 0; j < M; ++j)
            if (Z[i * M + j]) row += (double)A[i * M + j];
        total += row;
    }
    return total;
}

static int block_feasible(const uint8_t* Z, int N, int M) {
    for (int i = 0; i < M; ++i) {
        int r = 0, c = 0;
        for (int j = 0; j < M; ++j) {
            r += Z[i * M + j] != 0;
            c += Z[j * M + i] != 0;
        }
        if (r != N || c != N) return 0;
    }
    return 1;
}

/* R1-R3, then R4 and R5.  info[0..2] as in round_block, info[3] = R4 swaps,
 * info[4] = 1 when the previous mask was taken.  prev may be NULL.          */
static int round_block_ex(const float* S, const float* A, int N, int M, int L, int K,
                          const uint8_t* prev, uint8_t* Z, int* order, int* info,
                          float* gains) {
    int st = round_block(S, A, N, M, L, Z, order, info, NULL, NULL, NULL);
    info[3] = info[4] = 0;
    if (st != OR_OK) return st;
    info[3] = polish_block(A, M, K, Z, gains);
    if (!block_feasible(Z, N, M)) return OR_ERR_INVARIANT;
    if (prev && block_feasible(prev, N, M) &&
        block_objective(A, prev, M) > block_objective(A, Z, M)) {
        memcpy(Z, prev, (size_t)(M * M));
        info[4] = 1;
    }
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Exact optimum of one block ("Core claim": the LP over 0 <= S <= 1 with row
 * and column sums N is integral -- bipartite b-matching / capacitated OT).
 * Min-cost flow by successive shortest paths with Dijkstra on reduced costs:
 * source -> row i (cap N, cost 0), row i -> col j (cap 1, cost -A_ij),
 * col j -> sink (cap N, cost 0); push N*M units one at a time.  Returns the
 * optimum sum of A over the chosen mask (fp64) and the mask in Z.           */
double oracle_exact_opt_block(const float* A, int N, int M, uint8_t* Z) {
    const int V = 2 * M + 2, S = 2 * M, T = 2 * M + 1;
    /* dense residual graph: cap[u][v], cost[u][v] */
    int cap[66][66];
    double cost[66][66], pot[66], dist[66];
    int prev[66], done[66];
    memset(cap, 0, sizeof cap);
    for (int u = 0; u < V; ++u)
        for (int v = 0; v < V; ++v) cost[u][v] = 0.0;
    for (int i = 0; i < M; ++i) {
        cap[S][i] = N;
        cap[M + i][T] = N;
        for (int j = 0; j < M; ++j) {
            cap[i][M + j] = 1;
            cost[i][M + j] = -(double)A[i * M + j];
            cost[M + j][i] = (double)A[i * M + j];
        }
    }
    /* initial potentials: shortest distances in the (acyclic) start graph */
    for (int u = 0; u < V; ++u) pot[u] = 0.0;
    for (int j = 0; j < M; ++j) {
        double mn = 0.0;
        for (int i = 0; i < M; ++i)
            if (cost[i][M + j] < mn) mn = cost[i][M + j];
        pot[M + j] = mn;
    }
    {
        double mn = 0.0;
        for (int j = 0; j < M; ++j)
            if (pot[M + j] < mn) mn = pot[M + j];
        pot[T] = mn;
    }
    for (int unit = 0; unit < N * M; ++unit) {
        for (int u = 0; u < V; ++u) {
            dist[u] = INFINITY;
            done[u] = 0;
            prev[u] = -1;
        }
        dist[S] = 0.0;
        for (;;) {
            int u = -1;
            for (int w = 0; w < V; ++w)
                if (!done[w] && dist[w] < INFINITY && (u < 0 || dist[w] < dist[u])) u = w;
            if (u < 0) break;
            done[u] = 1;
            for (int v = 0; v < V; ++v) {
                if (cap[u][v] <= 0 || done[v]) continue;
                double rc = cost[u][v] + pot[u] - pot[v];
                if (rc < 0.0) rc = 0.0; /* rounding noise only */
                if (dist[u] + rc < dist[v]) {
                    dist[v] = dist[u] + rc;
                    prev[v] = u;
                }
            }
        }
        if (dist[T] == INFINITY) return NAN;
        for (int u = 0; u < V; ++u)
            if (dist[u] < INFINITY) pot[u] += dist[u];
        for (int v = T; v != S; v = prev[v]) {
            int u = prev[v];
            cap[u][v] -= 1;
            cap[v][u] += 1;
        }
    }
    double obj = 0.0;
    for (int i = 0; i < M; ++i)
        for (int j = 0; j < M; ++j) {
            int used = (cap[i][M + j] == 0);
            if (Z) Z[i * M + j] = (uint8_t)used;
            if (used) obj += (double)A[i * M + j];
        }
    return obj;
}

/* ------------------------------------------------------------------------ */
/* Exported entry points.                                                    */

static int check_shape(int64_t rows, int64_t cols, int64_t ld, int N, int M) {
    if (M < 1 || M > 32 || N < 1 || N > M) return OR_ERR_ARG;
    if (rows <= 0 || cols <= 0 || rows % M || cols % M || ld < cols) return OR_ERR_ARG;
    return OR_OK;
}

/* Dykstra on the listed blocks (block id = bi * (cols/M) + bj).  Outputs, per
 * listed block, M*M values row-major: S64 (fp64, may be NULL) and S32 (fp32 by
 * round-to-nearest, may be NULL).  Parallel over blocks with OpenMP.         */
int oracle_dykstra_blocks(const float* W, int64_t rows, int64_t cols, int64_t ld,
                          int N, int M, double tau, int iters,
                          const int64_t* block_ids, int64_t nblocks,
                          double* S64, float* S32, int nthreads) {
    if (check_shape(rows, cols, ld, N, M) || iters < 1 || !(tau >= 0.0) || !isfinite(tau))
        return OR_ERR_ARG;
    const int64_t nbc = cols / M, nb_total = (rows / M) * nbc;
    for (int64_t b = 0; b < nblocks; ++b)
        if (block_ids[b] < 0 || block_ids[b] >= nb_total) return OR_ERR_ARG;
    int status = OR_OK;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
#pragma omp parallel
    {
        float A[1024];
        double X[1024], Q[1024];
#pragma omp for schedule(dynamic, 16)
        for (int64_t b = 0; b < nblocks; ++b) {
            int64_t id = block_ids[b];
            gather_abs(W, ld, id / nbc, id % nbc, M, A);
            int st = dykstra_block(A, N, M, tau, iters, X, Q);
            if (st != OR_OK) {
#pragma omp atomic write
                status = st;
                continue;
            }
            for (int k = 0; k < M * M; ++k) {
                if (S64) S64[b * M * M + k] = X[k];
                if (S32) S32[b * M * M + k] = (float)X[k];
            }
        }
    }
    return status;
}

/* Dykstra on every block; S64 / S32 are full matrices [rows x cols]
 * row-major with leading dimension cols (either may be NULL).               */
int oracle_dykstra(const float* W, int64_t rows, int64_t cols, int64_t ld, int N, int M,
                   double tau, int iters, double* S64, float* S32, int nthreads) {
    if (check_shape(rows, cols, ld, N, M) || iters < 1 || !(tau >= 0.0) || !isfinite(tau))
        return OR_ERR_ARG;
    const int64_t nbc = cols / M, nb = (rows / M) * nbc;
    int status = OR_OK;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
#pragma omp parallel
    {
        float A[1024];
        double X[1024], Q[1024];
#pragma omp for schedule(dynamic, 16)
        for (int64_t id = 0; id < nb; ++id) {
            int64_t bi = id / nbc, bj = id % nbc;
            gather_abs(W, ld, bi, bj, M, A);
            int st = dykstra_block(A, N, M, tau, iters, X, Q);
            if (st != OR_OK) {
#pragma omp atomic write
                status = st;
                continue;
            }
            for (int i = 0; i < M; ++i)
                for (int j = 0; j < M; ++j) {
                    int64_t o = (bi * M + i) * cols + bj * M + j;
                    if (S64) S64[o] = X[i * M + j];
                    if (S32) S32[o] = (float)X[i * M + j];
                }
        }
    }
    return status;
}

/* One block of rounding on dense M*M arrays (S32 and A row-major); Z gets the
 * 0/1 mask; info and the optional move traces (NULL = not wanted) as in
 * round_block.                                                               */
int oracle_round_block(const float* S32, const float* A, int N, int M, int ls_steps,
                       uint8_t* Z, int* info, uint8_t* Zgreedy, float* move_scores,
                       int* move_ijs) {
    if (M < 1 || M > 32 || N < 1 || N > M || ls_steps < 0) return OR_ERR_ARG;
    int order[1024];
    return round_block(S32, A, N, M, ls_steps, Z, order, info, Zgreedy, move_scores, move_ijs);
}

/* fp32 mode of the Dykstra steps on the listed blocks (block id as in
 * oracle_dykstra_blocks); S gets M*M fp32 values per listed block.           */
int oracle_dykstra_blocks_f32(const float* W, int64_t rows, int64_t cols, int64_t ld,
                              int N, int M, float tau, int iters,
                              const int64_t* block_ids, int64_t nblocks, float* S,
                              int nthreads) {
    if (check_shape(rows, cols, ld, N, M) || iters < 1 || !(tau >= 0.0f) || !isfinite(tau))
        return OR_ERR_ARG;
    const int64_t nbc = cols / M, nb_total = (rows / M) * nbc;
    for (int64_t b = 0; b < nblocks; ++b)
        if (block_ids[b] < 0 || block_ids[b] >= nb_total) return OR_ERR_ARG;
    int status = OR_OK;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
#pragma omp parallel
    {
        float A[1024], X[1024], Q[1024];
#pragma omp for schedule(dynamic, 16)
        for (int64_t b = 0; b < nblocks; ++b) {
            int64_t id = block_ids[b];
            gather_abs(W, ld, id / nbc, id % nbc, M, A);
            int st = dykstra_block_f32(A, N, M, tau, iters, X, Q);
            if (st != OR_OK) {
#pragma omp atomic write
                status = st;
                continue;
            }
            for (int k = 0; k < M * M; ++k) S[b * M * M + k] = X[k];
        }
    }
    return status;
}

/* Rounding of every block of a matrix.  S32 [rows x cols] with leading
 * dimension lds; W [rows x cols] with leading dimension ld (A = |W|).  The
 * mask is packed row-major into uint32 words, ceil(cols/32) words per row,
 * bit (c % 32) of word c / 32 is column c (the page fixes no layout).  stats (may be NULL)
 * accumulates [blocks with D > 0, total D, R2 moves, R3 moves].             */
int oracle_round(const float* S32, int64_t lds, const float* W, int64_t ld,
                 int64_t rows, int64_t cols, int N, int M, int ls_steps,
                 uint32_t* mask, int64_t* stats, int nthreads) {
    if (check_shape(rows, cols, ld, N, M) || lds < cols || ls_steps < 0) return OR_ERR_ARG;
    const int64_t nbc = cols / M, nb = (rows / M) * nbc, wpr = (cols + 31) / 32;
    memset(mask, 0, (size_t)(rows * wpr) * sizeof(uint32_t));
    int status = OR_OK;
    int64_t s0 = 0, s1 = 0, s2 = 0, s3 = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
#pragma omp parallel reduction(+ : s0, s1, s2, s3)
    {
        float A[1024], S[1024];
        uint8_t Z[1024];
        int order[1024], info[3];
#pragma omp for schedule(dynamic, 16)
        for (int64_t id = 0; id < nb; ++id) {
            int64_t bi = id / nbc, bj = id % nbc;
            gather_abs(W, ld, bi, bj, M, A);
            for (int i = 0; i < M; ++i)
                for (int j = 0; j < M; ++j) S[i * M + j] = S32[(bi * M + i) * lds + bj * M + j];
            int st = round_block(S, A, N, M, ls_steps, Z, order, info, NULL, NULL, NULL);
            if (st != OR_OK) {
#pragma omp atomic write
                status = st;
                continue;
            }
            s0 += info[0] > 0;
            s1 += info[0];
            s2 += info[1];
            s3 += info[2];
            for (int i = 0; i < M; ++i)
                for (int j = 0; j < M; ++j)
                    if (Z[i * M + j]) {
                        int64_t r = bi * M + i, c = bj * M + j;
                        /* blocks of one row never share a word bit; words of
                           M < 32 blocks are shared, so combine atomically */
#pragma omp atomic update
                        mask[r * wpr + c / 32] |= (uint32_t)1u << (c % 32);
                    }
        }
    }
    if (stats) {
        stats[0] += s0;
        stats[1] += s1;
        stats[2] += s2;
        stats[3] += s3;
    }
    return status;
}

/* oracle_round_block with the optional stages: polish_steps = K of R4 and
 * prev (dense M*M 0/1, or NULL) for R5.  info[5] as in round_block_ex;
 * gains (may be NULL) receives the applied R4 gains.                        */
int oracle_round_block_ex(const float* S32, const float* A, int N, int M, int ls_steps,
                          int polish_steps, const uint8_t* prev, uint8_t* Z, int* info,
                          float* gains) {
    if (M < 1 || M > 32 || N < 1 || N > M || ls_steps < 0 || polish_steps < 0) return OR_ERR_ARG;
    int order[1024];
    return round_block_ex(S32, A, N, M, ls_steps, polish_steps, prev, Z, order, info, gains);
}

/* oracle_round with the optional stages; prev_mask (packed like mask, or
 * NULL) is the caller's previous mask.  stats (may be NULL) accumulates
 * [blocks with D > 0, total D, R2 moves, R3 moves, R4 swaps, blocks that kept
 * the previous mask].                                                       */
int oracle_round_ex(const float* S32, int64_t lds, const float* W, int64_t ld,
                    int64_t rows, int64_t cols, int N, int M, int ls_steps, int polish_steps,
                    const uint32_t* prev_mask, uint32_t* mask, int64_t* stats, int nthreads) {
    if (check_shape(rows, cols, ld, N, M) || lds < cols || ls_steps < 0 || polish_steps < 0)
        return OR_ERR_ARG;
    const int64_t nbc = cols / M, nb = (rows / M) * nbc, wpr = (cols + 31) / 32;
    uint32_t* out = mask;
    if (prev_mask == mask) { /* in place: keep the previous words readable */
        out = (uint32_t*)malloc((size_t)(rows * wpr) * sizeof(uint32_t));
        if (!out) return OR_ERR_ARG;
    }
    memset(out, 0, (size_t)(rows * wpr) * sizeof(uint32_t));
    int status = OR_OK;
    int64_t s0 = 0, s1 = 0, s2 = 0, s3 = 0, s4 = 0, s5 = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
#pragma omp parallel reduction(+ : s0, s1, s2, s3, s4, s5)
    {
        float A[1024], S[1024];
        uint8_t Z[1024], P[1024];
        int order[1024], info[5];
#pragma omp for schedule(dynamic, 16)
        for (int64_t id = 0; id < nb; ++id) {
            int64_t bi = id / nbc, bj = id % nbc;
            gather_abs(W, ld, bi, bj, M, A);
            for (int i = 0; i < M; ++i)
                for (int j = 0; j < M; ++j) {
                    S[i * M + j] = S32[(bi * M + i) * lds + bj * M + j];
                    if (prev_mask) {
                        int64_t r = bi * M + i, c = bj * M + j;
                        P[i * M + j] = (uint8_t)((prev_mask[r * wpr + c / 32] >> (c % 32)) & 1u);
                    }
                }
            int st = round_block_ex(S, A, N, M, ls_steps, polish_steps, prev_mask ? P : NULL, Z,
                                    order, info, NULL);
            if (st != OR_OK) {
#pragma omp atomic write
                status = st;
                continue;
            }
            s0 += info[0] > 0;
            s1 += info[0];
            s2 += info[1];
            s3 += info[2];
            s4 += info[3];
            s5 += info[4];
            for (int i = 0; i < M; ++i)
                for (int j = 0; j < M; ++j)
                    if (Z[i * M + j]) {
                        int64_t r = bi * M + i, c = bj * M + j;
#pragma omp atomic update
                        out[r * wpr + c / 32] |= (uint32_t)1u << (c % 32);
                    }
        }
    }
    if (out != mask) {
        memcpy(mask, out, (size_t)(rows * wpr) * sizeof(uint32_t));
        free(out);
    }
    if (stats) {
        stats[0] += s0;
        stats[1] += s1;
        stats[2] += s2;
        stats[3] += s3;
        stats[4] += s4;
        stats[5] += s5;
    }
    return status;
}

/* Exact optimum objective per listed block (fp64).                          */
int oracle_exact_opt_blocks(const float* W, int64_t rows, int64_t cols, int64_t ld, int N,
                            int M, const int64_t* block_ids, int64_t nblocks, double* opt,
                            int nthreads) {
    if (check_shape(rows, cols, ld, N, M)) return OR_ERR_ARG;
    const int64_t nbc = cols / M, nb_total = (rows / M) * nbc;
    for (int64_t b = 0; b < nblocks; ++b)
        if (block_ids[b] < 0 || block_ids[b] >= nb_total) return OR_ERR_ARG;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
#pragma omp parallel
    {
        float A[1024];
#pragma omp for schedule(dynamic, 4)
        for (int64_t b = 0; b < nblocks; ++b) {
            int64_t id = block_ids[b];
            gather_abs(W, ld, id / nbc, id % nbc, M, A);
            opt[b] = oracle_exact_opt_block(A, N, M, NULL);
        }
    }
    return OR_OK;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
