/*
 * fp64 CPU oracle for the backward pass of the DeepSeek-Sparse-Attention
 * lightning indexer.  TEST INFRASTRUCTURE ONLY: nothing in the product path
 * links or calls this file; only the tests, the smoke check and the CPU
 * baseline leg of the benchmark do.  It shares no code with the HIP kernels.
 *
 * What it computes (plain definition, no blocking, no fusion):
 *
 *   forward score  I[t,s] = sum_h w[t,h] * relu(q[t,h,:] . k[s,:]), restricted
 *   to the per-query top-k ids; an id outside [0, S_k) (canonically -1) is a
 *   padding slot (NVIDIA/cudnn-frontend PR #730, "Benchmark harness" comment:
 *   the fp64 `ref_grads` reference and the -1 / positive-out-of-range padding
 *   equivalence battery; same PR, review thread: a positive out-of-range local
 *   id is padding and must not alias the next batch).
 *
 *   score gradient (PR #730 harness docstring: kernel 1 turns index_score,
 *   attn_score and grad_loss into the per-slot gradient signal; sm_scale is
 *   folded in at run time):
 *     V       = { j : 0 <= id_j < S_k }
 *     z_j     = sm_scale * I[t,j]                 (j in V)
 *     P_j     = exp(z_j - max z) / sum_V exp(z - max z)
 *     dI_j    = grad_loss * sm_scale * (P_j - p[t,j])   (j in V), 0 otherwise
 *   This is d/dI of grad_loss * KL(p || P) when p sums to 1 over V.
 *
 *   gradient GEMMs (PR #730 harness, `ref_grads`, with the grad signal g = dI):
 *     S[h,j]    = q[t,h,:] . k[id_j,:]
 *     G[h,j]    = dI_j * w[t,h] * [S[h,j] > 0]
 *     dW[t,h]   = sum_{j in V} dI_j * max(S[h,j], 0)
 *     dQ[t,h,:] = sum_{j in V} G[h,j] * k[id_j,:]
 *     dK[s,:]  += sum_h G[h,j] * q[t,h,:]        for every (t, j in V) with id_j = s
 *
 *   dense causal variant (PR #549: a separate dense indexer-backward test;
 *   PR #730 summary: q-causal-offset behaviour preserved): the key set of query
 *   t is { s : 0 <= s <= min(t + q_offset, S_k - 1) } and I, p are indexed
 *   [t, s] directly.
 *
 * Layouts (row-major, contiguous): q [B,S_q,H,D], k [B,S_k,D], w [B,S_q,H],
 * ids/I/p [B,S_q,topk] (dense: I/p [B,S_q,S_k]), dq [B,S_q,H,D],
 * dw [B,S_q,H], dk [B,S_k,D].  Every floating-point input is fp64; the
 * caller converts bf16/fp32 values exactly.  Ids are local to each batch.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static int is_valid(int64_t id, int64_t S_k) { return id >= 0 && id < S_k; }

/* Score gradient of one query row over n candidate slots.  key_of[j] gives
 * the key of slot j, or -1 when the slot is padding. */
static void row_score_grad(int64_t n, const int64_t* key_of, const double* I,
                           const double* p, double sm_scale, double grad_loss,
                           double* dI) {
    double m = -INFINITY;
    int any = 0;
    for (int64_t j = 0; j < n; ++j) {
        dI[j] = 0.0;
        if (key_of[j] < 0) continue;
        double z = sm_scale * I[j];
        if (!any || z > m) m = z;
        any = 1;
    }
    if (!any) return;
    double Z = 0.0;
    for (int64_t j = 0; j < n; ++j)
        if (key_of[j] >= 0) Z += exp(sm_scale * I[j] - m);
    for (int64_t j = 0; j < n; ++j)
        if (key_of[j] >= 0) {
            double P = exp(sm_scale * I[j] - m) / Z;
            dI[j] = grad_loss * sm_scale * (P - p[j]);
        }
}

/* Backward of one query row.  Writes dq_t [H,D] and dw_t [H] (overwritten);
 * when dk_b is non-null adds the row's dK contribution into dk_b [S_k,D]. */
static void row_backward(int64_t n, const int64_t* key_of, const double* dI,
                         const double* q_t, const double* k_b, const double* w_t,
                         int64_t H, int64_t D, double* dq_t, double* dw_t, double* dk_b) {
    memset(dq_t, 0, sizeof(double) * (size_t)(H * D));
    memset(dw_t, 0, sizeof(double) * (size_t)H);
    for (int64_t j = 0; j < n; ++j) {
        int64_t s = key_of[j];
        if (s < 0) continue;
        const double* ks = k_b + s * D;
        for (int64_t h = 0; h < H; ++h) {
            const double* qh = q_t + h * D;
            double S = 0.0;
            for (int64_t d = 0; d < D; ++d) S += qh[d] * ks[d];
            dw_t[h] += dI[j] * (S > 0.0 ? S : 0.0);
            double G = (S > 0.0) ? dI[j] * w_t[h] : 0.0;
            if (G == 0.0) continue;
            double* dqh = dq_t + h * D;
            for (int64_t d = 0; d < D; ++d) dqh[d] += G * ks[d];
            if (dk_b) {
                double* dks = dk_b + s * D;
                for (int64_t d = 0; d < D; ++d) dks[d] += G * qh[d];
            }
        }
    }
}

/* Candidate slots of one row: sparse reads ids, dense enumerates 0..S_k-1. */
static int64_t row_keys(int dense, const int32_t* ids_t, int64_t topk, int64_t S_k,
                        int64_t t, int64_t q_offset, int64_t* key_of) {
    if (!dense) {
        for (int64_t j = 0; j < topk; ++j) key_of[j] = is_valid(ids_t[j], S_k) ? ids_t[j] : -1;
        return topk;
    }
    for (int64_t s = 0; s < S_k; ++s) key_of[s] = (s <= t + q_offset) ? s : -1;
    return S_k;
}

typedef struct {
    int dense;
    int64_t B, S_q, S_k, H, D, topk, q_offset;
    const double *q, *k, *w, *I, *p;
    const int32_t* ids;
    double sm_scale, grad_loss;
} problem;

static int64_t row_len(const problem* P) { return P->dense ? P->S_k : P->topk; }

static void one_row(const problem* P, int64_t b, int64_t t, int64_t* key_of, double* dI,
                    double* dq_t, double* dw_t, double* dk_b) {
    int64_t n = row_len(P);
    int64_t r = b * P->S_q + t;
    row_keys(P->dense, P->ids ? P->ids + r * n : NULL, P->topk, P->S_k, t, P->q_offset, key_of);
    row_score_grad(n, key_of, P->I + r * n, P->p + r * n, P->sm_scale, P->grad_loss, dI);
    row_backward(n, key_of, dI, P->q + r * P->H * P->D, P->k + b * P->S_k * P->D,
                 P->w + r * P->H, P->H, P->D, dq_t, dw_t, dk_b);
}

static int check(const problem* P) {
    if (P->B <= 0 || P->S_q <= 0 || P->S_k <= 0 || P->H <= 0 || P->D <= 0) return -1;
    if (!P->dense && P->topk <= 0) return -1;
    return 0;
}

/* Full backward: dq, dw, dk are overwritten.  Rows are independent; the dK
 * contributions are summed per thread and the per-thread sums are added in
 * thread order, so a fixed thread count gives a fixed result. */
static int full(const problem* P, double* dq, double* dw, double* dk) {
    if (check(P)) return -1;
    int64_t n = row_len(P);
    size_t dk_elems = (size_t)(P->B * P->S_k * P->D);
    memset(dk, 0, sizeof(double) * dk_elems);
    int nthreads = 1;
#ifdef _OPENMP
    nthreads = omp_get_max_threads();
#endif
    double* part = (double*)calloc((size_t)nthreads * dk_elems, sizeof(double));
    if (!part) return -2;
    int64_t rows = P->B * P->S_q;
#pragma omp parallel
    {
        int tid = 0;
#ifdef _OPENMP
        tid = omp_get_thread_num();
#endif
        int64_t* key_of = (int64_t*)malloc(sizeof(int64_t) * (size_t)n);
        double* dI = (double*)malloc(sizeof(double) * (size_t)n);
        double* mine = part + (size_t)tid * dk_elems;
#pragma omp for schedule(static)
        for (int64_t r = 0; r < rows; ++r) {
            int64_t b = r / P->S_q, t = r % P->S_q;
            one_row(P, b, t, key_of, dI, dq + r * P->H * P->D, dw + r * P->H,
                    mine + b * P->S_k * P->D);
        }
        free(key_of);
        free(dI);
    }
    for (int th = 0; th < nthreads; ++th)
        for (size_t e = 0; e < dk_elems; ++e) dk[e] += part[(size_t)th * dk_elems + e];
    free(part);
    return 0;
}

/* dQ/dW for a list of rows (flat index b*S_q + t); dq_rows [n_rows,H,D], dw_rows [n_rows,H]. */
static int rows_only(const problem* P, int64_t n_rows, const int64_t* rows, double* dq_rows,
                     double* dw_rows) {
    if (check(P)) return -1;
    for (int64_t i = 0; i < n_rows; ++i)
        if (rows[i] < 0 || rows[i] >= P->B * P->S_q) return -1;
    int64_t n = row_len(P);
#pragma omp parallel
    {
        int64_t* key_of = (int64_t*)malloc(sizeof(int64_t) * (size_t)n);
        double* dI = (double*)malloc(sizeof(double) * (size_t)n);
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < n_rows; ++i)
            one_row(P, rows[i] / P->S_q, rows[i] % P->S_q, key_of, dI,
                    dq_rows + i * P->H * P->D, dw_rows + i * P->H, NULL);
        free(key_of);
        free(dI);
    }
    return 0;
}

/* dK for a list of key rows (flat index b*S_k + s); dk_rows [n_keys,D].
 * Every query row of the key's batch is scanned for slots that select it. */
static int dk_only(const problem* P, int64_t n_keys, const int64_t* keys, double* dk_rows) {
    if (check(P)) return -1;
    for (int64_t i = 0; i < n_keys; ++i)
        if (keys[i] < 0 || keys[i] >= P->B * P->S_k) return -1;
    int64_t n = row_len(P);
    int64_t H = P->H, D = P->D;
    memset(dk_rows, 0, sizeof(double) * (size_t)(n_keys * D));
#pragma omp parallel
    {
        int64_t* key_of = (int64_t*)malloc(sizeof(int64_t) * (size_t)n);
        double* dI = (double*)malloc(sizeof(double) * (size_t)n);
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < n_keys; ++i) {
            int64_t b = keys[i] / P->S_k, s = keys[i] % P->S_k;
            const double* ks = P->k + (b * P->S_k + s) * D;
            double* out = dk_rows + i * D;
            for (int64_t t = 0; t < P->S_q; ++t) {
                int64_t r = b * P->S_q + t;
                row_keys(P->dense, P->ids ? P->ids + r * n : NULL, P->topk, P->S_k, t,
                         P->q_offset, key_of);
                int hit = 0;
                for (int64_t j = 0; j < n; ++j) hit |= (key_of[j] == s);
                if (!hit) continue;
                row_score_grad(n, key_of, P->I + r * n, P->p + r * n, P->sm_scale,
                               P->grad_loss, dI);
                const double* q_t = P->q + r * H * D;
                const double* w_t = P->w + r * H;
                for (int64_t j = 0; j < n; ++j) {
                    if (key_of[j] != s) continue;
                    for (int64_t h = 0; h < H; ++h) {
                        double S = 0.0;
                        for (int64_t d = 0; d < D; ++d) S += q_t[h * D + d] * ks[d];
                        if (!(S > 0.0)) continue;
                        double G = dI[j] * w_t[h];
                        for (int64_t d = 0; d < D; ++d) out[d] += G * q_t[h * D + d];
                    }
                }
            }
        }
        free(key_of);
        free(dI);
    }
    return 0;
}

/* ---- exported entry points ------------------------------------------------ */

#define SPARSE_PROBLEM                                                                \
    problem P = {0, B, S_q, S_k, H, D, topk, 0, q, k, w, I, p, ids, sm_scale, grad_loss}
#define DENSE_PROBLEM                                                                 \
    problem P = {1, B, S_q, S_k, H, D, S_k, q_offset, q, k, w, I, p, NULL, sm_scale, grad_loss}

int oracle_sparse(const double* q, const double* k, const double* w, const int32_t* ids,
                  const double* I, const double* p, int64_t B, int64_t S_q, int64_t S_k,
                  int64_t H, int64_t D, int64_t topk, double sm_scale, double grad_loss,
                  double* dq, double* dw, double* dk) {
    SPARSE_PROBLEM;
    return full(&P, dq, dw, dk);
}

int oracle_sparse_rows(const double* q, const double* k, const double* w, const int32_t* ids,
                       const double* I, const double* p, int64_t B, int64_t S_q, int64_t S_k,
                       int64_t H, int64_t D, int64_t topk, double sm_scale, double grad_loss,
                       int64_t n_rows, const int64_t* rows, double* dq_rows, double* dw_rows) {
    SPARSE_PROBLEM;
    return rows_only(&P, n_rows, rows, dq_rows, dw_rows);
}

int oracle_sparse_dk_rows(const double* q, const double* k, const double* w, const int32_t* ids,
                          const double* I, const double* p, int64_t B, int64_t S_q, int64_t S_k,
                          int64_t H, int64_t D, int64_t topk, double sm_scale, double grad_loss,
                          int64_t n_keys, const int64_t* keys, double* dk_rows) {
    SPARSE_PROBLEM;
    return dk_only(&P, n_keys, keys, dk_rows);
}

int oracle_dense(const double* q, const double* k, const double* w, const double* I,
                 const double* p, int64_t B, int64_t S_q, int64_t S_k, int64_t H, int64_t D,
                 int64_t q_offset, double sm_scale, double grad_loss, double* dq, double* dw,
                 double* dk) {
    DENSE_PROBLEM;
    return full(&P, dq, dw, dk);
}

int oracle_dense_rows(const double* q, const double* k, const double* w, const double* I,
                      const double* p, int64_t B, int64_t S_q, int64_t S_k, int64_t H, int64_t D,
                      int64_t q_offset, double sm_scale, double grad_loss, int64_t n_rows,
                      const int64_t* rows, double* dq_rows, double* dw_rows) {
    DENSE_PROBLEM;
    return rows_only(&P, n_rows, rows, dq_rows, dw_rows);
}

int oracle_dense_dk_rows(const double* q, const double* k, const double* w, const double* I,
                         const double* p, int64_t B, int64_t S_q, int64_t S_k, int64_t H,
                         int64_t D, int64_t q_offset, double sm_scale, double grad_loss,
                         int64_t n_keys, const int64_t* keys, double* dk_rows) {
    DENSE_PROBLEM;
    return dk_only(&P, n_keys, keys, dk_rows);
}

/* The score gradient dI of every row: sparse [B,S_q,topk], dense [B,S_q,S_k]. */
int oracle_score_grad(int dense, const int32_t* ids, const double* I, const double* p, int64_t B,
                      int64_t S_q, int64_t S_k, int64_t topk, int64_t q_offset, double sm_scale,
                      double grad_loss, double* dI) {
    int64_t n = dense ? S_k : topk;
    if (B <= 0 || S_q <= 0 || S_k <= 0 || n <= 0) return -1;
    int64_t* key_of = (int64_t*)malloc(sizeof(int64_t) * (size_t)n);
    if (!key_of) return -2;
    for (int64_t r = 0; r < B * S_q; ++r) {
        row_keys(dense, dense ? NULL : ids + r * n, topk, S_k, r % S_q, q_offset, key_of);
        row_score_grad(n, key_of, I + r * n, p + r * n, sm_scale, grad_loss, dI + r * n);
    }
    free(key_of);
    return 0;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
