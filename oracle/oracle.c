/*
 * oracle.c -- plain, slow, float64 CPU oracle for causal GQA attention.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the bench's CPU
 * baseline use it. It shares no code with the HIP library.
 *
 * What it computes (the plain definition, not the tiled algorithm):
 *   The NanoEuler blog page ("Tiled FlashAttention") presents tiling as a way
 *   to cut global-memory round trips; the tiled kernel therefore reaches the
 *   ordinary softmax-attention result. This file writes that result out
 *   directly, one query row at a time, in float64:
 *
 *     s_ij   = scale * <q_i, k_j>           for visible j (j <= i if causal)
 *     LSE_i  = log sum_j exp(s_ij)          (natural log, visible j only)
 *     P_ij   = exp(s_ij - LSE_i)
 *     O_i    = sum_j P_ij v_j
 *
 *   and the exact gradient of O for an upstream gradient dO (the softmax
 *   Jacobian-vector product written out; the pages say the backward is
 *   hand-derived and gradient-checked, the formula is the textbook one):
 *
 *     dV_j  += sum_i P_ij dO_i
 *     dP_ij  = <dO_i, v_j>
 *     D_i    = sum_j P_ij dP_ij
 *     dS_ij  = P_ij (dP_ij - D_i)
 *     dQ_i   = scale * sum_j dS_ij k_j
 *     dK_j  += scale * sum_i dS_ij q_i
 *
 *   Grouped-query attention: query head hq reads KV head hq / (Hq / Hkv)
 *   (consecutive query heads share a KV head). dK and dV of a KV head sum the
 *   contributions of every query head in its group.
 *
 * Layout: contiguous row-major [B, H, N, d] for q, k, v, o, dO and the
 * gradients; [B, Hq, N] for lse. All arrays are float64.
 *
 * Parallelism: OpenMP over (b, kv-head) units only; inside a unit the query
 * heads and rows run serially, so results are bitwise independent of the
 * thread count.
 *
 * The max subtraction below only keeps exp() from overflowing in float64; the
 * result equals the naive exp(s)/sum(exp(s)).
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static int visible(int causal, int i, int j) { return causal ? (j <= i) : 1; }

/* Scores of one query row against every visible key, then LSE.
 * s[j] is written for visible j; returns LSE_i. */
static double row_scores(const double* qi, const double* kh, int N, int d, int causal,
                         int i, double scale, double* s) {
    double m = -INFINITY;
    for (int j = 0; j < N; ++j) {
        if (!visible(causal, i, j)) continue;
        double dot = 0.0;
        for (int c = 0; c < d; ++c) dot += qi[c] * kh[(size_t)j * d + c];
        s[j] = scale * dot;
        if (s[j] > m) m = s[j];
    }
    double l = 0.0;
    for (int j = 0; j < N; ++j)
        if (visible(causal, i, j)) l += exp(s[j] - m);
    return m + log(l);
}

int oracle_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Forward: o [B,Hq,N,d], lse [B,Hq,N]. */
void oracle_attn_fwd(const double* q, const double* k, const double* v,
                     double* o, double* lse,
                     int B, int Hq, int Hkv, int N, int d, int causal, double scale) {
    const int group = Hq / Hkv;
    const int units = B * Hkv;
#pragma omp parallel for schedule(dynamic, 1)
    for (int u = 0; u < units; ++u) {
        const int b = u / Hkv, hkv = u % Hkv;
        double* s = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
        const double* kh = k + ((size_t)b * Hkv + hkv) * N * d;
        const double* vh = v + ((size_t)b * Hkv + hkv) * N * d;
        for (int g = 0; g < group; ++g) {
            const int hq = hkv * group + g;
            const size_t qoff = ((size_t)b * Hq + hq) * N;
            for (int i = 0; i < N; ++i) {
                const double* qi = q + (qoff + i) * d;
                double L = row_scores(qi, kh, N, d, causal, i, scale, s);
                lse[qoff + i] = L;
                double* oi = o + (qoff + i) * d;
                for (int c = 0; c < d; ++c) oi[c] = 0.0;
                for (int j = 0; j < N; ++j) {
                    if (!visible(causal, i, j)) continue;
                    double p = exp(s[j] - L);
                    for (int c = 0; c < d; ++c) oi[c] += p * vh[(size_t)j * d + c];
                }
            }
        }
        free(s);
    }
}

/* Backward: dq [B,Hq,N,d], dk and dv [B,Hkv,N,d], fully overwritten.
 * P is recomputed from q, k (the definition); nothing from the forward is reused. */
void oracle_attn_bwd(const double* q, const double* k, const double* v, const double* dout,
                     double* dq, double* dk, double* dv,
                     int B, int Hq, int Hkv, int N, int d, int causal, double scale) {
    const int group = Hq / Hkv;
    const int units = B * Hkv;
#pragma omp parallel for schedule(dynamic, 1)
    for (int u = 0; u < units; ++u) {
        const int b = u / Hkv, hkv = u % Hkv;
        double* s = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
        double* dp = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
        const size_t kvoff = ((size_t)b * Hkv + hkv) * N * d;
        const double* kh = k + kvoff;
        const double* vh = v + kvoff;
        double* dkh = dk + kvoff;
        double* dvh = dv + kvoff;
        memset(dkh, 0, sizeof(double) * (size_t)N * d);
        memset(dvh, 0, sizeof(double) * (size_t)N * d);
        for (int g = 0; g < group; ++g) {
            const int hq = hkv * group + g;
            const size_t qoff = ((size_t)b * Hq + hq) * N;
            for (int i = 0; i < N; ++i) {
                const double* qi = q + (qoff + i) * d;
                const double* doi = dout + (qoff + i) * d;
                double* dqi = dq + (qoff + i) * d;
                double L = row_scores(qi, kh, N, d, causal, i, scale, s);
                /* P_ij (kept in s), dP_ij and D_i = sum_j P_ij dP_ij */
                double D = 0.0;
                for (int j = 0; j < N; ++j) {
                    if (!visible(causal, i, j)) continue;
                    s[j] = exp(s[j] - L);
                    double acc = 0.0;
                    for (int c = 0; c < d; ++c) acc += doi[c] * vh[(size_t)j * d + c];
                    dp[j] = acc;
                    D += s[j] * dp[j];
                }
                for (int c = 0; c < d; ++c) dqi[c] = 0.0;
                for (int j = 0; j < N; ++j) {
                    if (!visible(causal, i, j)) continue;
                    const double p = s[j];
                    const double ds = p * (dp[j] - D);
                    for (int c = 0; c < d; ++c) {
                        dvh[(size_t)j * d + c] += p * doi[c];
                        dqi[c] += scale * ds * kh[(size_t)j * d + c];
                        dkh[(size_t)j * d + c] += scale * ds * qi[c];
                    }
                }
            }
        }
        free(s);
        free(dp);
    }
}
