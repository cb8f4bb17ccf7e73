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

/* Sampled outputs of one (b, kv-head) unit, for shapes where the full oracle
 * is too slow. Same definitions as above; the unit's G = Hq/Hkv query heads
 * are passed as q, dout [G, N, d] and its KV head as k, v [N, d].
 *   For each listed query row (row_g[r], row_i[r]): o_rows[r, :], lse_rows[r],
 *   dq_rows[r, :].
 *   For each listed key row keys[t]: dk_rows[t, :], dv_rows[t, :] (summed over
 *   the G query heads). These need LSE_i and D_i of every query row, which a
 *   first pass computes (OpenMP over rows; each row is independent). */
void oracle_attn_sampled(const double* q, const double* k, const double* v, const double* dout,
                         int G, int N, int d, int causal, double scale,
                         int n_rows, const int* row_g, const int* row_i,
                         double* o_rows, double* lse_rows, double* dq_rows,
                         int n_keys, const int* keys, double* dk_rows, double* dv_rows) {
    /* query rows: O, LSE, dQ */
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < n_rows; ++r) {
        const int g = row_g[r], i = row_i[r];
        double* s = (double*)malloc(sizeof(double) * (size_t)N);
        double* dp = (double*)malloc(sizeof(double) * (size_t)N);
        const double* qi = q + ((size_t)g * N + i) * d;
        const double* doi = dout + ((size_t)g * N + i) * d;
        double L = row_scores(qi, k, N, d, causal, i, scale, s);
        lse_rows[r] = L;
        double* oi = o_rows + (size_t)r * d;
        double* dqi = dq_rows + (size_t)r * d;
        for (int c = 0; c < d; ++c) { oi[c] = 0.0; dqi[c] = 0.0; }
        double D = 0.0;
        for (int j = 0; j < N; ++j) {
            if (!visible(causal, i, j)) continue;
            s[j] = exp(s[j] - L);
            double acc = 0.0;
            for (int c = 0; c < d; ++c) acc += doi[c] * v[(size_t)j * d + c];
            dp[j] = acc;
            D += s[j] * dp[j];
            for (int c = 0; c < d; ++c) oi[c] += s[j] * v[(size_t)j * d + c];
        }
        for (int j = 0; j < N; ++j) {
            if (!visible(causal, i, j)) continue;
            const double ds = s[j] * (dp[j] - D);
            for (int c = 0; c < d; ++c) dqi[c] += scale * ds * k[(size_t)j * d + c];
        }
        free(s);
        free(dp);
    }
    if (n_keys <= 0) return;
    /* row statistics LSE_i and D_i for every query row of the unit */
    double* lse_all = (double*)malloc(sizeof(double) * (size_t)G * N);
    double* d_all = (double*)malloc(sizeof(double) * (size_t)G * N);
#pragma omp parallel for schedule(dynamic, 16)
    for (long gi = 0; gi < (long)G * N; ++gi) {
        const int g = (int)(gi / N), i = (int)(gi % N);
        double* s = (double*)malloc(sizeof(double) * (size_t)N);
        const double* qi = q + ((size_t)g * N + i) * d;
        const double* doi = dout + ((size_t)g * N + i) * d;
        double L = row_scores(qi, k, N, d, causal, i, scale, s);
        double D = 0.0;
        for (int j = 0; j < N; ++j) {
            if (!visible(causal, i, j)) continue;
            double acc = 0.0;
            for (int c = 0; c < d; ++c) acc += doi[c] * v[(size_t)j * d + c];
            D += exp(s[j] - L) * acc;
        }
        lse_all[gi] = L;
        d_all[gi] = D;
        free(s);
    }
    /* key rows: dK_j, dV_j over every query head of the group and every row */
#pragma omp parallel for schedule(dynamic, 1)
    for (int t = 0; t < n_keys; ++t) {
        const int j = keys[t];
        double* dkj = dk_rows + (size_t)t * d;
        double* dvj = dv_rows + (size_t)t * d;
        for (int c = 0; c < d; ++c) { dkj[c] = 0.0; dvj[c] = 0.0; }
        for (int g = 0; g < G; ++g) {
            for (int i = 0; i < N; ++i) {
                if (!visible(causal, i, j)) continue;
                const double* qi = q + ((size_t)g * N + i) * d;
                const double* doi = dout + ((size_t)g * N + i) * d;
                double dot = 0.0, acc = 0.0;
                for (int c = 0; c < d; ++c) {
                    dot += qi[c] * k[(size_t)j * d + c];
                    acc += doi[c] * v[(size_t)j * d + c];
                }
                const double p = exp(scale * dot - lse_all[(size_t)g * N + i]);
                const double ds = p * (acc - d_all[(size_t)g * N + i]);
                for (int c = 0; c < d; ++c) {
                    dvj[c] += p * doi[c];
                    dkj[c] += scale * ds * qi[c];
                }
            }
        }
    }
    free(lse_all);
    free(d_all);
}

/*
 * Few-query attention over a cached sequence (inference; the blog page's FAQ
 * says inference works and runs on 8 GB cards): Nq query rows that are the
 * last Nq positions of a sequence of Nk >= Nq tokens, whose keys and values
 * are all present in k and v. Query row i sits at sequence position
 * p_i = Nk - Nq + i; causally it sees keys j <= p_i, otherwise every key.
 * The definitions are those of the forward above:
 *
 *     s_ij  = scale * <q_i, k_j>            for visible j
 *     LSE_i = log sum_j exp(s_ij)
 *     O_i   = sum_j exp(s_ij - LSE_i) v_j
 *
 * With Nq = Nk this is exactly oracle_attn_fwd.
 * Layout: q, o [B, Hq, Nq, d]; k, v [B, Hkv, Nk, d]; lse [B, Hq, Nq].
 */
void oracle_attn_decode(const double* q, const double* k, const double* v,
                        double* o, double* lse,
                        int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, double scale) {
    const int group = Hq / Hkv;
    const int units = B * Hkv;
#pragma omp parallel for schedule(dynamic, 1)
    for (int u = 0; u < units; ++u) {
        const int b = u / Hkv, hkv = u % Hkv;
        double* s = (double*)malloc(sizeof(double) * (size_t)(Nk > 0 ? Nk : 1));
        const double* kh = k + ((size_t)b * Hkv + hkv) * Nk * d;
        const double* vh = v + ((size_t)b * Hkv + hkv) * Nk * d;
        for (int g = 0; g < group; ++g) {
            const int hq = hkv * group + g;
            const size_t qoff = ((size_t)b * Hq + hq) * Nq;
            for (int i = 0; i < Nq; ++i) {
                const int pos = Nk - Nq + i;   /* sequence position of this query */
                const double* qi = q + (qoff + i) * d;
                double L = row_scores(qi, kh, Nk, d, causal, pos, scale, s);
                lse[qoff + i] = L;
                double* oi = o + (qoff + i) * d;
                for (int c = 0; c < d; ++c) oi[c] = 0.0;
                for (int j = 0; j < Nk; ++j) {
                    if (!visible(causal, pos, j)) continue;
                    double p = exp(s[j] - L);
                    for (int c = 0; c < d; ++c) oi[c] += p * vh[(size_t)j * d + c];
                }
            }
        }
        free(s);
    }
}

/*
 * Rotary position embedding (RoPE; the blog page's FAQ lists RoPE among the
 * techniques the trainer supports) applied to q and k before the attention.
 * The pages name RoPE only; the form used is the rotate-half pairing: for a
 * row at sequence position n and i < d/2, the pair (x_i, x_{i+d/2}) becomes
 *
 *     (x_i cos - x_{i+d/2} sin,  x_{i+d/2} cos + x_i sin),   cos, sin = table[n][i]
 *
 * with the caller's tables (normally cos/sin of n * base^(-2i/d)). The
 * attention then runs on the rotated q and k. The rotation is orthogonal per
 * pair, so the gradients of the unrotated q and k are the rotated-space
 * gradients turned back by the transpose:
 *
 *     (g_i cos + g_{i+d/2} sin,  g_{i+d/2} cos - g_i sin).
 *
 * Tables: cs, sn [N][d/2]; tensors as in the forward ([B, H, N, d]).
 */
static void rope_apply(double* x, const double* cs, const double* sn, size_t heads, int N, int d, int transpose) {
    const int h = d / 2;
    for (size_t r = 0; r < heads * (size_t)N; ++r) {
        const int n = (int)(r % (size_t)N);
        double* row = x + r * d;
        for (int i = 0; i < h; ++i) {
            const double c = cs[(size_t)n * h + i], s = sn[(size_t)n * h + i];
            const double a = row[i], b = row[i + h];
            if (!transpose) {
                row[i] = a * c - b * s;
                row[i + h] = b * c + a * s;
            } else {
                row[i] = a * c + b * s;
                row[i + h] = b * c - a * s;
            }
        }
    }
}

static double* dup(const double* x, size_t n) {
    double* y = (double*)malloc(sizeof(double) * (n ? n : 1));
    memcpy(y, x, sizeof(double) * n);
    return y;
}

void oracle_attn_fwd_rope(const double* q, const double* k, const double* v, const double* cs, const double* sn,
                          double* o, double* lse, int B, int Hq, int Hkv, int N, int d, int causal, double scale) {
    double* qr = dup(q, (size_t)B * Hq * N * d);
    double* kr = dup(k, (size_t)B * Hkv * N * d);
    rope_apply(qr, cs, sn, (size_t)B * Hq, N, d, 0);
    rope_apply(kr, cs, sn, (size_t)B * Hkv, N, d, 0);
    oracle_attn_fwd(qr, kr, v, o, lse, B, Hq, Hkv, N, d, causal, scale);
    free(qr);
    free(kr);
}

void oracle_attn_bwd_rope(const double* q, const double* k, const double* v, const double* dout,
                          const double* cs, const double* sn, double* dq, double* dk, double* dv,
                          int B, int Hq, int Hkv, int N, int d, int causal, double scale) {
    double* qr = dup(q, (size_t)B * Hq * N * d);
    double* kr = dup(k, (size_t)B * Hkv * N * d);
    rope_apply(qr, cs, sn, (size_t)B * Hq, N, d, 0);
    rope_apply(kr, cs, sn, (size_t)B * Hkv, N, d, 0);
    oracle_attn_bwd(qr, kr, v, dout, dq, dk, dv, B, Hq, Hkv, N, d, causal, scale);
    rope_apply(dq, cs, sn, (size_t)B * Hq, N, d, 1);
    rope_apply(dk, cs, sn, (size_t)B * Hkv, N, d, 1);
    free(qr);
    free(kr);
}
