// attn_fwd_mfma.hip -- causal GQA attention forward on gfx950 matrix cores.
//
// The loop is the one of the NanoEuler "Tiled FlashAttention" section (one
// workgroup per query tile; for each K/V tile: stage it on chip, Q*K^T, online
// softmax, accumulate the output), re-shaped for CDNA4:
//
//  * A workgroup is 4 waves x 32 query rows (BR = 128). Each wave keeps its Q
//    rows in registers as the B operand of S^T = K * Q^T, so the score
//    accumulator holds one query per lane (lane = 32h + r -> query r): the row
//    max and row sum are in-lane reductions plus one half-wave exchange.
//  * K/V tiles (BC = 64 keys) are double-buffered in LDS and prefetched one
//    tile ahead into registers: the global loads for tile j+2 are issued while
//    tile j is computed and land in LDS after it, so their latency is hidden
//    behind a whole tile of math. Loads are branch-free (rows past the end are
//    clamped to the last row and masked out of the softmax).
//  * K stays bf16 (A operand of S^T, read at row perm32(m) so accumulator e
//    holds key 16(e/8) + 8h + e%8). V is converted to fp16 when it is written
//    to LDS and stays row-major; the transposing LDS load (ds_read_b64_tr_b16)
//    reads it as the A operand of O^T += V^T * P^T, whose B operand is the
//    probability tile taken straight from the score accumulator.
//  * P is rounded to fp16 (11-bit significand) rather than bf16: bf16 rounding
//    of P shifts O, hence the backward's D = rowsum(dO o O), enough to break
//    the bf16 accuracy bound on the peaked-softmax workloads. The row sum adds
//    the rounded fp16 values (v_dot2), so O is normalised by exactly the
//    weights it accumulated.
//  * Lazy rescaling: the running max m only moves when a tile's max exceeds it
//    by more than 8 (log2 units); otherwise probabilities are taken against the
//    stale max and stay <= 2^8, which fp16 and the fp32 accumulators hold
//    exactly as well. Most tiles therefore skip the O rescale entirely.
//  * Causal tile skipping: a query tile visits only the K/V tiles that start at
//    or below its last row; a wave whose rows all precede a tile skips its
//    math; the mask is applied only on tiles crossing the diagonal or the end.
//  * Grid order: longest (last) query tiles first; when the number of
//    (batch, KV head) units is a multiple of 8, the workgroups of one unit are
//    placed on one XCD (workgroups are dealt to the 8 XCDs round-robin), so
//    its K/V tiles stay in that XCD's L2.
#include "tca_internal.h"

namespace tca {

namespace fwd {
constexpr int NW = 4;            // waves per workgroup
constexpr int BR = 32 * NW;      // query rows per workgroup
constexpr int BC = 64;           // keys per K/V tile
constexpr int PAD = 8;           // 16-bit elements of row padding (16 bytes)
constexpr float kTau = 8.f;      // lazy-rescale threshold, log2 units
}  // namespace fwd

// Global -> registers: the K and V rows k0 .. k0 + BC - 1 (clamped to N - 1);
// thread tid owns the 16-byte chunks tid + 256u, so a wave reads whole rows.
template <int D, int KCH>
__device__ __forceinline__ void load_kv_tile(u32x4 (&kreg)[KCH], u32x4 (&vreg)[KCH], const bf16_t* kh,
                                             const bf16_t* vh, int k0, int N, int tid) {
    constexpr int CPR = D / 8;
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
        const int cid = tid + 256 * u;
        const int key = min(k0 + cid / CPR, N - 1);
        const size_t off = (size_t)key * D + (cid % CPR) * 8;
        kreg[u] = *reinterpret_cast<const u32x4*>(kh + off);
        vreg[u] = *reinterpret_cast<const u32x4*>(vh + off);
    }
}

// Registers -> LDS: K as bf16 rows, V converted to fp16 rows.
template <int D, int KCH>
__device__ __forceinline__ void store_kv_tile(const u32x4 (&kreg)[KCH], const u32x4 (&vreg)[KCH],
                                              bf16_t (*Ks)[D + fwd::PAD], _Float16 (*Vs)[D + fwd::PAD],
                                              int tid) {
    constexpr int CPR = D / 8;
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
        const int cid = tid + 256 * u;
        const int row = cid / CPR, col = (cid % CPR) * 8;
        *reinterpret_cast<u32x4*>(&Ks[row][col]) = kreg[u];
        *reinterpret_cast<u32x4*>(&Vs[row][col]) = bf16x8_to_f16x8(vreg[u]);
    }
}

template <int D>
__global__ void __launch_bounds__(256, (D == 64) ? 4 : 2)
fwd_mfma_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                const bf16_t* __restrict__ v, float* __restrict__ o, float* __restrict__ lse,
                int Hq, int Hkv, int N, int causal, float scale, int nqt, int units) {
    using namespace fwd;
    constexpr int DC = D / 16;          // 16-deep chunks of the head dimension
    constexpr int DB = D / 32;          // 32-wide blocks of the head dimension
    constexpr int NB = BC / 32;         // 32-key blocks per tile
    constexpr int LD = D + PAD;         // LDS row stride (elements)
    constexpr int CPR = D / 8;          // 16-byte chunks per row
    constexpr int KCH = BC * CPR / 256; // chunks per thread per tensor per tile
    __shared__ __attribute__((aligned(16))) bf16_t Ks[2][BC][LD];
    __shared__ __attribute__((aligned(16))) _Float16 Vs[2][BC][LD];

    const int group = Hq / Hkv;
    const TileMap tm = map_workgroup(blockIdx.x, nqt, units, Hkv, group);
    const int hq = tm.hkv * group + tm.g;
    const size_t bh = (size_t)tm.b * Hq + hq;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, h = lane >> 5, r = lane & 31;
    const int q0w = tm.qt * BR + 32 * w;   // first query row of this wave
    const int qi = q0w + r;                // this lane's query row
    const bf16_t* qh = q + bh * N * D;
    const bf16_t* kh = k + ((size_t)tm.b * Hkv + tm.hkv) * N * D;
    const bf16_t* vh = v + ((size_t)tm.b * Hkv + tm.hkv) * N * D;
    const float sl2 = scale * kLog2e;      // scores in log2 units

    // Q rows of this wave as B operands: lane holds Q[qi][16c + 8h .. +7]
    bf16x8 qb[DC];
    {
        const bf16_t* qrow = qh + (size_t)min(qi, N - 1) * D + 8 * h;
#pragma unroll
        for (int c = 0; c < DC; ++c) {
            const bf16x8 val = *reinterpret_cast<const bf16x8*>(qrow + 16 * c);
            qb[c] = (qi < N) ? val : bf16x8{};
        }
    }

    // K/V tile prefetch registers: thread owns chunks tid + 256u (coalesced rows)
    u32x4 kreg[KCH], vreg[KCH];
    f32x16 oacc[DB];
#pragma unroll
    for (int x = 0; x < DB; ++x) oacc[x] = f32x16{};
    float m_s = -INFINITY;   // running (possibly stale) max, log2 units
    float l_run = 0.f;       // sum of this lane's fp16 probabilities (other half added at the end)

    const int last_q = min(N, (tm.qt + 1) * BR) - 1;
    const int kend = causal ? last_q + 1 : N;   // keys needed by this workgroup
    const int ntile = (kend + BC - 1) / BC;
    const int krow_a = perm32(r);

    load_kv_tile<D, KCH>(kreg, vreg, kh, vh, 0, N, tid);
    store_kv_tile<D, KCH>(kreg, vreg, Ks[0], Vs[0], tid);
    if (ntile > 1) load_kv_tile<D, KCH>(kreg, vreg, kh, vh, BC, N, tid);
    __syncthreads();

    for (int j = 0; j < ntile; ++j) {
        const int buf = j & 1, k0 = j * BC;
        const bool active = !causal || k0 <= q0w + 31;
        if (active) {
            // ---- S^T = K * Q^T  (rows: keys, permuted; columns: this wave's queries)
            f32x16 s[NB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) s[nb] = f32x16{};
#pragma unroll
            for (int c = 0; c < DC; ++c)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8*>(&Ks[buf][32 * nb + krow_a][16 * c + 8 * h]);
                    s[nb] = mfma_bf16(a, qb[c], s[nb]);
                }
            // ---- mask: only tiles crossing the diagonal or the end of the sequence
            if ((k0 + BC > N) || (causal && k0 + BC - 1 > q0w)) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int key = k0 + 32 * nb + 16 * (e >> 3) + 8 * h + (e & 7);
                        if (key >= N || (causal && key > qi)) s[nb][e] = -INFINITY;
                    }
            }
            // ---- online softmax with lazy rescaling (log2 domain)
            float mx = s[0][0];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[nb][e]);
            const float mt = max_halves(mx) * sl2;
            if (__any(mt > m_s + kTau)) {
                const float m_new = fmaxf(m_s, mt);
                const float alpha = fast_exp2(m_s - m_new);
                l_run *= alpha;
#pragma unroll
                for (int x = 0; x < DB; ++x)
#pragma unroll
                    for (int e = 0; e < 16; ++e) oacc[x][e] *= alpha;
                m_s = m_new;
            }
            const float mb = (m_s == -INFINITY) ? 0.f : m_s;
            // ---- P (fp16) and O^T += V^T * P^T
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int c2 = 0; c2 < 2; ++c2) {
                    float p[8];
#pragma unroll
                    for (int t = 0; t < 8; ++t) p[t] = fast_exp2(fmaf(s[nb][8 * c2 + t], sl2, -mb));
                    uint32_t pk[4];
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        pk[t] = pack_f16(p[2 * t], p[2 * t + 1]);
                        l_run = add_f16_pair(pk[t], l_run);
                    }
                    const f16x8 pb = __builtin_bit_cast(f16x8, u32x4{pk[0], pk[1], pk[2], pk[3]});
#pragma unroll
                    for (int x = 0; x < DB; ++x) {
                        const f16x8 a = lds_tr_operand(&Vs[buf][0][0], LD, 32 * nb + 16 * c2, 32 * x, h, r);
                        oacc[x] = mfma_f16(a, pb, oacc[x]);
                    }
                }
        }
        if (j + 1 < ntile) {
            store_kv_tile<D, KCH>(kreg, vreg, Ks[buf ^ 1], Vs[buf ^ 1], tid);
            if (j + 2 < ntile) load_kv_tile<D, KCH>(kreg, vreg, kh, vh, (j + 2) * BC, N, tid);
        }
        __syncthreads();
    }

    // ---- epilogue: normalise, store O (fp32) and LSE (natural log)
    // accumulator e of dim block x holds dim 32x + 8(e/4) + 4h + e%4 of query qi
    const float l_tot = sum_halves(l_run);
    if (qi < N) {
        const float inv = 1.f / l_tot;
        float* orow = o + (bh * N + qi) * D;
#pragma unroll
        for (int x = 0; x < DB; ++x)
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4) {
                const float4 val = {oacc[x][4 * a4 + 0] * inv, oacc[x][4 * a4 + 1] * inv,
                                    oacc[x][4 * a4 + 2] * inv, oacc[x][4 * a4 + 3] * inv};
                *reinterpret_cast<float4*>(orow + 32 * x + 8 * a4 + 4 * h) = val;
            }
        if (h == 0) lse[bh * N + qi] = (m_s + __log2f(l_tot)) * kLn2;
    }
}

bool mfma_path(const AttnArgs& a) { return a.dtype == ATTN_BF16 && (a.d == 64 || a.d == 128); }

hipError_t launch_fwd_mfma(const AttnArgs& a, hipStream_t st) {
    const int nqt = (a.N + fwd::BR - 1) / fwd::BR;
    const int units = a.B * a.Hkv;
    const dim3 grid((unsigned)(nqt * a.B * a.Hq));
    if (a.d == 64)
        hipLaunchKernelGGL(fwd_mfma_kernel<64>, grid, dim3(256), 0, st, (const bf16_t*)a.q,
                           (const bf16_t*)a.k, (const bf16_t*)a.v, a.o, a.lse, a.Hq, a.Hkv, a.N,
                           a.causal, a.scale, nqt, units);
    else
        hipLaunchKernelGGL(fwd_mfma_kernel<128>, grid, dim3(256), 0, st, (const bf16_t*)a.q,
                           (const bf16_t*)a.k, (const bf16_t*)a.v, a.o, a.lse, a.Hq, a.Hkv, a.N,
                           a.causal, a.scale, nqt, units);
    return hipGetLastError();
}

}  // namespace tca
