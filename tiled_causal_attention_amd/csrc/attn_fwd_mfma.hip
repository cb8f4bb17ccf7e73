// attn_fwd_mfma.hip -- causal GQA attention forward on gfx950 matrix cores.
//
// The loop is the one of the NanoEuler "Tiled FlashAttention" section (one
// workgroup per query tile; for each K/V tile: stage it on chip, Q*K^T, online
// softmax, accumulate the output), re-shaped for CDNA4:
//
//  * A workgroup is 4 waves x 32 query rows (BR = 128). Each wave keeps its Q
//    rows in registers as the B operand of S^T = K * Q^T, so the score
//    accumulator holds one query per lane (lane = 32h + r -> query r) and the
//    row max / row sum of the online softmax are in-lane reductions plus one
//    exchange between the two half-waves.
//  * K tiles (BC = 64 keys) are staged in LDS as bf16 rows; the A operand reads
//    row perm32(m), which makes accumulator e hold key 16(e/8) + 8h + e%8. The
//    probabilities then feed O^T += V^T * P^T directly from registers as the B
//    operand, in natural key order, with no LDS round trip.
//  * V tiles are staged transposed (V^T, [d][key]) and converted to fp16, so
//    the A operand of O^T += V^T * P^T is one 16-byte LDS read per lane. P is
//    rounded to fp16 (11-bit significand) rather than bf16: the bf16 rounding
//    of P and of the stored O shifts the backward's D = rowsum(dO o O) enough
//    to break the bf16 accuracy bound on the peaked-softmax workloads.
//  * Causal tile skipping: a query tile visits only K/V tiles that start at or
//    below its last row; a wave whose rows all precede a tile skips its math;
//    the mask is applied only on tiles that cross the diagonal or the end of
//    the sequence.
//  * The output accumulator is O^T (lane = query), so the online-softmax
//    rescale is one multiply per register by the lane's own factor.
//  * Grid order: the longest (last) query tiles are dispatched first.
#include "tca_internal.h"

namespace tca {

namespace fwd {
constexpr int NW = 4;            // waves per workgroup
constexpr int BR = 32 * NW;      // query rows per workgroup
constexpr int BC = 64;           // keys per K/V tile
constexpr int KPAD = 8;          // bf16 elements of row padding (16 bytes)
}  // namespace fwd

template <int D>
__global__ void __launch_bounds__(256, 2)
fwd_mfma_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                const bf16_t* __restrict__ v, float* __restrict__ o, float* __restrict__ lse,
                int BH, int Hq, int Hkv, int N, int causal, float scale, int nqt) {
    using namespace fwd;
    constexpr int DC = D / 16;   // 16-deep chunks of the head dimension
    constexpr int DB = D / 32;   // 32-wide blocks of the head dimension
    constexpr int NB = BC / 32;  // 32-key blocks per tile
    __shared__ __attribute__((aligned(16))) bf16_t Ks[BC][D + KPAD];
    __shared__ __attribute__((aligned(16))) _Float16 Vt[D][BC + KPAD];

    const int wg = blockIdx.x;
    const int qt = nqt - 1 - wg / BH;   // longest query tiles first
    const int bh = wg % BH;
    const int b = bh / Hq, hq = bh % Hq, hkv = hq / (Hq / Hkv);
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, h = lane >> 5, r = lane & 31;
    const int q0w = qt * BR + 32 * w;    // first query row of this wave
    const int qi = q0w + r;              // this lane's query row
    const bf16_t* qh = q + (size_t)bh * N * D;
    const bf16_t* kh = k + ((size_t)b * Hkv + hkv) * N * D;
    const bf16_t* vh = v + ((size_t)b * Hkv + hkv) * N * D;
    const float sl2 = scale * kLog2e;    // scores in log2 units

    // Q rows of this wave as B operands: lane holds Q[qi][16c + 8h .. +7]
    bf16x8 qb[DC];
#pragma unroll
    for (int c = 0; c < DC; ++c) {
        if (qi < N) qb[c] = *reinterpret_cast<const bf16x8*>(qh + (size_t)qi * D + 16 * c + 8 * h);
        else qb[c] = bf16x8{};
    }
    f32x16 oacc[DB];
#pragma unroll
    for (int x = 0; x < DB; ++x) oacc[x] = f32x16{};
    float m_run = -INFINITY;   // running max, log2 units
    float l_run = 0.f;         // running sum of this lane's keys (other half added at the end)

    const int last_q = min(N, (qt + 1) * BR) - 1;
    const int kend = causal ? last_q + 1 : N;   // keys needed by this workgroup
    for (int k0 = 0; k0 < kend; k0 += BC) {
        // ---- stage K rows (bf16, 16-byte chunks)
        constexpr int KCH = BC * D / 8;
#pragma unroll
        for (int u = 0; u < KCH / 256; ++u) {
            const int cid = tid + 256 * u;
            const int row = cid / (D / 8), col = (cid % (D / 8)) * 8;
            uint4 val = {0u, 0u, 0u, 0u};
            if (k0 + row < N) val = *reinterpret_cast<const uint4*>(kh + (size_t)(k0 + row) * D + col);
            *reinterpret_cast<uint4*>(&Ks[row][col]) = val;
        }
        // ---- stage V transposed as fp16: each item is 4 keys x 4 dims
        constexpr int VIT = (BC / 4) * (D / 4);
#pragma unroll
        for (int u = 0; u < (VIT + 255) / 256; ++u) {
            const int it = tid + 256 * u;
            if (VIT % 256 == 0 || it < VIT) {
                const int dq4 = it % (D / 4), kq4 = it / (D / 4);
                uint2 rows[4];
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int key = k0 + 4 * kq4 + rr;
                    rows[rr] = (key < N) ? *reinterpret_cast<const uint2*>(vh + (size_t)key * D + 4 * dq4)
                                         : uint2{0u, 0u};
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float f[4];
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) {
                        const uint32_t wv = (e < 2) ? rows[rr].x : rows[rr].y;
                        f[rr] = (e & 1) ? bf16_hi(wv) : bf16_lo(wv);
                    }
                    uint2 pk = {pack_f16(f[0], f[1]), pack_f16(f[2], f[3])};
                    *reinterpret_cast<uint2*>(&Vt[4 * dq4 + e][4 * kq4]) = pk;
                }
            }
        }
        __syncthreads();

        const bool active = !causal || k0 <= q0w + 31;
        if (active) {
            // ---- S^T = K * Q^T  (rows: keys, permuted; columns: this wave's queries)
            f32x16 s[NB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) s[nb] = f32x16{};
#pragma unroll
            for (int c = 0; c < DC; ++c) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8*>(&Ks[32 * nb + perm32(r)][16 * c + 8 * h]);
                    s[nb] = mfma_bf16(a, qb[c], s[nb]);
                }
            }
            // ---- mask (only tiles crossing the diagonal or the sequence end)
            const bool need_mask = (k0 + BC > N) || (causal && k0 + BC - 1 > q0w);
            if (need_mask) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int key = k0 + 32 * nb + 16 * (e >> 3) + 8 * h + (e & 7);
                        if (key >= N || (causal && key > qi)) s[nb][e] = -INFINITY;
                    }
            }
            // ---- online softmax (log2 domain)
            float mx = -INFINITY;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[nb][e]);
            mx = fmaxf(mx, swap_halves(mx));
            const float m_new = fmaxf(m_run, mx * sl2);
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
            const float alpha = fast_exp2(m_run - m_use);
            float psum = 0.f;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const float p = fast_exp2(fmaf(s[nb][e], sl2, -m_use));
                    s[nb][e] = p;
                    psum += p;
                }
            l_run = fmaf(l_run, alpha, psum);
            m_run = m_new;
#pragma unroll
            for (int x = 0; x < DB; ++x)
#pragma unroll
                for (int e = 0; e < 16; ++e) oacc[x][e] *= alpha;
            // ---- O^T += V^T * P^T   (A: V^T rows from LDS, B: P from registers)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int c2 = 0; c2 < 2; ++c2) {
                    const f16x8 pb = to_f16x8(s[nb][8 * c2 + 0], s[nb][8 * c2 + 1], s[nb][8 * c2 + 2],
                                              s[nb][8 * c2 + 3], s[nb][8 * c2 + 4], s[nb][8 * c2 + 5],
                                              s[nb][8 * c2 + 6], s[nb][8 * c2 + 7]);
#pragma unroll
                    for (int x = 0; x < DB; ++x) {
                        const f16x8 a = *reinterpret_cast<const f16x8*>(&Vt[32 * x + r][32 * nb + 16 * c2 + 8 * h]);
                        oacc[x] = mfma_f16(a, pb, oacc[x]);
                    }
                }
        }
        __syncthreads();
    }

    // ---- epilogue: normalise, store O (fp32) and LSE (natural log)
    const float l_tot = l_run + swap_halves(l_run);
    if (qi < N) {
        const float inv = 1.f / l_tot;
        float* orow = o + ((size_t)bh * N + qi) * D;
#pragma unroll
        for (int x = 0; x < DB; ++x)
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4) {
                float4 val = {oacc[x][4 * a4 + 0] * inv, oacc[x][4 * a4 + 1] * inv,
                              oacc[x][4 * a4 + 2] * inv, oacc[x][4 * a4 + 3] * inv};
                *reinterpret_cast<float4*>(orow + 32 * x + 8 * a4 + 4 * h) = val;
            }
        if (h == 0) lse[(size_t)bh * N + qi] = (m_run + __log2f(l_tot)) * kLn2;
    }
}

bool mfma_path(const AttnArgs& a) { return a.dtype == ATTN_BF16 && (a.d == 64 || a.d == 128); }

hipError_t launch_fwd_mfma(const AttnArgs& a, hipStream_t st) {
    const int BH = a.B * a.Hq;
    const int nqt = (a.N + fwd::BR - 1) / fwd::BR;
    const dim3 grid((unsigned)(nqt * BH));
    if (a.d == 64)
        hipLaunchKernelGGL(fwd_mfma_kernel<64>, grid, dim3(256), 0, st, (const bf16_t*)a.q,
                           (const bf16_t*)a.k, (const bf16_t*)a.v, a.o, a.lse, BH, a.Hq, a.Hkv, a.N,
                           a.causal, a.scale, nqt);
    else
        hipLaunchKernelGGL(fwd_mfma_kernel<128>, grid, dim3(256), 0, st, (const bf16_t*)a.q,
                           (const bf16_t*)a.k, (const bf16_t*)a.v, a.o, a.lse, BH, a.Hq, a.Hkv, a.N,
                           a.causal, a.scale, nqt);
    return hipGetLastError();
}

}  // namespace tca
