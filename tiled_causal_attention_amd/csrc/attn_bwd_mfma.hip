// attn_bwd_mfma.hip -- causal GQA attention backward on gfx950 matrix cores.
//
// K/V-tile parallel: a workgroup owns BC = 128 keys of one (batch, query head)
// and keeps their dK, dV accumulators in registers while it walks the query
// tiles at or below the diagonal. For every query tile (BR rows):
//
//   S    = Q K^T           bf16 product, fp32 accumulate     (P recomputed:)
//   P    = exp2(S*scale*log2e - LSE*log2e)   from the forward's saved LSE
//   dP   = dO V^T          bf16 product
//   dS   = P o (dP - D)    D = rowsum(dO o O) from the preprocess kernel
//   dV  += P^T dO          fp16 product (P rounded to fp16)
//   dK  += dS^T Q          fp16 product (dS rounded to fp16)
//   dQ  += dS K * scale    fp16 product, added to global dq with fp32 atomics
//
// Layout choices (see tca_device.h for the operand layouts):
//  * S and dP are computed with queries as rows and keys as columns, so each
//    lane owns one key; P and dS are then already in the A-operand layout of
//    the two products that contract over queries (dV, dK).
//  * Q and dO tiles are staged twice: as bf16 rows (A operands of S and dP,
//    read at row perm32(m) so accumulator e holds query 16(e/8) + 8h + e%8)
//    and transposed as fp16 ([d][query], B operands of dV and dK).
//  * dQ contracts over keys, so dS goes through LDS ([query][key], fp16) and
//    the four waves split the BR x d dQ tile into 32x32 blocks; K^T (fp16) is
//    staged once per workgroup for it.
//  * When several query heads share a KV head, each head's workgroup adds its
//    dK, dV into fp32 outputs cleared by the preprocess (atomics); with one
//    query head per KV head they are stored directly.
//  * Grid order: K/V tile 0 (the longest causal walk) first.
#include "tca_internal.h"

namespace tca {

namespace bwd {
constexpr int NW = 4;
constexpr int BC = 32 * NW;   // keys per workgroup
constexpr int PAD = 8;        // 16-bit elements of row padding (16 bytes)
template <int D> struct Cfg;
template <> struct Cfg<64> { static constexpr int BR = 64; };
template <> struct Cfg<128> { static constexpr int BR = 32; };
}  // namespace bwd

template <int D, bool ATOMIC_KV>
__global__ void __launch_bounds__(256, (D == 64) ? 2 : 1)
bwd_mfma_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                const bf16_t* __restrict__ v, const float* __restrict__ lse,
                const bf16_t* __restrict__ dout, const float* __restrict__ delta,
                float* __restrict__ dq, float* __restrict__ dk, float* __restrict__ dv,
                int BH, int Hq, int Hkv, int N, int causal, float scale) {
    using namespace bwd;
    constexpr int BR = Cfg<D>::BR;
    constexpr int DC = D / 16, DB = D / 32, QB = BR / 32;
    __shared__ __attribute__((aligned(16))) bf16_t Qs[BR][D + PAD];
    __shared__ __attribute__((aligned(16))) bf16_t dOs[BR][D + PAD];
    __shared__ __attribute__((aligned(16))) _Float16 Qt[D][BR + PAD];
    __shared__ __attribute__((aligned(16))) _Float16 dOt[D][BR + PAD];
    __shared__ __attribute__((aligned(16))) float Ls[BR];
    __shared__ __attribute__((aligned(16))) float Dl[BR];
    __shared__ __attribute__((aligned(16))) _Float16 dSs[BR][BC + PAD];
    __shared__ __attribute__((aligned(16))) _Float16 Kt[D][BC + PAD];

    const int wg = blockIdx.x;
    const int kt = wg / BH;           // K/V tile: tile 0 has the longest causal walk
    const int bh = wg % BH;
    const int b = bh / Hq, hq = bh % Hq, hkv = hq / (Hq / Hkv);
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, h = lane >> 5, r = lane & 31;
    const int kbase = kt * BC;
    const int kw = kbase + 32 * w + r;   // this lane's key
    const size_t kvoff = ((size_t)b * Hkv + hkv) * N * D;
    const bf16_t* kh = k + kvoff;
    const bf16_t* vh = v + kvoff;
    const bf16_t* qh = q + (size_t)bh * N * D;
    const bf16_t* doh = dout + (size_t)bh * N * D;
    const float* lseh = lse + (size_t)bh * N;
    const float* delh = delta + (size_t)bh * N;
    float* dqh = dq + (size_t)bh * N * D;
    const float sl2 = scale * kLog2e;

    // K and V rows of this lane's key as B operands (lane holds row kw, dims 16c + 8h .. +7)
    bf16x8 kb[DC], vb[DC];
#pragma unroll
    for (int c = 0; c < DC; ++c) {
        if (kw < N) {
            kb[c] = *reinterpret_cast<const bf16x8*>(kh + (size_t)kw * D + 16 * c + 8 * h);
            vb[c] = *reinterpret_cast<const bf16x8*>(vh + (size_t)kw * D + 16 * c + 8 * h);
        } else {
            kb[c] = bf16x8{};
            vb[c] = bf16x8{};
        }
    }
    // K^T (fp16) for the dQ product: items of 4 keys x 4 dims
    {
        constexpr int IT = (BC / 4) * (D / 4);
#pragma unroll
        for (int u = 0; u < IT / 256; ++u) {
            const int it = tid + 256 * u;
            const int dq4 = it % (D / 4), kq4 = it / (D / 4);
            uint2 rows[4];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int key = kbase + 4 * kq4 + rr;
                rows[rr] = (key < N) ? *reinterpret_cast<const uint2*>(kh + (size_t)key * D + 4 * dq4)
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
                *reinterpret_cast<uint2*>(&Kt[4 * dq4 + e][4 * kq4]) = uint2{pack_f16(f[0], f[1]), pack_f16(f[2], f[3])};
            }
        }
    }

    f32x16 dka[DB], dva[DB];
#pragma unroll
    for (int x = 0; x < DB; ++x) {
        dka[x] = f32x16{};
        dva[x] = f32x16{};
    }

    const int nqt = (N + BR - 1) / BR;
    const int qt0 = causal ? kbase / BR : 0;
    for (int qt = qt0; qt < nqt; ++qt) {
        const int qbase = qt * BR;
        __syncthreads();   // the previous step is done reading LDS
        // ---- stage Q and dO: bf16 rows and fp16 transposed, items of 4 rows x 4 dims
        {
            constexpr int IT = (BR / 4) * (D / 4);
#pragma unroll
            for (int u = 0; u < (IT + 255) / 256; ++u) {
                const int it = tid + 256 * u;
                if (IT % 256 == 0 || it < IT) {
                    const int dq4 = it % (D / 4), rq4 = it / (D / 4);
                    uint2 qr[4], dr[4];
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) {
                        const int row = qbase + 4 * rq4 + rr;
                        if (row < N) {
                            qr[rr] = *reinterpret_cast<const uint2*>(qh + (size_t)row * D + 4 * dq4);
                            dr[rr] = *reinterpret_cast<const uint2*>(doh + (size_t)row * D + 4 * dq4);
                        } else {
                            qr[rr] = uint2{0u, 0u};
                            dr[rr] = uint2{0u, 0u};
                        }
                        *reinterpret_cast<uint2*>(&Qs[4 * rq4 + rr][4 * dq4]) = qr[rr];
                        *reinterpret_cast<uint2*>(&dOs[4 * rq4 + rr][4 * dq4]) = dr[rr];
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        float fq[4], fd[4];
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr) {
                            const uint32_t wq = (e < 2) ? qr[rr].x : qr[rr].y;
                            const uint32_t wd = (e < 2) ? dr[rr].x : dr[rr].y;
                            fq[rr] = (e & 1) ? bf16_hi(wq) : bf16_lo(wq);
                            fd[rr] = (e & 1) ? bf16_hi(wd) : bf16_lo(wd);
                        }
                        *reinterpret_cast<uint2*>(&Qt[4 * dq4 + e][4 * rq4]) =
                            uint2{pack_f16(fq[0], fq[1]), pack_f16(fq[2], fq[3])};
                        *reinterpret_cast<uint2*>(&dOt[4 * dq4 + e][4 * rq4]) =
                            uint2{pack_f16(fd[0], fd[1]), pack_f16(fd[2], fd[3])};
                    }
                }
            }
            if (tid < BR) {
                const int row = qbase + tid;
                Ls[tid] = (row < N) ? lseh[row] * kLog2e : 0.f;
                Dl[tid] = (row < N) ? delh[row] : 0.f;
            }
        }
        __syncthreads();

        // ---- S = Q K^T and dP = dO V^T (rows: queries, permuted; columns: this wave's keys)
        f32x16 s[QB], dp[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            s[qb] = f32x16{};
            dp[qb] = f32x16{};
        }
#pragma unroll
        for (int c = 0; c < DC; ++c)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const bf16x8 aq = *reinterpret_cast<const bf16x8*>(&Qs[32 * qb + perm32(r)][16 * c + 8 * h]);
                const bf16x8 ad = *reinterpret_cast<const bf16x8*>(&dOs[32 * qb + perm32(r)][16 * c + 8 * h]);
                s[qb] = mfma_bf16(aq, kb[c], s[qb]);
                dp[qb] = mfma_bf16(ad, vb[c], dp[qb]);
            }

        // ---- P and dS (accumulator e of block qb: query qbase + 32qb + 16(e/8) + 8h + e%8)
        const int kw0 = kbase + 32 * w;
        const bool need_mask = (qbase + BR > N) || (kw0 + 32 > N) || (causal && qbase < kw0 + 31);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) {
                const int qq = 32 * qb + 16 * c2 + 8 * h;   // first tile row of this 8-group
                const float4 l0 = *reinterpret_cast<const float4*>(&Ls[qq]);
                const float4 l1 = *reinterpret_cast<const float4*>(&Ls[qq + 4]);
                const float4 d0 = *reinterpret_cast<const float4*>(&Dl[qq]);
                const float4 d1 = *reinterpret_cast<const float4*>(&Dl[qq + 4]);
                const float lv[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
                const float dl[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const int e = 8 * c2 + t;
                    float p = fast_exp2(fmaf(s[qb][e], sl2, -lv[t]));
                    if (need_mask) {
                        const int qrow = qbase + qq + t;
                        if (qrow >= N || kw >= N || (causal && kw > qrow)) p = 0.f;
                    }
                    s[qb][e] = p;
                    dp[qb][e] = p * (dp[qb][e] - dl[t]);
                }
            }

        // ---- dV += P^T dO and dK += dS^T Q  (A: this lane's key row; B: transposed tiles)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) {
                const int e0 = 8 * c2;
                const f16x8 pa = to_f16x8(s[qb][e0 + 0], s[qb][e0 + 1], s[qb][e0 + 2], s[qb][e0 + 3],
                                          s[qb][e0 + 4], s[qb][e0 + 5], s[qb][e0 + 6], s[qb][e0 + 7]);
                const f16x8 da = to_f16x8(dp[qb][e0 + 0], dp[qb][e0 + 1], dp[qb][e0 + 2], dp[qb][e0 + 3],
                                          dp[qb][e0 + 4], dp[qb][e0 + 5], dp[qb][e0 + 6], dp[qb][e0 + 7]);
                const int qq = 32 * qb + 16 * c2 + 8 * h;
#pragma unroll
                for (int x = 0; x < DB; ++x) {
                    const f16x8 bo = *reinterpret_cast<const f16x8*>(&dOt[32 * x + r][qq]);
                    const f16x8 bq = *reinterpret_cast<const f16x8*>(&Qt[32 * x + r][qq]);
                    dva[x] = mfma_f16(pa, bo, dva[x]);
                    dka[x] = mfma_f16(da, bq, dka[x]);
                }
                // dS to LDS as [query][key] for the dQ product
#pragma unroll
                for (int t = 0; t < 8; ++t) dSs[qq + t][32 * w + r] = da[t];
            }
        __syncthreads();

        // ---- dQ (BR x D) += dS (BR x BC) * K (BC x D), 32x32 blocks split over the waves
#pragma unroll
        for (int blk = w; blk < QB * DB; blk += NW) {
            const int qb = blk / DB, x = blk % DB;
            f32x16 acc = f32x16{};
#pragma unroll
            for (int kc = 0; kc < BC / 16; ++kc) {
                const f16x8 a = *reinterpret_cast<const f16x8*>(&dSs[32 * qb + r][16 * kc + 8 * h]);
                const f16x8 bk = *reinterpret_cast<const f16x8*>(&Kt[32 * x + r][16 * kc + 8 * h]);
                acc = mfma_f16(a, bk, acc);
            }
            // accumulator e: query 32qb + 8(e/4) + 4h + e%4, dim 32x + r
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int qrow = qbase + 32 * qb + 8 * (e >> 2) + 4 * h + (e & 3);
                if (qrow < N) unsafeAtomicAdd(dqh + (size_t)qrow * D + 32 * x + r, scale * acc[e]);
            }
        }
    }

    // ---- epilogue: accumulator e of dim block x holds key kbase + 32w + 8(e/4) + 4h + e%4, dim 32x + r
#pragma unroll
    for (int x = 0; x < DB; ++x)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int key = kbase + 32 * w + 8 * (e >> 2) + 4 * h + (e & 3);
            if (key < N) {
                const size_t off = kvoff + (size_t)key * D + 32 * x + r;
                if (ATOMIC_KV) {
                    unsafeAtomicAdd(dk + off, scale * dka[x][e]);
                    unsafeAtomicAdd(dv + off, dva[x][e]);
                } else {
                    dk[off] = scale * dka[x][e];
                    dv[off] = dva[x][e];
                }
            }
        }
}

bool bwd_mfma_atomic_dkdv(const AttnArgs& a) { return a.Hq != a.Hkv; }

template <int D>
static hipError_t launch_bwd_mfma_d(const AttnArgs& a, hipStream_t st) {
    const int BH = a.B * a.Hq;
    const int nkt = (a.N + bwd::BC - 1) / bwd::BC;
    const dim3 grid((unsigned)(nkt * BH));
    if (bwd_mfma_atomic_dkdv(a))
        hipLaunchKernelGGL((bwd_mfma_kernel<D, true>), grid, dim3(256), 0, st, (const bf16_t*)a.q,
                           (const bf16_t*)a.k, (const bf16_t*)a.v, (const float*)a.lse,
                           (const bf16_t*)a.dout, (const float*)a.workspace, a.dq, a.dk, a.dv, BH,
                           a.Hq, a.Hkv, a.N, a.causal, a.scale);
    else
        hipLaunchKernelGGL((bwd_mfma_kernel<D, false>), grid, dim3(256), 0, st, (const bf16_t*)a.q,
                           (const bf16_t*)a.k, (const bf16_t*)a.v, (const float*)a.lse,
                           (const bf16_t*)a.dout, (const float*)a.workspace, a.dq, a.dk, a.dv, BH,
                           a.Hq, a.Hkv, a.N, a.causal, a.scale);
    return hipGetLastError();
}

hipError_t launch_bwd_mfma(const AttnArgs& a, hipStream_t st) {
    return (a.d == 64) ? launch_bwd_mfma_d<64>(a, st) : launch_bwd_mfma_d<128>(a, st);
}

}  // namespace tca
