// mix_ceiling.hip -- what the attention kernels' per-block instruction mixes can
// reach on gfx950 matrix cores when nothing else is in the way (not part of the
// attention library; the benchmark report's --ceiling mode runs it).
//
// Each wave loops over one 32 x 32 block of (query, key) pairs per iteration and
// issues the instructions a kernel issues for such a block, with the same data
// dependences (scores -> softmax -> probability product), but no global memory
// traffic: operands sit in LDS tiles (or registers) that are never refreshed,
// so the loop measures the issue, latency and co-issue limits of the mix itself.
// The mixes:
//   MFMA_ONLY   8 independent 32x32x16 products (two chains of 4), no VALU
//   EXP_ONLY    16 v_exp_f32, FMA_ONLY 16 v_fma_f32, CVT_ONLY 8 v_cvt_pk_f16_f32
//               (independent values; the per-instruction issue cost)
//   FWD         the forward at d = 64: S^T = K Q^T from LDS (4 products), row
//               max, lazy-rescale test, 16 exp2 of fma(s, c, -m), fp16 packing,
//               row sum by v_dot2, O^T += V^T P^T with V read transposed (4)
//   FWD_REG     FWD with both operands of every product in registers (no LDS)
//   FWD_STAGED  FWD plus the per-tile K/V staging of the real kernel (2 + 2
//               16-byte chunks per lane stored to the other LDS buffer, V
//               converted bf16 -> fp16) and one workgroup barrier per block
//   DQ          the dQ pass at d = 64: S^T, dP^T - D (8 products), 16 exp,
//               dS = P (dP - D), fp16 packing, dQ^T += K^T dS^T (4 products)
//   DKDV        the dK/dV pass at d = 64: S, dP - D (8 products, A from LDS),
//               16 exp, dS, fp16 packing of P and dS, dV += P^T dO and
//               dK += dS^T Q with the B operands read transposed (8 products)
//   FWD_2Q      FWD with 64 queries per wave: each K (and V) operand read from LDS
//               feeds the products of two 32-query blocks (16 products per iteration)
//   FWD_W8      FWD in 8-wave workgroups (two waves of a workgroup per SIMD)
//   FWD_PP      FWD_W8 with the two 4-wave halves ping-ponging: one half issues the
//               products while the other computes the softmax, barrier-separated
// Every wave records the s_memtime and s_memrealtime (100 MHz) counters around
// its loop; the real-time count gives nanoseconds per block.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mix {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

enum Mix { MFMA_ONLY = 0, EXP_ONLY, FMA_ONLY, CVT_ONLY, FWD, FWD_REG, FWD_STAGED, DQ, DKDV, FWD_W8, FWD_PP, FWD_2Q,
           NUM_MIX };

constexpr int LD = 72;                 // LDS row stride (16-bit elements), as the kernels' d = 64 tiles
constexpr int TILE = 64 * LD;          // one 64-row tile
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_f16(f16x8 a, f16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float vmax3(float a, float b, float c) { return vmax(vmax(a, b), c); }
__device__ __forceinline__ float max16(const f32x16& s) {
    const float a = vmax3(s[0], s[1], s[2]), b = vmax3(s[3], s[4], s[5]), c = vmax3(s[6], s[7], s[8]);
    const float d = vmax3(s[9], s[10], s[11]), e = vmax3(s[12], s[13], s[14]);
    return vmax(vmax3(a, b, c), vmax3(d, e, s[15]));
}
__device__ __forceinline__ float max_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
    f16x2 h = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, h);
}
__device__ __forceinline__ float add_f16_pair(uint32_t pair, float acc) {
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pair), one, acc, false);
}
__device__ __forceinline__ f16x8 to_f16x8(const f32x16& s, int c2) {
    f16x8 r;
#pragma unroll
    for (int t = 0; t < 8; ++t) r[t] = (_Float16)s[8 * c2 + t];
    return r;
}
__device__ __forceinline__ int perm32(int m) { return (m & ~0xC) | ((m & 4) << 1) | ((m & 8) >> 1); }
// lane (h, r) <- tile[row0 + 8h + t][col0 + r], t = 0..7 (transposing LDS reads)
__device__ __forceinline__ f16x8 tr_operand(const _Float16* tile, int row0, int col0, int h, int r) {
    const _Float16* p = tile + (row0 + 8 * h + ((r & 15) >> 2)) * LD + col0 + 16 * (r >> 4) + 4 * (r & 3);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 4 * LD));
    const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(f16x8, v);
}
__device__ __forceinline__ uint32_t cvt_bf16pair_f16(uint32_t w) {
    return pack_f16(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
}

template <int M> constexpr int kMinWaves = (M == DKDV || M == DQ || M == FWD_2Q) ? 2 : 4;

template <int M>
__global__ void __launch_bounds__(256, kMinWaves<M>)
mix_kernel(float* __restrict__ out, unsigned long long* __restrict__ cycles, int iters) {
    // two 64-row tiles per operand kind, double-buffered as the kernels' K/V tiles
    __shared__ __attribute__((aligned(16))) _Float16 A0[2 * TILE];   // K (bf16 bits) / Q
    __shared__ __attribute__((aligned(16))) _Float16 A1[2 * TILE];   // V (fp16) / dO
    __shared__ __attribute__((aligned(16))) float stat[2][128];       // row statistics (dK/dV pass)
    const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, r = lane & 31;
    // small bounded values, so every exponential stays in range
    for (int i = tid; i < 2 * TILE; i += 256) {
        const float x = (float)((i * 37 + 11) % 61) * (1.f / 256.f) - 0.1f;
        A1[i] = (_Float16)x;
        if (M == FWD || M == FWD_REG || M == FWD_STAGED) {
            const __bf16 b = (__bf16)x;
            A0[i] = __builtin_bit_cast(_Float16, b);
        } else {
            A0[i] = (_Float16)(-x);
        }
    }
    for (int i = tid; i < 256; i += 256) stat[i >> 7][i & 127] = 0.25f - (float)(i % 5) * 0.05f;
    __syncthreads();

    bf16x8 qb[4];
    f16x8 kb[4], vb[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float x = (float)((lane * 7 + c * 3 + i) % 9) * 0.05f - 0.2f;
            qb[c][i] = (__bf16)x;
            kb[c][i] = (_Float16)(x * 0.5f);
            vb[c][i] = (_Float16)(0.3f - x);
        }
    const float sl2 = 0.125f * kLog2e;
    f32x16 acc[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) acc[x] = f32x16{};
    float m_s = -0x1p100f, l_run = 0.f;
    float vals[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) vals[t] = (float)((lane + t) & 7) * 0.01f;
    u32x4 stg[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) stg[u] = u32x4{(uint32_t)(lane * 0x10001u + u), 0x3f803f80u, 0x3e003e00u, 0x3c003c00u};
    const int krow = perm32(r);

    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
        __asm__ volatile("" ::: "memory");   // the tiles are re-read every iteration
        const int buf = it & 1;
        const _Float16* a0 = A0 + buf * TILE;
        const _Float16* a1 = A1 + buf * TILE;
        if constexpr (M == MFMA_ONLY) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                acc[0] = mfma_bf16(qb[c], qb[(c + 1) & 3], acc[0]);
                acc[1] = mfma_f16(kb[c], vb[c], acc[1]);
            }
        } else if constexpr (M == EXP_ONLY) {
#pragma unroll
            for (int t = 0; t < 16; ++t) vals[t] = __builtin_amdgcn_exp2f(vals[t]);
        } else if constexpr (M == FMA_ONLY) {
#pragma unroll
            for (int t = 0; t < 16; ++t) vals[t] = fmaf(vals[t], sl2, -0.25f);
        } else if constexpr (M == CVT_ONLY) {
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const uint32_t p = pack_f16(vals[2 * t], vals[2 * t + 1]);
                vals[2 * t] = __uint_as_float(p);
            }
        } else if constexpr (M == FWD || M == FWD_REG || M == FWD_STAGED) {
            f32x16 s = f32x16{};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const bf16x8 a = (M == FWD_REG) ? qb[(c + 2) & 3]
                                                : *reinterpret_cast<const bf16x8*>(a0 + (32 * buf + krow) * LD + 16 * c + 8 * h);
                s = mfma_bf16(a, qb[c], s);
            }
            const float mt = max_halves(max16(s)) * sl2;
            if (__any(mt > m_s + 8.f)) {
                const float m_new = vmax(m_s, mt);
                const float alpha = __builtin_amdgcn_exp2f(m_s - m_new);
                l_run *= alpha;
#pragma unroll
                for (int x = 0; x < 2; ++x)
#pragma unroll
                    for (int e = 0; e < 16; ++e) acc[x][e] *= alpha;
                m_s = m_new;
            }
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) {
                uint32_t pk[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const float p0 = __builtin_amdgcn_exp2f(fmaf(s[8 * c2 + 2 * t], sl2, -m_s));
                    const float p1 = __builtin_amdgcn_exp2f(fmaf(s[8 * c2 + 2 * t + 1], sl2, -m_s));
                    pk[t] = pack_f16(p0, p1);
                    l_run = add_f16_pair(pk[t], l_run);
                }
                const f16x8 pb = __builtin_bit_cast(f16x8, u32x4{pk[0], pk[1], pk[2], pk[3]});
#pragma unroll
                for (int x = 0; x < 2; ++x) {
                    const f16x8 a = (M == FWD_REG) ? vb[2 * c2 + x] : tr_operand(a1, 16 * c2, 32 * x, h, r);
                    acc[x] = mfma_f16(a, pb, acc[x]);
                }
            }
            if constexpr (M == FWD_STAGED) {
                // the next tile into the other buffer: K as is, V converted to fp16
                const int row = tid >> 3, col = (tid & 7) * 8;
                _Float16* kd = A0 + (buf ^ 1) * TILE + row * LD + col;
                _Float16* vd = A1 + (buf ^ 1) * TILE + row * LD + col;
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const u32x4 kw = stg[u] ^ (uint32_t)it, vw = stg[u + 2] ^ (uint32_t)(it & 0x00ff00ff);
                    *reinterpret_cast<u32x4*>(kd + u * 32 * LD) = kw & 0x3fff3fffu;
                    *reinterpret_cast<u32x4*>(vd + u * 32 * LD) =
                        u32x4{cvt_bf16pair_f16(vw.x & 0x3fff3fffu), cvt_bf16pair_f16(vw.y & 0x3fff3fffu),
                              cvt_bf16pair_f16(vw.z & 0x3fff3fffu), cvt_bf16pair_f16(vw.w & 0x3fff3fffu)};
                }
                __syncthreads();
            }
        } else if constexpr (M == FWD_2Q) {
            // two 32-query blocks per K/V operand read (64 queries x 32 keys per iteration,
            // counted as two blocks): Q of the second block in kb's registers
            f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(a0 + (32 * buf + krow) * LD + 16 * c + 8 * h);
                s0 = mfma_bf16(a, qb[c], s0);
                s1 = mfma_bf16(a, __builtin_bit_cast(bf16x8, kb[c]), s1);
            }
            float ms[2] = {m_s, l_run};   // per-block running max (second block keeps its own)
            f32x16* sp[2] = {&s0, &s1};
#pragma unroll
            for (int qb2 = 0; qb2 < 2; ++qb2) {
                f32x16& sv = *sp[qb2];
                const float mt = max_halves(max16(sv)) * sl2;
                if (__any(mt > ms[qb2] + 8.f)) {
                    const float m_new = vmax(ms[qb2], mt);
                    const float alpha = __builtin_amdgcn_exp2f(ms[qb2] - m_new);
                    vals[qb2] *= alpha;
#pragma unroll
                    for (int x = 0; x < 2; ++x)
#pragma unroll
                        for (int e = 0; e < 16; ++e) acc[2 * qb2 + x][e] *= alpha;
                    ms[qb2] = m_new;
                }
            }
            m_s = ms[0];
            l_run = ms[1];
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) {
                f16x8 pb[2];
#pragma unroll
                for (int qb2 = 0; qb2 < 2; ++qb2) {
                    f32x16& sv = *sp[qb2];
                    uint32_t pk[4];
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const float p0 = __builtin_amdgcn_exp2f(fmaf(sv[8 * c2 + 2 * t], sl2, -ms[qb2]));
                        const float p1 = __builtin_amdgcn_exp2f(fmaf(sv[8 * c2 + 2 * t + 1], sl2, -ms[qb2]));
                        pk[t] = pack_f16(p0, p1);
                        vals[qb2] = add_f16_pair(pk[t], vals[qb2]);
                    }
                    pb[qb2] = __builtin_bit_cast(f16x8, u32x4{pk[0], pk[1], pk[2], pk[3]});
                }
#pragma unroll
                for (int x = 0; x < 2; ++x) {
                    const f16x8 a = tr_operand(a1, 16 * c2, 32 * x, h, r);
                    acc[x] = mfma_f16(a, pb[0], acc[x]);
                    acc[2 + x] = mfma_f16(a, pb[1], acc[2 + x]);
                }
            }
        } else if constexpr (M == DQ) {
            f32x16 s = f32x16{}, dp = f32x16{} - 0.3f;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const f16x8 ak = *reinterpret_cast<const f16x8*>(a0 + (32 * buf + krow) * LD + 16 * c + 8 * h);
                const bf16x8 av = *reinterpret_cast<const bf16x8*>(a1 + (32 * buf + krow) * LD + 16 * c + 8 * h);
                s = mfma_f16(ak, kb[c], s);
                dp = mfma_bf16(av, qb[c], dp);
            }
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const float p = __builtin_amdgcn_exp2f(fmaf(s[e], sl2, -0.5f));
                s[e] = p * dp[e];
            }
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) {
                const f16x8 dsb = to_f16x8(s, c2);
#pragma unroll
                for (int x = 0; x < 2; ++x) acc[x] = mfma_f16(tr_operand(a0, 32 * buf + 16 * c2, 32 * x, h, r), dsb, acc[x]);
            }
        } else if constexpr (M == DKDV) {
            const float* Dt = stat[buf];
            f32x16 s = f32x16{}, dp;
            {
                const int qq = 8 * h;
                const f32x4 d0 = *reinterpret_cast<const f32x4*>(Dt + qq), d1 = *reinterpret_cast<const f32x4*>(Dt + qq + 4);
                const f32x4 d2 = *reinterpret_cast<const f32x4*>(Dt + qq + 16), d3 = *reinterpret_cast<const f32x4*>(Dt + qq + 20);
                dp = f32x16{d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3],
                            d2[0], d2[1], d2[2], d2[3], d3[0], d3[1], d3[2], d3[3]};
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int off = (32 * buf + krow) * LD + 16 * c + 8 * h;
                s = mfma_f16(*reinterpret_cast<const f16x8*>(a0 + off), kb[c], s);
                dp = mfma_f16(*reinterpret_cast<const f16x8*>(a1 + off), vb[c], dp);
            }
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) {
                const f32x4 l0 = *reinterpret_cast<const f32x4*>(Dt + 64 + 16 * c2 + 8 * h);
                const f32x4 l1 = *reinterpret_cast<const f32x4*>(Dt + 64 + 16 * c2 + 8 * h + 4);
                const float lv[8] = {l0[0], l0[1], l0[2], l0[3], l1[0], l1[1], l1[2], l1[3]};
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const int e = 8 * c2 + t;
                    const float p = __builtin_amdgcn_exp2f(fmaf(s[e], sl2, -lv[t]));
                    s[e] = p;
                    dp[e] = p * dp[e];
                }
            }
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) {
                const f16x8 pa = to_f16x8(s, c2), da = to_f16x8(dp, c2);
#pragma unroll
                for (int x = 0; x < 2; ++x) {
                    acc[x] = mfma_f16(pa, tr_operand(a1, 32 * buf + 16 * c2, 32 * x, h, r), acc[x]);
                    acc[2 + x] = mfma_f16(da, tr_operand(a0, 32 * buf + 16 * c2, 32 * x, h, r), acc[2 + x]);
                }
            }
        }
    }
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();

    float sum = l_run + m_s;
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int e = 0; e < 16; ++e) sum += acc[x][e];
#pragma unroll
    for (int t = 0; t < 16; ++t) sum += vals[t];
    out[blockIdx.x * 256 + tid] = sum;
    if (lane == 0) {
        cycles[2 * (blockIdx.x * 8 + (tid >> 6))] = t1 - t0;
        cycles[2 * (blockIdx.x * 8 + (tid >> 6)) + 1] = r1 - r0;
    }
}

// The forward's block with 8-wave workgroups (waves w and w + 4 share a SIMD).
// FWD_W8: every wave runs the block as FWD does. FWD_PP (ping-pong): waves 0-3
// and 4-7 are two groups whose phases are offset by one, separated by workgroup
// barriers: while one group issues its matrix products (O += V^T P^T of the
// previous block, then S^T = K Q^T of the next), the other computes the softmax
// of the scores it has, so each SIMD holds one wave in each phase.
template <int M>
__global__ void __launch_bounds__(512, 1)
mix8_kernel(float* __restrict__ out, unsigned long long* __restrict__ cycles, int iters) {
    __shared__ __attribute__((aligned(16))) _Float16 A0[2 * TILE];   // K (bf16 bits)
    __shared__ __attribute__((aligned(16))) _Float16 A1[2 * TILE];   // V (fp16)
    const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, r = lane & 31;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = w >> 2;
    for (int i = tid; i < 2 * TILE; i += 512) {
        const float x = (float)((i * 37 + 11) % 61) * (1.f / 256.f) - 0.1f;
        A1[i] = (_Float16)x;
        const __bf16 b = (__bf16)x;
        A0[i] = __builtin_bit_cast(_Float16, b);
    }
    __syncthreads();
    bf16x8 qb[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int i = 0; i < 8; ++i) qb[c][i] = (__bf16)((float)((lane * 7 + c * 3 + i) % 9) * 0.05f - 0.2f);
    const float sl2 = 0.125f * kLog2e;
    f32x16 acc[2] = {f32x16{}, f32x16{}};
    f32x16 s = f32x16{};
    f16x8 pb[2] = {f16x8{}, f16x8{}};
    float m_s = -0x1p100f, l_run = 0.f;
    const int krow = perm32(r);
    auto products = [&](int buf) {   // O^T += V^T P^T (previous block), S^T = K Q^T (next block)
        const _Float16* a0 = A0 + buf * TILE;
        const _Float16* a1 = A1 + buf * TILE;
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
            for (int x = 0; x < 2; ++x) acc[x] = mfma_f16(tr_operand(a1, 16 * c2, 32 * x, h, r), pb[c2], acc[x]);
        s = f32x16{};
#pragma unroll
        for (int c = 0; c < 4; ++c)
            s = mfma_bf16(*reinterpret_cast<const bf16x8*>(a0 + (32 * buf + krow) * LD + 16 * c + 8 * h), qb[c], s);
    };
    auto softmax = [&]() {
        const float mt = max_halves(max16(s)) * sl2;
        if (__any(mt > m_s + 8.f)) {
            const float m_new = vmax(m_s, mt);
            const float alpha = __builtin_amdgcn_exp2f(m_s - m_new);
            l_run *= alpha;
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[x][e] *= alpha;
            m_s = m_new;
        }
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
            uint32_t pk[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const float p0 = __builtin_amdgcn_exp2f(fmaf(s[8 * c2 + 2 * t], sl2, -m_s));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(s[8 * c2 + 2 * t + 1], sl2, -m_s));
                pk[t] = pack_f16(p0, p1);
                l_run = add_f16_pair(pk[t], l_run);
            }
            pb[c2] = __builtin_bit_cast(f16x8, u32x4{pk[0], pk[1], pk[2], pk[3]});
        }
    };
    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
        __asm__ volatile("" ::: "memory");
        const int buf = it & 1;
        if constexpr (M == FWD_PP) {
            if (grp == 0) products(buf); else softmax();
            __syncthreads();
            if (grp == 0) softmax(); else products(buf);
            __syncthreads();
        } else {
            products(buf);
            softmax();
        }
    }
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    float sum = l_run + m_s;
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int e = 0; e < 16; ++e) sum += acc[x][e] + s[e];
    out[blockIdx.x * 512 + tid] = sum;
    if (lane == 0) {
        cycles[2 * (blockIdx.x * 8 + w)] = t1 - t0;
        cycles[2 * (blockIdx.x * 8 + w) + 1] = r1 - r0;
    }
}

template <int M>
static hipError_t launch(float* out, unsigned long long* cycles, int blocks, int iters, hipStream_t st) {
    if constexpr (M == FWD_W8 || M == FWD_PP)
        hipLaunchKernelGGL(mix8_kernel<M>, dim3((unsigned)blocks), dim3(512), 0, st, out, cycles, iters);
    else
        hipLaunchKernelGGL(mix_kernel<M>, dim3((unsigned)blocks), dim3(256), 0, st, out, cycles, iters);
    return hipGetLastError();
}

}  // namespace mix

// Waves per workgroup of mix `mix_id`: 8 for FWD_W8 and FWD_PP, else 4.
extern "C" int tca_mix_waves_per_block(int mix_id) {
    return (mix_id == mix::FWD_W8 || mix_id == mix::FWD_PP) ? 8 : 4;
}

// Run mix `mix_id` (0 .. tca_mix_count() - 1, in the order of the Mix enum) on
// `blocks` workgroups of 64 * tca_mix_waves_per_block(mix_id) threads, each wave
// looping `iters` times over one 32x32 block. `out`: blocks * 512 floats;
// `cycles`: blocks * 8 pairs (s_memtime ticks, s_memrealtime 100 MHz ticks) around
// each wave's loop, wave w of block b at pair 8b + w (device memory, written; 4-wave
// mixes leave pairs 4..7 of each block untouched). Returns 0 or a HIP error code.
extern "C" int tca_mix_launch(int mix_id, float* out, unsigned long long* cycles, int blocks, int iters,
                              void* stream) {
    using namespace mix;
    if (out == nullptr || cycles == nullptr || blocks < 1 || iters < 1) return (int)hipErrorInvalidValue;
    hipStream_t st = (hipStream_t)stream;
    switch (mix_id) {
        case MFMA_ONLY: return (int)launch<MFMA_ONLY>(out, cycles, blocks, iters, st);
        case EXP_ONLY: return (int)launch<EXP_ONLY>(out, cycles, blocks, iters, st);
        case FMA_ONLY: return (int)launch<FMA_ONLY>(out, cycles, blocks, iters, st);
        case CVT_ONLY: return (int)launch<CVT_ONLY>(out, cycles, blocks, iters, st);
        case FWD: return (int)launch<FWD>(out, cycles, blocks, iters, st);
        case FWD_REG: return (int)launch<FWD_REG>(out, cycles, blocks, iters, st);
        case FWD_STAGED: return (int)launch<FWD_STAGED>(out, cycles, blocks, iters, st);
        case DQ: return (int)launch<DQ>(out, cycles, blocks, iters, st);
        case DKDV: return (int)launch<DKDV>(out, cycles, blocks, iters, st);
        case FWD_W8: return (int)launch<FWD_W8>(out, cycles, blocks, iters, st);
        case FWD_PP: return (int)launch<FWD_PP>(out, cycles, blocks, iters, st);
        case FWD_2Q: return (int)launch<FWD_2Q>(out, cycles, blocks, iters, st);
        default: return (int)hipErrorInvalidValue;
    }
}

extern "C" int tca_mix_count(void) { return (int)mix::NUM_MIX; }

// Workgroups of mix `mix_id` that fit one CU at once (registers and LDS), i.e. the
// most waves per SIMD it can run at; -1 on error.
extern "C" int tca_mix_max_blocks_per_cu(int mix_id) {
    using namespace mix;
    int n = -1;
    hipError_t e = hipErrorInvalidValue;
    switch (mix_id) {
        case MFMA_ONLY: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, mix_kernel<MFMA_ONLY>, 256, 0); break;
        case EXP_ONLY: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, mix_kernel<EXP_ONLY>, 256, 0); break;
        case FMA_ONLY: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, mix_kernel<FMA_ONLY>, 256, 0); break;
        case CVT_ONLY: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, mix_kernel<CVT_ONLY>, 256, 0); break;
        case FWD: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, mix_kernel<FWD>, 256, 0); break;
        case FWD_REG: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, mix_kernel<FWD_REG>, 256, 0); break;
        case FWD_STAGED: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, mix_kernel<FWD_STAGED>, 256, 0); break;
        case DQ: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, mix_kernel<DQ>, 256, 0); break;
        case DKDV: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, mix_kernel<DKDV>, 256, 0); break;
        case FWD_W8: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, mix8_kernel<FWD_W8>, 512, 0); break;
        case FWD_PP: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, mix8_kernel<FWD_PP>, 512, 0); break;
        case FWD_2Q: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, mix_kernel<FWD_2Q>, 256, 0); break;
        default: break;
    }
    return e == hipSuccess ? n : -1;
}

// Matrix-core products per 32x32 block of each mix (0 for the VALU-only ones).
extern "C" int tca_mix_mfma_per_block(int mix_id) {
    static const int n[] = {8, 0, 0, 0, 8, 8, 8, 12, 16, 8, 8, 16};
    return (mix_id >= 0 && mix_id < (int)mix::NUM_MIX) ? n[mix_id] : -1;
}
