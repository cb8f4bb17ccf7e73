// attn_generic.hip -- float32-arithmetic attention kernels for any supported
// head dimension and input type.
//
// These kernels follow the tile loop of the NanoEuler "Tiled FlashAttention"
// section literally: one block per query tile, K/V tiles staged in LDS
// between barriers, and an online softmax per query row. A query row (forward,
// dQ) or key row (dK/dV) belongs to SPL consecutive lanes, each holding 32 of
// its head dimensions (SPL = d / 32 for d >= 64, else 1, so a lane never holds
// more than 32 dimensions of any row); dot products are completed across the
// SPL lanes by xor-shuffles, which give every lane of the row the bitwise same
// sum, so the lanes of a row take the same softmax decisions. Every reduction has
// a fixed order and the results are deterministic. They serve float32 inputs,
// where the accuracy target is float32, and bf16 inputs with small head
// dimensions.
#include "tca_internal.h"

namespace tca {

constexpr int kGenThreads = 64;   // one wave per block
constexpr int kGenTile = 32;      // K/V (or Q/dO) rows staged per LDS tile
template <int D> constexpr int kSpl = D >= 64 ? D / 32 : 1;           // lanes per row
template <int D> constexpr int kDp = D / kSpl<D>;                      // dimensions per lane
template <int D> constexpr int kGenRows = kGenThreads / kSpl<D>;       // rows per block

// Sum over the SPL lanes of a row (consecutive lanes); every lane gets the same bits.
template <int SPL>
__device__ __forceinline__ float row_sum(float x) {
    if constexpr (SPL >= 2) x += __shfl_xor(x, 1, 64);
    if constexpr (SPL >= 4) x += __shfl_xor(x, 2, 64);
    return x;
}

// T: input element type; OT: output element type of o, dq, dk, dv (float32,
// or bfloat16 rounded to nearest even when stored)
template <typename T, typename OT, int D>
__global__ void __launch_bounds__(kGenThreads)
fwd_generic_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                   OT* __restrict__ o, float* __restrict__ lse,
                   int Hq, int Hkv, int N, int causal, float scale) {
    constexpr int SPL = kSpl<D>, DP = kDp<D>, ROWS = kGenRows<D>;
    __shared__ float Ks[kGenTile][D];
    __shared__ float Vs[kGenTile][D];
    const int bh = blockIdx.y;
    const int b = bh / Hq, hq = bh % Hq, hkv = hq / (Hq / Hkv);
    const int part = threadIdx.x % SPL, c0 = part * DP;   // this lane's dimensions c0 .. c0 + DP - 1
    const int i = blockIdx.x * ROWS + threadIdx.x / SPL;
    const T* qh = q + (size_t)bh * N * D;
    const T* kh = k + ((size_t)b * Hkv + hkv) * N * D;
    const T* vh = v + ((size_t)b * Hkv + hkv) * N * D;

    float qr[DP], acc[DP];
    float m = -INFINITY, l = 0.f;
#pragma unroll
    for (int c = 0; c < DP; ++c) {
        qr[c] = (i < N) ? load_as_f32(qh + (size_t)i * D + c0 + c) : 0.f;
        acc[c] = 0.f;
    }
    const int last_row = min(N, (int)(blockIdx.x + 1) * ROWS) - 1;
    const int kend = causal ? last_row + 1 : N;
    for (int k0 = 0; k0 < kend; k0 += kGenTile) {
        for (int x = threadIdx.x; x < kGenTile * D; x += kGenThreads) {
            const int r = x / D, c = x % D;
            const bool ok = k0 + r < N;
            Ks[r][c] = ok ? load_as_f32(kh + (size_t)(k0 + r) * D + c) : 0.f;
            Vs[r][c] = ok ? load_as_f32(vh + (size_t)(k0 + r) * D + c) : 0.f;
        }
        __syncthreads();
        if (i < N) {
            for (int jj = 0; jj < kGenTile; ++jj) {
                const int j = k0 + jj;
                if (j >= N || (causal && j > i)) break;
                float dot = 0.f;
#pragma unroll
                for (int c = 0; c < DP; ++c) dot = fmaf(qr[c], Ks[jj][c0 + c], dot);
                const float s = scale * row_sum<SPL>(dot);
                if (s > m) {
                    const float alpha = expf(m - s);
                    l *= alpha;
#pragma unroll
                    for (int c = 0; c < DP; ++c) acc[c] *= alpha;
                    m = s;
                }
                const float p = expf(s - m);
                l += p;
#pragma unroll
                for (int c = 0; c < DP; ++c) acc[c] = fmaf(p, Vs[jj][c0 + c], acc[c]);
            }
        }
        __syncthreads();
    }
    if (i < N) {
        const float inv = 1.f / l;
        OT* oi = o + ((size_t)bh * N + i) * D + c0;
#pragma unroll
        for (int c = 0; c < DP; ++c) store_out1(oi + c, acc[c] * inv);
        if (part == 0) lse[(size_t)bh * N + i] = m + logf(l);
    }
}

// dK, dV for one KV head: one row of lanes per key, looping over every query head
// of the group and every visible query. No atomics: each key row is owned by one
// row of lanes.
template <typename T, typename OT, int D>
__global__ void __launch_bounds__(kGenThreads)
bwd_dkdv_generic_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                        const float* __restrict__ lse, const T* __restrict__ dout,
                        const float* __restrict__ delta,
                        OT* __restrict__ dk, OT* __restrict__ dv,
                        int Hq, int Hkv, int N, int causal, float scale) {
    constexpr int SPL = kSpl<D>, DP = kDp<D>, ROWS = kGenRows<D>;
    __shared__ float Qs[kGenTile][D];
    __shared__ float dOs[kGenTile][D];
    __shared__ float Ls[kGenTile], Ds[kGenTile];
    const int bkv = blockIdx.y;
    const int b = bkv / Hkv, hkv = bkv % Hkv, group = Hq / Hkv;
    const int part = threadIdx.x % SPL, c0 = part * DP;
    const int j = blockIdx.x * ROWS + threadIdx.x / SPL;
    const size_t kvoff = (size_t)bkv * N * D;

    float kr[DP], vr[DP], dkr[DP], dvr[DP];
#pragma unroll
    for (int c = 0; c < DP; ++c) {
        kr[c] = (j < N) ? load_as_f32(k + kvoff + (size_t)j * D + c0 + c) : 0.f;
        vr[c] = (j < N) ? load_as_f32(v + kvoff + (size_t)j * D + c0 + c) : 0.f;
        dkr[c] = 0.f;
        dvr[c] = 0.f;
    }
    const int first_key = blockIdx.x * ROWS;
    const int qstart = causal ? (first_key / kGenTile) * kGenTile : 0;
    for (int g = 0; g < group; ++g) {
        const int hq = hkv * group + g;
        const size_t qrow0 = ((size_t)b * Hq + hq) * N;
        for (int i0 = qstart; i0 < N; i0 += kGenTile) {
            for (int x = threadIdx.x; x < kGenTile * D; x += kGenThreads) {
                const int r = x / D, c = x % D;
                const bool ok = i0 + r < N;
                Qs[r][c] = ok ? load_as_f32(q + (qrow0 + i0 + r) * D + c) : 0.f;
                dOs[r][c] = ok ? load_as_f32(dout + (qrow0 + i0 + r) * D + c) : 0.f;
            }
            for (int r = threadIdx.x; r < kGenTile; r += kGenThreads) {
                const bool ok = i0 + r < N;
                Ls[r] = ok ? lse[qrow0 + i0 + r] : 0.f;
                Ds[r] = ok ? delta[qrow0 + i0 + r] : 0.f;
            }
            __syncthreads();
            if (j < N) {
                for (int ii = 0; ii < kGenTile; ++ii) {
                    const int i = i0 + ii;
                    if (i >= N) break;
                    if (causal && j > i) continue;
                    float s = 0.f, dp = 0.f;
#pragma unroll
                    for (int c = 0; c < DP; ++c) {
                        s = fmaf(Qs[ii][c0 + c], kr[c], s);
                        dp = fmaf(dOs[ii][c0 + c], vr[c], dp);
                    }
                    s = row_sum<SPL>(s);
                    dp = row_sum<SPL>(dp);
                    const float p = expf(scale * s - Ls[ii]);
                    const float ds = p * (dp - Ds[ii]);
#pragma unroll
                    for (int c = 0; c < DP; ++c) {
                        dvr[c] = fmaf(p, dOs[ii][c0 + c], dvr[c]);
                        dkr[c] = fmaf(ds, Qs[ii][c0 + c], dkr[c]);
                    }
                }
            }
            __syncthreads();
        }
    }
    if (j < N) {
        OT* dkj = dk + kvoff + (size_t)j * D + c0;
        OT* dvj = dv + kvoff + (size_t)j * D + c0;
#pragma unroll
        for (int c = 0; c < DP; ++c) {
            store_out1(dkj + c, scale * dkr[c]);
            store_out1(dvj + c, dvr[c]);
        }
    }
}

// dQ: one row of lanes per query row, looping over the visible keys. The row
// first forms D_i = <dO_i, O_i> and publishes it (the dK/dV kernel reads it).
template <typename T, typename OT, int D>
__global__ void __launch_bounds__(kGenThreads)
bwd_dq_generic_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                      const OT* __restrict__ o, const float* __restrict__ lse,
                      const T* __restrict__ dout, float* __restrict__ delta, OT* __restrict__ dq,
                      int Hq, int Hkv, int N, int causal, float scale) {
    constexpr int SPL = kSpl<D>, DP = kDp<D>, ROWS = kGenRows<D>;
    __shared__ float Ks[kGenTile][D];
    __shared__ float Vs[kGenTile][D];
    const int bh = blockIdx.y;
    const int b = bh / Hq, hq = bh % Hq, hkv = hq / (Hq / Hkv);
    const int part = threadIdx.x % SPL, c0 = part * DP;
    const int i = blockIdx.x * ROWS + threadIdx.x / SPL;
    const size_t qrow = (size_t)bh * N + i;
    const T* kh = k + ((size_t)b * Hkv + hkv) * N * D;
    const T* vh = v + ((size_t)b * Hkv + hkv) * N * D;

    float qr[DP], dor[DP], dqr[DP];
#pragma unroll
    for (int c = 0; c < DP; ++c) {
        qr[c] = (i < N) ? load_as_f32(q + qrow * D + c0 + c) : 0.f;
        dor[c] = (i < N) ? load_as_f32(dout + qrow * D + c0 + c) : 0.f;
        dqr[c] = 0.f;
    }
    const float L = (i < N) ? lse[qrow] : 0.f;
    float Di = 0.f;
    if (i < N) {
#pragma unroll
        for (int c = 0; c < DP; ++c) Di = fmaf(dor[c], load_as_f32(o + qrow * D + c0 + c), Di);
        Di = row_sum<SPL>(Di);
        if (part == 0) delta[qrow] = Di;
    }
    const int last_row = min(N, (int)(blockIdx.x + 1) * ROWS) - 1;
    const int kend = causal ? last_row + 1 : N;
    for (int k0 = 0; k0 < kend; k0 += kGenTile) {
        for (int x = threadIdx.x; x < kGenTile * D; x += kGenThreads) {
            const int r = x / D, c = x % D;
            const bool ok = k0 + r < N;
            Ks[r][c] = ok ? load_as_f32(kh + (size_t)(k0 + r) * D + c) : 0.f;
            Vs[r][c] = ok ? load_as_f32(vh + (size_t)(k0 + r) * D + c) : 0.f;
        }
        __syncthreads();
        if (i < N) {
            for (int jj = 0; jj < kGenTile; ++jj) {
                const int j = k0 + jj;
                if (j >= N || (causal && j > i)) break;
                float s = 0.f, dp = 0.f;
#pragma unroll
                for (int c = 0; c < DP; ++c) {
                    s = fmaf(qr[c], Ks[jj][c0 + c], s);
                    dp = fmaf(dor[c], Vs[jj][c0 + c], dp);
                }
                s = row_sum<SPL>(s);
                dp = row_sum<SPL>(dp);
                const float p = expf(scale * s - L);
                const float ds = p * (dp - Di);
#pragma unroll
                for (int c = 0; c < DP; ++c) dqr[c] = fmaf(ds, Ks[jj][c0 + c], dqr[c]);
            }
        }
        __syncthreads();
    }
    if (i < N) {
#pragma unroll
        for (int c = 0; c < DP; ++c) store_out1(dq + qrow * D + c0 + c, scale * dqr[c]);
    }
}

// ---------------------------------------------------------------- launchers
template <typename T, typename OT, int D>
static hipError_t launch_fwd_generic_t(const AttnArgs& a, hipStream_t st) {
    dim3 grid((a.N + kGenRows<D> - 1) / kGenRows<D>, a.B * a.Hq);
    hipLaunchKernelGGL((fwd_generic_kernel<T, OT, D>), grid, dim3(kGenThreads), 0, st,
                       (const T*)a.q, (const T*)a.k, (const T*)a.v, (OT*)a.o, a.lse,
                       a.Hq, a.Hkv, a.N, a.causal, a.scale);
    return hipGetLastError();
}

template <typename T, typename OT, int D>
static hipError_t launch_bwd_generic_dq_t(const AttnArgs& a, hipStream_t st) {
    dim3 gq((a.N + kGenRows<D> - 1) / kGenRows<D>, a.B * a.Hq);
    hipLaunchKernelGGL((bwd_dq_generic_kernel<T, OT, D>), gq, dim3(kGenThreads), 0, st,
                       (const T*)a.q, (const T*)a.k, (const T*)a.v, (const OT*)a.o,
                       (const float*)a.lse, (const T*)a.dout, (float*)a.workspace, (OT*)a.dq,
                       a.Hq, a.Hkv, a.N, a.causal, a.scale);
    return hipGetLastError();
}

template <typename T, typename OT, int D>
static hipError_t launch_bwd_generic_dkdv_t(const AttnArgs& a, hipStream_t st) {
    dim3 gkv((a.N + kGenRows<D> - 1) / kGenRows<D>, a.B * a.Hkv);
    hipLaunchKernelGGL((bwd_dkdv_generic_kernel<T, OT, D>), gkv, dim3(kGenThreads), 0, st,
                       (const T*)a.q, (const T*)a.k, (const T*)a.v, (const float*)a.lse,
                       (const T*)a.dout, (const float*)a.workspace, (OT*)a.dk, (OT*)a.dv,
                       a.Hq, a.Hkv, a.N, a.causal, a.scale);
    return hipGetLastError();
}

// (input type, output type, head dimension) -> one instantiation
#define TCA_DISPATCH(A_, ST_, LAUNCH)                                                        \
    do {                                                                                     \
        const bool in32 = (A_).dtype == ATTN_F32, out32 = (A_).out_dtype == ATTN_F32;         \
        switch ((A_).d) {                                                                    \
            case 16:                                                                         \
                return in32 ? (out32 ? LAUNCH<float, float, 16>(A_, ST_) : LAUNCH<float, bf16_t, 16>(A_, ST_))   \
                            : (out32 ? LAUNCH<bf16_t, float, 16>(A_, ST_) : LAUNCH<bf16_t, bf16_t, 16>(A_, ST_)); \
            case 32:                                                                         \
                return in32 ? (out32 ? LAUNCH<float, float, 32>(A_, ST_) : LAUNCH<float, bf16_t, 32>(A_, ST_))   \
                            : (out32 ? LAUNCH<bf16_t, float, 32>(A_, ST_) : LAUNCH<bf16_t, bf16_t, 32>(A_, ST_)); \
            case 64:                                                                         \
                return in32 ? (out32 ? LAUNCH<float, float, 64>(A_, ST_) : LAUNCH<float, bf16_t, 64>(A_, ST_))   \
                            : (out32 ? LAUNCH<bf16_t, float, 64>(A_, ST_) : LAUNCH<bf16_t, bf16_t, 64>(A_, ST_)); \
            case 128:                                                                        \
                return in32 ? (out32 ? LAUNCH<float, float, 128>(A_, ST_) : LAUNCH<float, bf16_t, 128>(A_, ST_)) \
                            : (out32 ? LAUNCH<bf16_t, float, 128>(A_, ST_) : LAUNCH<bf16_t, bf16_t, 128>(A_, ST_)); \
            default: return hipErrorInvalidValue;                                            \
        }                                                                                    \
    } while (0)

hipError_t launch_fwd_generic(const AttnArgs& a, hipStream_t st) { TCA_DISPATCH(a, st, launch_fwd_generic_t); }
hipError_t launch_bwd_generic_dq(const AttnArgs& a, hipStream_t st) { TCA_DISPATCH(a, st, launch_bwd_generic_dq_t); }
hipError_t launch_bwd_generic_dkdv(const AttnArgs& a, hipStream_t st) { TCA_DISPATCH(a, st, launch_bwd_generic_dkdv_t); }

}  // namespace tca
