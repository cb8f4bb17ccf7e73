// attn_rope.hip -- rotary position embedding and strided q/k/v around the
// attention kernels.
//
// The blog page's FAQ lists RoPE among the trainer's techniques, and q, k, v
// come out of one fused projection, i.e. as views [B, N, H, d] of a single
// [B, N, (Hq + 2 Hkv) d] buffer. This file reads such strided tensors (any
// batch, head and row strides; the head dimension contiguous), rotates q and k
// (rotate-half pairing: (x_i, x_{i+d/2}) -> (x_i cos - x_{i+d/2} sin,
// x_{i+d/2} cos + x_i sin), cos/sin = table[n][i] for row position n), and
// writes contiguous [B, H, N, d] copies for the attention kernels. After the
// backward it turns dq and dk back with the transpose rotation
// ((g_i cos + g_{i+d/2} sin, g_{i+d/2} cos - g_i sin)) and scatters dq, dk, dv
// into the caller's layouts, rounding once to the output type.
//
// Each step is one HBM-bound pass (a thread per 8 pairs of a row, consecutive
// threads on consecutive pairs). On the matrix-core path the kernels take over all
// of it except the rotation of k: they read q and v through their strides, rotate
// q in registers and store dq, dk, dv through their strides (dq, dk turned back),
// and only k is rotated here, into a contiguous fp16 copy (the precision the
// kernels rotate q to), for the tiles of every query block to read.
#include "tca_internal.h"

namespace tca {

namespace rope {
constexpr int kThreads = 256;
}

// dst(b, h, n, :) = R(src(b, h, n, :)) with R the rotation at position n
// (rot = 1), its transpose (rot = 2) or the identity (rot = 0). A thread moves 8
// consecutive pairs (i, i + d/2) of one row, so a row takes d/16 threads (a power
// of two: the chunk index is a shift, the row index 32-bit). Up to three such
// copies (q, k, v staging, or the dq, dk, dv scatter) share one launch: thread
// idx belongs to the job whose [begin, begin + count) range holds it.
// 8 consecutive elements as float32: 16-byte vector loads when every row start is
// 16-byte aligned (VEC), else element loads; and the matching stores.
template <bool VEC>
__device__ __forceinline__ void load8(const bf16_t* p, float (&x)[8]) {
    if constexpr (VEC) {
        load8_f32(p, x);
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = bf16_to_f32(p[e]);
    }
}
template <bool VEC>
__device__ __forceinline__ void load8(const float* p, float (&x)[8]) {
    if constexpr (VEC) {
        load8_f32(p, x);
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = p[e];
    }
}
template <bool VEC>
__device__ __forceinline__ void store8(bf16_t* p, const float (&x)[8]) {
    if constexpr (VEC) {
        *reinterpret_cast<u32x4*>(p) = u32x4{pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]), pack_bf16(x[4], x[5]),
                                             pack_bf16(x[6], x[7])};
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) store_out1(p + e, x[e]);
    }
}
template <bool VEC>
__device__ __forceinline__ void store8(_Float16* p, const float (&x)[8]) {
    if constexpr (VEC) {
        *reinterpret_cast<u32x4*>(p) = u32x4{pack_f16(x[0], x[1]), pack_f16(x[2], x[3]), pack_f16(x[4], x[5]),
                                             pack_f16(x[6], x[7])};
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] = (_Float16)x[e];
    }
}
template <bool VEC>
__device__ __forceinline__ void store8(float* p, const float (&x)[8]) {
    if constexpr (VEC) {
        *reinterpret_cast<f32x4*>(p) = f32x4{x[0], x[1], x[2], x[3]};
        *reinterpret_cast<f32x4*>(p + 4) = f32x4{x[4], x[5], x[6], x[7]};
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] = x[e];
    }
}

template <typename TI, typename TO, bool VEC>
__global__ void __launch_bounds__(rope::kThreads)
layout_copy_kernel(CopyJobs jobs, const float* __restrict__ cs, const float* __restrict__ sn, int N, int d,
                   int chunk_shift, long long total) {
    const long long idx = (long long)blockIdx.x * rope::kThreads + threadIdx.x;
    if (idx >= total) return;
    const int jn = (jobs.n > 1 && idx >= jobs.j[1].begin) + (jobs.n > 2 && idx >= jobs.j[2].begin);
    // the thread's job selected by value: the descriptors stay in scalar registers
    // (an indexed access would first load them per lane from the argument block)
    const CopyJob J = jn == 0 ? jobs.j[0] : (jn == 1 ? jobs.j[1] : jobs.j[2]);
    const long long li = idx - J.begin;
    const int half = d / 2;
    const int i0 = 8 * (int)(li & ((1 << chunk_shift) - 1));
    const unsigned row = (unsigned)(li >> chunk_shift);   // (b, h, n); B*H*N < 2^31
    const unsigned n = row % (unsigned)N;
    const unsigned bh = row / (unsigned)N;
    const unsigned h = bh % (unsigned)J.H;
    const unsigned b = bh / (unsigned)J.H;
    const TI* s = static_cast<const TI*>(J.src) + b * J.sb + h * J.sh + (long long)n * J.sn + i0;
    TO* t = static_cast<TO*>(J.dst) + b * J.db + h * J.dh + (long long)n * J.dn + i0;
    // the row's table entries first (they depend on the position only), so their
    // loads and the data's are in flight together
    float cv[8], sv8[8];
    if (cs != nullptr) {
        const float* cp = cs + (long long)n * half + i0;
        const float* sp = sn + (long long)n * half + i0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            cv[e] = cp[e];
            sv8[e] = sp[e];
        }
    }
    float x1[8], x2[8];
    load8<VEC>(s, x1);
    load8<VEC>(s + half, x2);
    if (J.rot != 0) {
        const float sg = J.rot == 1 ? 1.f : -1.f;   // the transpose flips the sine
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float c = cv[e], sv = sg * sv8[e];
            const float a = x1[e], bb = x2[e];
            x1[e] = a * c - bb * sv;
            x2[e] = bb * c + a * sv;
        }
    }
    store8<VEC>(t, x1);
    store8<VEC>(t + half, x2);
}

template <typename TI, typename TO>
static hipError_t copy_t(CopyJobs jobs, const float* cs, const float* sn, int N, int d, hipStream_t st) {
    int shift = 0;
    while ((8 << shift) < d / 2) ++shift;   // d / 16 threads per row
    long long total = 0;
    for (int j = 0; j < jobs.n; ++j) {
        jobs.j[j].begin = total;
        total += jobs.j[j].count;
    }
    if (total == 0) return hipSuccess;
    // 16-byte vectors need every row start aligned: base pointers and strides in bytes
    bool vec = true;
    for (int j = 0; j < jobs.n; ++j) {
        const CopyJob& J = jobs.j[j];
        const long long ei = sizeof(TI), eo = sizeof(TO);
        vec = vec && ((uintptr_t)J.src % 16 == 0) && ((uintptr_t)J.dst % 16 == 0) && (J.sb * ei) % 16 == 0 &&
              (J.sh * ei) % 16 == 0 && (J.sn * ei) % 16 == 0 && (J.db * eo) % 16 == 0 && (J.dh * eo) % 16 == 0 &&
              (J.dn * eo) % 16 == 0;
    }
    const dim3 grid((unsigned)((total + rope::kThreads - 1) / rope::kThreads));
    if (vec)
        hipLaunchKernelGGL((layout_copy_kernel<TI, TO, true>), grid, dim3(rope::kThreads), 0, st, jobs, cs, sn, N, d,
                           shift, total);
    else
        hipLaunchKernelGGL((layout_copy_kernel<TI, TO, false>), grid, dim3(rope::kThreads), 0, st, jobs, cs, sn, N,
                           d, shift, total);
    return hipGetLastError();
}

hipError_t layout_copy(attn_dtype ti, attn_dtype to, const CopyJobs& jobs, const float* cs, const float* sn, int N,
                       int d, hipStream_t st) {
    if (ti == ATTN_F32)
        return to == ATTN_F32 ? copy_t<float, float>(jobs, cs, sn, N, d, st) : copy_t<float, bf16_t>(jobs, cs, sn, N, d, st);
    return to == ATTN_F32 ? copy_t<bf16_t, float>(jobs, cs, sn, N, d, st) : copy_t<bf16_t, bf16_t>(jobs, cs, sn, N, d, st);
}

hipError_t layout_copy_to_f16(const CopyJobs& jobs, const float* cs, const float* sn, int N, int d, hipStream_t st) {
    return copy_t<bf16_t, _Float16>(jobs, cs, sn, N, d, st);
}

CopyJob copy_job(const void* src, const attn_layout& sl, void* dst, const attn_layout& dl, int B, int H, int N, int d,
                 int rot) {
    CopyJob j;
    j.src = src;
    j.dst = dst;
    j.sb = sl.stride_b;
    j.sh = sl.stride_h;
    j.sn = sl.stride_n;
    j.db = dl.stride_b;
    j.dh = dl.stride_h;
    j.dn = dl.stride_n;
    j.H = H;
    j.rot = rot;
    j.count = (long long)B * H * N * (d / 16);   // one thread per 8 pairs of a row
    j.begin = 0;
    return j;
}

}  // namespace tca
