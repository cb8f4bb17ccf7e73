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
// Each step is one HBM-bound pass (a thread per (row, pair i < d/2): two
// elements read, two written, consecutive threads on consecutive i).
#include "tca_internal.h"

namespace tca {

namespace rope {
constexpr int kThreads = 256;
}

// dst(b, h, n, :) = R(src(b, h, n, :)) with R the rotation at position n
// (rot = 1), its transpose (rot = 2) or the identity (rot = 0).
template <typename TI, typename TO>
__global__ void __launch_bounds__(rope::kThreads)
layout_copy_kernel(const TI* __restrict__ src, TO* __restrict__ dst, const float* __restrict__ cs,
                   const float* __restrict__ sn, long long s_b, long long s_h, long long s_n, long long d_b,
                   long long d_h, long long d_n, int H, int N, int d, int rot, long long total) {
    const long long idx = (long long)blockIdx.x * rope::kThreads + threadIdx.x;
    if (idx >= total) return;
    const int half = d / 2;
    const int i = (int)(idx % half);
    const long long row = idx / half;     // (b, h, n)
    const int n = (int)(row % N);
    const long long bh = row / N;
    const int h = (int)(bh % H);
    const long long b = bh / H;
    const TI* s = src + b * s_b + h * s_h + (long long)n * s_n;
    TO* t = dst + b * d_b + h * d_h + (long long)n * d_n;
    const float x1 = load_as_f32(s + i), x2 = load_as_f32(s + i + half);
    float y1 = x1, y2 = x2;
    if (rot != 0) {
        const float c = cs[(long long)n * half + i], sv = sn[(long long)n * half + i];
        if (rot == 1) {
            y1 = x1 * c - x2 * sv;
            y2 = x2 * c + x1 * sv;
        } else {
            y1 = x1 * c + x2 * sv;
            y2 = x2 * c - x1 * sv;
        }
    }
    store_out1(t + i, y1);
    store_out1(t + i + half, y2);
}

template <typename TI, typename TO>
static hipError_t copy_t(const void* src, const attn_layout& sl, void* dst, const attn_layout& dl, const float* cs,
                         const float* sn, int B, int H, int N, int d, int rot, hipStream_t st) {
    const long long total = (long long)B * H * N * (d / 2);
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL((layout_copy_kernel<TI, TO>), dim3((unsigned)((total + rope::kThreads - 1) / rope::kThreads)),
                       dim3(rope::kThreads), 0, st, (const TI*)src, (TO*)dst, cs, sn, sl.stride_b, sl.stride_h,
                       sl.stride_n, dl.stride_b, dl.stride_h, dl.stride_n, H, N, d, rot, total);
    return hipGetLastError();
}

hipError_t layout_copy(attn_dtype ti, const void* src, const attn_layout& sl, attn_dtype to, void* dst,
                       const attn_layout& dl, const float* cs, const float* sn, int B, int H, int N, int d, int rot,
                       hipStream_t st) {
    if (ti == ATTN_F32)
        return to == ATTN_F32 ? copy_t<float, float>(src, sl, dst, dl, cs, sn, B, H, N, d, rot, st)
                              : copy_t<float, bf16_t>(src, sl, dst, dl, cs, sn, B, H, N, d, rot, st);
    return to == ATTN_F32 ? copy_t<bf16_t, float>(src, sl, dst, dl, cs, sn, B, H, N, d, rot, st)
                          : copy_t<bf16_t, bf16_t>(src, sl, dst, dl, cs, sn, B, H, N, d, rot, st);
}

}  // namespace tca
