// attn_naive.hip -- the unoptimised, materialised-score forward.
//
// The NanoEuler article lists a "naive", unoptimised version kept for teaching,
// next to the tiled FlashAttention. This is that baseline on the GPU: the same
// definition computed the obvious way, with the whole score matrix S in device
// memory, so the tiled kernels can be compared against it:
//   1. S[b,hq,i,j] = scale <q_i, k_j>, -inf where key j is masked (one thread per score)
//   2. row softmax in place: P = exp(S - max) / sum, LSE = max + log(sum) (one wave per row)
//   3. O[b,hq,i,:] = sum_j P[b,hq,i,j] v_j (one thread per output element)
// Every read goes straight to global memory; nothing is tiled or staged. S takes
// B*Hq*N*N floats of the caller's workspace.
#include "tca_internal.h"

namespace tca {

namespace naive {
constexpr int kThreads = 256;
}

template <typename T>
__global__ void __launch_bounds__(naive::kThreads)
naive_scores_kernel(const T* __restrict__ q, const T* __restrict__ k, float* __restrict__ S, int Hq, int Hkv,
                    int N, int d, int causal, float scale, long long total) {
    const long long idx = (long long)blockIdx.x * naive::kThreads + threadIdx.x;
    if (idx >= total) return;
    const int j = (int)(idx % N);
    const long long rest = idx / N;
    const int i = (int)(rest % N);
    const long long bh = rest / N;
    const int b = (int)(bh / Hq), hq = (int)(bh % Hq), hkv = hq / (Hq / Hkv);
    float s = -INFINITY;
    if (!causal || j <= i) {
        const T* qi = q + (bh * N + i) * d;
        const T* kj = k + (((long long)b * Hkv + hkv) * N + j) * d;
        float dot = 0.f;
        for (int c = 0; c < d; ++c) dot = fmaf(load_as_f32(qi + c), load_as_f32(kj + c), dot);
        s = scale * dot;
    }
    S[idx] = s;
}

// One wave per row of S (rows = B * Hq * N): maximum, sum of exponentials, then
// the probabilities in place and the row's LSE (natural log).
__global__ void __launch_bounds__(64)
naive_softmax_kernel(float* __restrict__ S, float* __restrict__ lse, int N) {
    const long long row = blockIdx.x;
    float* r = S + row * N;
    float m = -INFINITY;
    for (int j = threadIdx.x; j < N; j += 64) m = fmaxf(m, r[j]);
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    float l = 0.f;
    for (int j = threadIdx.x; j < N; j += 64) l += expf(r[j] - m);
    for (int off = 32; off > 0; off >>= 1) l += __shfl_xor(l, off, 64);
    const float inv = 1.f / l;
    for (int j = threadIdx.x; j < N; j += 64) r[j] = expf(r[j] - m) * inv;
    if (threadIdx.x == 0) lse[row] = m + logf(l);
}

template <typename T, typename OT>
__global__ void __launch_bounds__(naive::kThreads)
naive_pv_kernel(const float* __restrict__ P, const T* __restrict__ v, OT* __restrict__ o, int Hq, int Hkv, int N,
                int d, long long total) {
    const long long idx = (long long)blockIdx.x * naive::kThreads + threadIdx.x;
    if (idx >= total) return;
    const int c = (int)(idx % d);
    const long long row = idx / d;          // (b, hq, i)
    const long long bh = row / N;
    const int b = (int)(bh / Hq), hq = (int)(bh % Hq), hkv = hq / (Hq / Hkv);
    const float* p = P + row * N;
    const T* vh = v + ((long long)b * Hkv + hkv) * N * d + c;
    float acc = 0.f;
    for (int j = 0; j < N; ++j) acc = fmaf(p[j], load_as_f32(vh + (long long)j * d), acc);
    store_out1(o + idx, acc);
}

size_t naive_workspace_size(int B, int Hq, int N) { return (size_t)B * Hq * N * N * sizeof(float); }

template <typename T, typename OT>
static hipError_t launch_naive_t(const AttnArgs& a, hipStream_t st) {
    float* S = static_cast<float*>(a.workspace);
    const long long rows = (long long)a.B * a.Hq * a.N;
    const long long scores = rows * a.N;
    const long long outs = rows * a.d;
    hipLaunchKernelGGL((naive_scores_kernel<T>), dim3((unsigned)((scores + naive::kThreads - 1) / naive::kThreads)),
                       dim3(naive::kThreads), 0, st, (const T*)a.q, (const T*)a.k, S, a.Hq, a.Hkv, a.N, a.d,
                       a.causal, a.scale, scores);
    hipLaunchKernelGGL(naive_softmax_kernel, dim3((unsigned)rows), dim3(64), 0, st, S, a.lse, a.N);
    hipLaunchKernelGGL((naive_pv_kernel<T, OT>), dim3((unsigned)((outs + naive::kThreads - 1) / naive::kThreads)),
                       dim3(naive::kThreads), 0, st, (const float*)S, (const T*)a.v, (OT*)a.o, a.Hq, a.Hkv, a.N,
                       a.d, outs);
    return hipGetLastError();
}

hipError_t launch_fwd_naive(const AttnArgs& a, hipStream_t st) {
    const bool in32 = a.dtype == ATTN_F32, out32 = a.out_dtype == ATTN_F32;
    if (in32) return out32 ? launch_naive_t<float, float>(a, st) : launch_naive_t<float, bf16_t>(a, st);
    return out32 ? launch_naive_t<bf16_t, float>(a, st) : launch_naive_t<bf16_t, bf16_t>(a, st);
}

}  // namespace tca
