// mfma_peak.hip -- measured dense matrix-core throughput of this GPU, for the
// benchmark report (not part of the attention library): every wave issues
// independent v_mfma_f32_32x32x16_bf16 back to back, with operands in
// registers and no memory traffic in the loop, so the rate is what the
// matrix cores sustain at the clock they run under load.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kChains = 4;   // independent accumulators per wave

__global__ void __launch_bounds__(256) mfma_peak_kernel(float* __restrict__ out, int iters) {
    const int tid = blockIdx.x * blockDim.x + threadIdx.x;
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(float)((tid + i) & 7);
        b[i] = (__bf16)(float)((tid * 3 + i) & 5);
    }
    f32x16 c[kChains];
#pragma unroll
    for (int j = 0; j < kChains; ++j) c[j] = f32x16{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < kChains; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[j], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < kChains; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += c[j][e];
    out[tid] = s;
}

// Launch `blocks` workgroups of 256 threads, each wave running iters x 4
// MFMAs (32x32x16: 32768 flops each). `out` holds blocks * 256 floats (device
// memory, written). Returns 0 or the HIP error code of the launch.
extern "C" int tca_mfma_peak_launch(float* out, int blocks, int iters, void* stream) {
    if (out == nullptr || blocks < 1 || iters < 1) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(mfma_peak_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, out, iters);
    return (int)hipGetLastError();
}

// Floating-point operations one launch performs.
extern "C" double tca_mfma_peak_flops(int blocks, int iters) {
    return (double)blocks * 4 /* waves */ * iters * kChains * 32.0 * 32.0 * 16.0 * 2.0;
}
