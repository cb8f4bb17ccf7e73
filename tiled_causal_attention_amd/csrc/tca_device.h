// tca_device.h -- shared device helpers for the gfx950 attention kernels:
// vector types, matrix-core wrappers, conversions and lane exchanges.
//
// Matrix-core layouts used throughout (v_mfma_f32_32x32x16_{bf16,f16}, one
// wave of 64 lanes; lane = 32*h + r with h in {0,1}, r in [0,32)):
//   A (32 x 16): lane holds A[m = r][k = 8h .. 8h+7]      (8 packed 16-bit values)
//   B (16 x 32): lane holds B[k = 8h .. 8h+7][n = r]
//   C (32 x 32): lane holds C[m = 8(e/4) + 4h + e%4][n = r] in accumulator e = 0..15
// so a product's output column index n is fixed per lane and can feed the next
// product as its B operand (n stays the lane) or as its A operand transposed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tca {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t bf16_t;   // raw bfloat16 bits in memory

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_f16(f16x8 a, f16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// bfloat16 bits -> float32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(bf16_t x) { return __uint_as_float((uint32_t)x << 16); }

// Two float32 -> packed fp16 pair, round to nearest even (v_cvt_pk_f16_f32).
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
    f16x2 h = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, h);
}

// Eight float32 accumulator values -> one fp16 operand.
__device__ __forceinline__ f16x8 to_f16x8(float a0, float a1, float a2, float a3,
                                          float a4, float a5, float a6, float a7) {
    f16x8 r = {(_Float16)a0, (_Float16)a1, (_Float16)a2, (_Float16)a3,
               (_Float16)a4, (_Float16)a5, (_Float16)a6, (_Float16)a7};
    return r;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Value held by lane (lane ^ 32): the other half of the wave.
__device__ __forceinline__ float swap_halves(float x) { return __shfl_xor(x, 32, 64); }

// Row permutation that makes a 32x32 accumulator feed the next product's
// 16-deep operand in natural order: swaps bits 2 and 3 of the row index.
// If the A operand's row m is loaded from source row perm32(m), accumulator
// e of lane (h, r) holds source row 16(e/8) + 8h + (e%8).
__device__ __forceinline__ int perm32(int m) {
    return (m & ~0xC) | ((m & 4) << 1) | ((m & 8) >> 1);
}

template <typename T>
__device__ __forceinline__ float load_as_f32(const T* p);
template <>
__device__ __forceinline__ float load_as_f32<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float load_as_f32<bf16_t>(const bf16_t* p) { return bf16_to_f32(*p); }

}  // namespace tca
