// Device-side helpers: bf16 storage conversion, activation functions and
// vector types for gfx950.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tps {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

#define TPS_LDS __attribute__((address_space(3)))

__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// fp32 -> bf16 with gfx950's v_cvt_pk_bf16_f32 (round to nearest even; a NaN
// stays a quiet NaN), two values per instruction.
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

__device__ __forceinline__ uint16_t f2bf(float f) { return (uint16_t)(pack_bf2(f, 0.f) & 0xffffu); }

// Exact GeLU: x * Phi(x), Phi(x) = (1 + erf(x / sqrt 2)) / 2.
__device__ __forceinline__ float gelu_f(float x) { return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f)); }

// d/dx GeLU = Phi(x) + x * phi(x), phi(x) = exp(-x^2/2) / sqrt(2 pi).
__device__ __forceinline__ float gelu_grad_f(float x) {
  float cdf = 0.5f * (1.0f + erff(x * 0.70710678118654752f));
  float pdf = 0.39894228040143268f * __expf(-0.5f * x * x);
  return cdf + x * pdf;
}

// Logistic function; the reciprocal is gfx950's v_rcp_f32 (1 ulp) rather than
// an IEEE division (a ten-instruction sequence per element).  Large |x| gives
// exactly 0 or 1.
__device__ __forceinline__ float sigmoid_f(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

__device__ __forceinline__ float silu_f(float x) { return x * sigmoid_f(x); }

}  // namespace tps
