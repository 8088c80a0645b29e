// MFMA-only calibration kernel (libtpcalib, declared in include/tpcalib.h):
// the bf16 matrix-core rate the GPU sustains with operands held in registers,
// no memory or LDS traffic in the loop.  Run with random operands it shows
// the power-limited ceiling of any bf16 GEMM on the same data; with zero
// operands, the clock the chip keeps when the matrix cores barely toggle.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tpcalib.h"

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;

__global__ __launch_bounds__(256, 1) void mfma_loop_kernel(const bf16x8* __restrict__ src, float* __restrict__ out,
                                                           int iters) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const bf16x8* s = src + (wave & 3) * 1024;   // 16 KiB per wave slot: 16 fragments x 64 lanes x 16 B
  bf16x8 a[2][4], b[2][4];
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[q][i] = s[(8 * q + i) * 64 + lane];
      b[q][i] = s[(8 * q + 4 + i) * 64 + lane];
    }
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[q][j], a[q][i], acc[i][j], 0, 0, 0);
  }
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) sum += acc[i][j][r];
  out[blockIdx.x * 256 + threadIdx.x] = sum;
}

// The same loop on v_mfma_f32_16x16x32_bf16 (half the FLOPs per instruction):
// 32 accumulator blocks of 16 x 16 (4 x 8), 24 operand fragments, 64
// instructions per iteration (the same FLOPs per iteration as above).
__global__ __launch_bounds__(256, 1) void mfma16_loop_kernel(const bf16x8* __restrict__ src, float* __restrict__ out,
                                                             int iters) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const bf16x8* s = src + (wave & 3) * 1536;   // 24 fragments x 64 lanes x 16 B per wave slot
  bf16x8 a[2][4], b[2][8];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
#pragma unroll
    for (int i = 0; i < 4; ++i) a[q][i] = s[(12 * q + i) * 64 + lane];
#pragma unroll
    for (int j = 0; j < 8; ++j) b[q][j] = s[(12 * q + 4 + j) * 64 + lane];
  }
  f32x4 acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          // written as one instruction with the accumulator pinned to the
          // accumulator registers (the builtin's register allocation
          // shuffles accumulators between register files every iteration)
          asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc[i][j]) : "v"(b[q][j]), "v"(a[q][i]));
  }
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) sum += acc[i][j][r];
  out[blockIdx.x * 256 + threadIdx.x] = sum;
}

}  // namespace

// Shader clock probe: one wave per workgroup reads the shader cycle counter
// (s_memtime) and the 100 MHz real-time counter (s_memrealtime), runs `spin`
// dependent integer steps, and reads both again; lane 0 writes the two
// differences.  The ratio times 100 MHz is the clock the wave ran at.
__global__ __launch_bounds__(64) void clock_probe_kernel(unsigned long long* out, int spin) {
  const unsigned long long c0 = __builtin_readcyclecounter();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  unsigned x = threadIdx.x;
  for (int i = 0; i < spin; ++i) {
    x = x * 3u + 1u;
    asm volatile("" : "+v"(x));
  }
  const unsigned long long c1 = __builtin_readcyclecounter();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  asm volatile("" ::"v"(x));
  if (threadIdx.x == 0) {
    out[2 * blockIdx.x] = c1 - c0;
    out[2 * blockIdx.x + 1] = r1 - r0;
  }
}

extern "C" int tpc_clock_probe(unsigned long long* out, int blocks, int spin, void* stream) {
  if (!out || blocks < 1 || spin < 1) return -1;
  hipLaunchKernelGGL(clock_probe_kernel, dim3(blocks), dim3(64), 0, static_cast<hipStream_t>(stream), out, spin);
  return (int)hipGetLastError();
}

extern "C" int tpc_mfma_loop(const void* src, float* out, int cus, int iters, int shape, void* stream) {
  if (!src || !out || iters < 1 || cus < 1 || (shape != 32 && shape != 16)) return -1;
  if (shape == 32)
    hipLaunchKernelGGL(mfma_loop_kernel, dim3(cus), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const bf16x8*>(src), out, iters);
  else
    hipLaunchKernelGGL(mfma16_loop_kernel, dim3(cus), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const bf16x8*>(src), out, iters);
  return (int)hipGetLastError();
}
