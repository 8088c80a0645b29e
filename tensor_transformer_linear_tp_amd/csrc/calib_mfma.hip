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

// LDS read-rate probe: one workgroup of `waves` wave64s per CU reads its 64 KiB LDS array in
// one access pattern, 8 reads in flight per wave, the address moving every iteration (so that
// no read can be reused); lane 0 of the workgroup records the shader cycles of the read loop
// and every thread writes a checksum.
//   kind 0: ds_read_b128, lanes on 1 KiB of consecutive bytes (one pass of all banks per
//           16 lanes);
//   kind 1: ds_read_b64_tr_b16, lanes on 512 consecutive bytes;
//   kind 2: ds_read_b64_tr_b16 in the column-fragment pattern of a 256-byte-row tile whose
//           16-byte chunk c of row r sits at c ^ (4 (r % 4) + (r / 4) % 4) (the attention
//           kernels' tiles read both ways), 32 columns x 16 rows per read pair.
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
__global__ __launch_bounds__(1024) void lds_rate_kernel(unsigned* out, unsigned long long* cycles, int iters,
                                                        int kind) {
  __shared__ __attribute__((aligned(16))) char lds[65536];
  for (int i = threadIdx.x; i < 65536 / 4; i += blockDim.x) reinterpret_cast<unsigned*>(lds)[i] = i;
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int base = (wave * 8192) & 65535;
  unsigned acc = 0;
  const unsigned long long t0 = __builtin_readcyclecounter();
  for (int it = 0; it < iters; ++it) {
    const int mv = (it * 64) & 4095;
    if (kind == 0) {
      u32x4 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        v[j] = *reinterpret_cast<const u32x4*>(lds + ((base + j * 1024 + lane * 16 + mv) & 65535));
#pragma unroll
      for (int j = 0; j < 8; ++j) acc += v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
    } else {
      i16x4 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        int off;
        if (kind == 1) {
          off = j * 512 + lane * 8;
        } else {
          const int h = lane >> 4, q = lane & 15;
          const int col = 32 * (j & 3) + 16 * (h & 1) + 4 * (q & 3);
          const int r = 16 * (j >> 2) + 8 * (h >> 1) + (q >> 2) + 4 * (it & 1);
          off = r * 256 + (((col >> 3) ^ (((r & 3) << 2) | ((r >> 2) & 3))) << 4) + (col & 7) * 2;
        }
        v[j] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(lds + ((base + off + mv) & 65535)));
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) acc += (unsigned)(v[j].x ^ v[j].y ^ v[j].z ^ v[j].w);
    }
  }
  __syncthreads();
  const unsigned long long t1 = __builtin_readcyclecounter();
  out[blockIdx.x * blockDim.x + threadIdx.x] = acc;
  if (threadIdx.x == 0) cycles[blockIdx.x] = t1 - t0;
}

extern "C" int tpc_lds_read_rate(unsigned* out, unsigned long long* cycles, int cus, int waves, int iters, int kind,
                                 void* stream) {
  if (!out || !cycles || cus < 1 || waves < 1 || waves > 16 || iters < 1 || kind < 0 || kind > 2) return -1;
  hipLaunchKernelGGL(lds_rate_kernel, dim3(cus), dim3(64 * waves), 0, static_cast<hipStream_t>(stream), out, cycles,
                     iters, kind);
  return (int)hipGetLastError();
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
