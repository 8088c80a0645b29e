// HBM-bound kernels of the shard path: the column-epilogue backward (dP from
// dY and the saved pre-activation, fused with fp32 column partial sums for the
// bias gradients), the ordered reduction of those partials, and the t-way sum
// of shard partials.  Each thread moves 8 consecutive columns with 16-byte
// accesses when the row segment is whole and aligned.
#include <algorithm>

#include "device_common.hpp"
#include "kernels.hpp"

namespace tps {
namespace {

template <typename T>
__device__ __forceinline__ void load8(const T* p, int nv, float (&v)[8]);
template <typename T>
__device__ __forceinline__ void store8(T* p, int nv, const float (&v)[8]);

template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, int nv, float (&v)[8]) {
  if (nv == 8 && (reinterpret_cast<uintptr_t>(p) & 15) == 0) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = __uint_as_float(w[e] << 16);
      v[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = e < nv ? bf2f(p[e]) : 0.f;
  }
}

template <>
__device__ __forceinline__ void store8<uint16_t>(uint16_t* p, int nv, const float (&v)[8]) {
  if (nv == 8 && (reinterpret_cast<uintptr_t>(p) & 15) == 0) {
    *reinterpret_cast<u32x4*>(p) =
        u32x4{pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]), pack_bf2(v[4], v[5]), pack_bf2(v[6], v[7])};
  } else {
    for (int e = 0; e < nv; ++e) p[e] = f2bf(v[e]);
  }
}

template <>
__device__ __forceinline__ void load8<float>(const float* p, int nv, float (&v)[8]) {
  if (nv == 8 && (reinterpret_cast<uintptr_t>(p) & 15) == 0) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = a[e];
      v[4 + e] = b[e];
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = e < nv ? p[e] : 0.f;
  }
}

template <>
__device__ __forceinline__ void store8<float>(float* p, int nv, const float (&v)[8]) {
  if (nv == 8 && (reinterpret_cast<uintptr_t>(p) & 15) == 0) {
    *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4*>(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
  } else {
    for (int e = 0; e < nv; ++e) p[e] = v[e];
  }
}

template <typename T>
__device__ __forceinline__ T from_f(float x);
template <>
__device__ __forceinline__ uint16_t from_f<uint16_t>(float x) { return f2bf(x); }
template <>
__device__ __forceinline__ float from_f<float>(float x) { return x; }

template <typename T>
__device__ __forceinline__ float to_f(T x);
template <>
__device__ __forceinline__ float to_f<uint16_t>(uint16_t x) { return bf2f(x); }
template <>
__device__ __forceinline__ float to_f<float>(float x) { return x; }

// Block (x = row block, y = column block): 32 column-threads x 8 row-threads
// over [64 rows] x [256 columns].
template <typename T>
__global__ __launch_bounds__(256) void act_bwd_kernel(const ActBwdArgs a) {
  __shared__ float red[8][2][256];
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  const int64_t n = (int64_t)blockIdx.y * 256 + 8 * tx;
  const int64_t rb = blockIdx.x;
  const bool swiglu = a.act == E_SWIGLU;
  float cg[8], cu[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) cg[e] = cu[e] = 0.f;
  if (n < a.N) {
    const int nv = (int)min<int64_t>(8, a.N - n);
    const T* dY = static_cast<const T*>(a.dY);
    const T* pre = static_cast<const T*>(a.pre);
    for (int q = 0; q < kColpartRows / 8; ++q) {
      const int64_t m = rb * kColpartRows + ty + 8 * q;
      if (m >= a.M) break;
      float dy[8], g[8], u[8];
      load8<T>(dY + m * a.lddy + n, nv, dy);
      if (a.act == E_STORE) {
#pragma unroll
        for (int e = 0; e < 8; ++e) g[e] = dy[e];
      } else if (a.act == E_GELU) {
        float p[8];
        load8<T>(pre + m * a.ldpre + n, nv, p);
#pragma unroll
        for (int e = 0; e < 8; ++e) g[e] = dy[e] * gelu_grad_f(p[e]);
      } else {
        float gg[8], uu[8];
        load8<T>(pre + m * a.ldpre + n, nv, gg);
        load8<T>(pre + m * a.ldpre + a.N + n, nv, uu);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float s = sigmoid_f(gg[e]);
          g[e] = dy[e] * uu[e] * (s * (1.0f + gg[e] * (1.0f - s)));
          u[e] = dy[e] * (gg[e] * s);
        }
      }
      if (a.dp) {
        store8<T>(static_cast<T*>(a.dp) + m * a.lddp + n, nv, g);
        if (swiglu) store8<T>(static_cast<T*>(a.dp_up) + m * a.lddp + n, nv, u);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        cg[e] += g[e];
        if (swiglu) cu[e] += u[e];
      }
    }
  }
  if (!a.colpart) return;   // uniform across the block
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    red[ty][0][8 * tx + e] = cg[e];
    red[ty][1][8 * tx + e] = cu[e];
  }
  __syncthreads();
  const int c = threadIdx.x;
  const int64_t nn = (int64_t)blockIdx.y * 256 + c;
  if (nn < a.N) {
    float s0 = 0.f, s1 = 0.f;
    for (int r = 0; r < 8; ++r) {
      s0 += red[r][0][c];
      s1 += red[r][1][c];
    }
    a.colpart[(rb * 2 + 0) * a.ldcp + nn] = s0;
    if (swiglu) a.colpart[(rb * 2 + 1) * a.ldcp + nn] = s1;
  }
}

// out[n] = sum over row blocks (ascending) of colpart[rb][part][n].
template <typename T>
__global__ __launch_bounds__(256) void colsum_finalize_kernel(const float* colpart, int64_t nrb, int64_t ldcp,
                                                              int64_t N, int part, T* out) {
  const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  float s = 0.f;
  for (int64_t rb = 0; rb < nrb; ++rb) s += colpart[(rb * 2 + part) * ldcp + n];
  out[n] = from_f<T>(s);
}

template <typename T>
__global__ __launch_bounds__(256) void sum_partials_kernel(const SumArgs a) {
  const int64_t cpr = (a.N + 7) / 8;
  const int64_t total = a.M * cpr;
  const T* parts = static_cast<const T*>(a.parts);
  const T* bias = static_cast<const T*>(a.bias);
  T* out = static_cast<T*>(a.out);
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total; idx += (int64_t)gridDim.x * 256) {
    const int64_t m = idx / cpr, n = (idx - m * cpr) * 8;
    const int nv = (int)min<int64_t>(8, a.N - n);
    float acc[8], v[8];
    load8<T>(parts + m * a.ld + n, nv, acc);
    for (int i = 1; i < a.t; ++i) {
      load8<T>(parts + i * a.part_stride + m * a.ld + n, nv, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += v[e];
    }
    if (bias)
      for (int e = 0; e < nv; ++e) acc[e] += to_f<T>(bias[n + e]);
    store8<T>(out + m * a.ldo + n, nv, acc);
  }
}

}  // namespace

hipError_t launch_act_bwd(int is_bf16, const ActBwdArgs& a, hipStream_t s) {
  dim3 grid((unsigned)((a.M + kColpartRows - 1) / kColpartRows), (unsigned)((a.N + 255) / 256));
  if (is_bf16) hipLaunchKernelGGL(act_bwd_kernel<uint16_t>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(act_bwd_kernel<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_colsum_finalize(int is_bf16, const float* colpart, int64_t nrb, int64_t ldcp, int64_t N,
                                  int part, void* out, hipStream_t s) {
  dim3 grid((unsigned)((N + 255) / 256));
  if (is_bf16)
    hipLaunchKernelGGL(colsum_finalize_kernel<uint16_t>, grid, dim3(256), 0, s, colpart, nrb, ldcp, N, part,
                       static_cast<uint16_t*>(out));
  else
    hipLaunchKernelGGL(colsum_finalize_kernel<float>, grid, dim3(256), 0, s, colpart, nrb, ldcp, N, part,
                       static_cast<float*>(out));
  return hipGetLastError();
}

hipError_t launch_sum_partials(int is_bf16, const SumArgs& a, hipStream_t s) {
  const int64_t total = a.M * ((a.N + 7) / 8);
  const int64_t blocks = std::min<int64_t>((total + 255) / 256, 256 * 16);
  if (is_bf16) hipLaunchKernelGGL(sum_partials_kernel<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(sum_partials_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace tps
