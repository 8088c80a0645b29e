// HBM-bound kernels of the shard path: the column-epilogue backward (dP from
// dY and the saved pre-activation, fused with fp32 column partial sums for the
// bias gradients), the ordered reduction of those partials, the t-way sum of
// shard partials, and its sequence-parallel form fused with the residual add
// and LayerNorm.  Each thread moves 8 consecutive columns with 16-byte
// accesses when the row segment is whole and aligned.
#include <algorithm>
#include <type_traits>
#include <utility>

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
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (e < nv) p[e] = f2bf(v[e]);
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
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (e < nv) p[e] = v[e];
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

// 8 columns at p: one 16-byte-aligned vector load when FULL, else the first
// nv elements one by one (the rest 0).  Callers pass 16-byte-aligned p when
// FULL (base pointers, leading dimensions and strides are validated so).
// STREAM: a nontemporal load, for data read once (measured ~12 % faster on
// the partial sums, which read 8 and write 1 buffer of 64 MiB).
template <bool FULL, typename T, bool STREAM = false>
__device__ __forceinline__ void ld8(const T* p, int nv, float (&v)[8]) {
  if constexpr (FULL) {
    if constexpr (sizeof(T) == 2) {
      const u32x4* q = reinterpret_cast<const u32x4*>(p);
      const u32x4 w = STREAM ? __builtin_nontemporal_load(q) : *q;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[2 * e] = __uint_as_float(w[e] << 16);
        v[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
      }
    } else {
      const f32x4* q = reinterpret_cast<const f32x4*>(p);
      const f32x4 x = STREAM ? __builtin_nontemporal_load(q) : q[0];
      const f32x4 y = STREAM ? __builtin_nontemporal_load(q + 1) : q[1];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] = x[e];
        v[4 + e] = y[e];
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = e < nv ? to_f<T>(p[e]) : 0.f;
  }
}

// Store of 8 columns at p: one 16-byte vector store when FULL (p 16-byte
// aligned), else the first nv elements.  STREAM: a nontemporal store.
template <bool FULL, typename T, bool STREAM = false>
__device__ __forceinline__ void st8(T* p, int nv, const float (&v)[8]) {
  if constexpr (FULL && sizeof(T) == 2) {
    const u32x4 w = {pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]), pack_bf2(v[4], v[5]), pack_bf2(v[6], v[7])};
    if (STREAM) __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p));
    else *reinterpret_cast<u32x4*>(p) = w;
  } else if constexpr (FULL) {
    const f32x4 x = {v[0], v[1], v[2], v[3]}, y = {v[4], v[5], v[6], v[7]};
    if (STREAM) {
      __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(p));
      __builtin_nontemporal_store(y, reinterpret_cast<f32x4*>(p + 4));
    } else {
      *reinterpret_cast<f32x4*>(p) = x;
      *reinterpret_cast<f32x4*>(p + 4) = y;
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (e < nv) p[e] = from_f<T>(v[e]);
  }
}

// Rows ty, ty + 8, ... (64 rows) of row block rb at columns n .. n + 7 of the
// activation backward, RB rows at a time with all their loads issued first
// (past the matrix the row index repeats the last row: loaded, not used);
// column sums of dP accumulate into cg (gate or single) and cu (up).
template <bool FULL, int ACT, typename T>
__device__ __forceinline__ void act_rows(const ActBwdArgs& a, int64_t rb, int ty, int64_t n, int nv, float (&cg)[8],
                                         float (&cu)[8]) {
  constexpr int RB = 4;
  constexpr bool swiglu = ACT == E_SWIGLU;
  const T* dY = static_cast<const T*>(a.dY);
  // Without an activation there is no Pre (it may be NULL): the pre-activation
  // loads then read dY again (values unused), so every load is unconditional.
  constexpr bool has_pre = ACT != E_STORE;
  const T* pre = has_pre ? static_cast<const T*>(a.pre) : dY;
  const int64_t ldpre = has_pre ? a.ldpre : a.lddy;
#pragma unroll
  for (int q0 = 0; q0 < kColpartRows / 8; q0 += RB) {
    float dy[RB][8], gg[RB][8], uu[RB][8];
#pragma unroll
    for (int j = 0; j < RB; ++j) {
      const int64_t m = min<int64_t>(rb * kColpartRows + ty + 8 * (q0 + j), a.M - 1);
      ld8<FULL, T, true>(dY + m * a.lddy + n, nv, dy[j]);
      ld8<FULL, T, true>(pre + m * ldpre + n, nv, gg[j]);
      ld8<FULL, T, true>(pre + m * ldpre + (swiglu ? a.N : 0) + n, nv, uu[j]);   // up half (SwiGLU only)
    }
#pragma unroll
    for (int j = 0; j < RB; ++j) {
      const int64_t m = rb * kColpartRows + ty + 8 * (q0 + j);
      const bool live = m < a.M;
      float g[8], u[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (ACT == E_STORE) {
          g[e] = dy[j][e];
          u[e] = 0.f;
        } else if (ACT == E_GELU) {
          g[e] = dy[j][e] * gelu_grad_f(gg[j][e]);
          u[e] = 0.f;
        } else {
          const float sg = sigmoid_f(gg[j][e]);
          g[e] = dy[j][e] * uu[j][e] * (sg * (1.0f + gg[j][e] * (1.0f - sg)));
          u[e] = dy[j][e] * (gg[j][e] * sg);
        }
        cg[e] += live ? g[e] : 0.f;
        cu[e] += live ? u[e] : 0.f;
      }
      if (live && a.dp) {
        st8<FULL>(static_cast<T*>(a.dp) + m * a.lddp + n, nv, g);
        if (swiglu) st8<FULL>(static_cast<T*>(a.dp_up) + m * a.lddp + n, nv, u);
      }
    }
  }
}

// Block (x = row block, y = column block): 32 column-threads x 8 row-threads
// over [64 rows] x [256 columns].
template <typename T, int ACT>
__global__ __launch_bounds__(256) void act_bwd_kernel(const ActBwdArgs a) {
  __shared__ float red[8][2][256];
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  const int64_t n = (int64_t)blockIdx.y * 256 + 8 * tx;
  const int64_t rb = blockIdx.x;
  constexpr bool swiglu = ACT == E_SWIGLU;
  float cg[8], cu[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) cg[e] = cu[e] = 0.f;
  if (n < a.N) {
    const int nv = (int)min<int64_t>(8, a.N - n);
    if (nv == 8) act_rows<true, ACT, T>(a, rb, ty, n, nv, cg, cu);
    else act_rows<false, ACT, T>(a, rb, ty, n, nv, cg, cu);
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

// acc = sum_{i<t} p[i * stride] over 8 columns, fp32, in ascending i.  The
// partials are loaded G at a time before any of them is added, so a thread
// keeps G loads in flight; past the last partial the load repeats partial t-1
// (a cache hit) and is not added.
template <bool FULL, typename T, int G>
__device__ __forceinline__ void sum_parts8(const T* p, int64_t stride, int t, int nv, float (&acc)[8]) {
  for (int i0 = 0; i0 < t; i0 += G) {
    float v[G][8];
#pragma unroll
    for (int j = 0; j < G; ++j) ld8<FULL, T, true>(p + min(i0 + j, t - 1) * stride, nv, v[j]);
#pragma unroll
    for (int j = 0; j < G; ++j) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (i0 + j == 0) acc[e] = v[j][e];
        else if (i0 + j < t) acc[e] += v[j][e];
      }
    }
  }
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
    float acc[8];
    if (nv == 8) sum_parts8<true, T, 8>(parts + m * a.ld + n, a.part_stride, a.t, nv, acc);
    else sum_parts8<false, T, 8>(parts + m * a.ld + n, a.part_stride, a.t, nv, acc);
    if (bias)
      for (int e = 0; e < nv; ++e) acc[e] += to_f<T>(bias[n + e]);
    if (nv == 8) st8<true, T, true>(out + m * a.ldo + n, nv, acc);   // 16-byte aligned: validated base and ld
    else store8<T>(out + m * a.ldo + n, nv, acc);
  }
}

// One token per thread: M* = max_r m_r, S* = sum_r s_r exp(m_r - M*) (shards
// in ascending r), lse = M* + ln S*, tgt = sum_r tgt_r, loss = lse - tgt.
// fp64 throughout (the inputs are exact in it), one rounding to fp32 per
// output.  A token whose every shard max is -inf gets lse = -inf.
__global__ __launch_bounds__(256) void ce_combine_kernel(const CECombineArgs a) {
  const int64_t m = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (m >= a.M) return;
  double mx = -INFINITY;
  for (int r = 0; r < a.R; ++r) mx = fmax(mx, (double)a.maxes[(int64_t)r * a.stride + m]);
  double s = 0.0, t = 0.0;
  for (int r = 0; r < a.R; ++r) {
    const int64_t i = (int64_t)r * a.stride + m;
    const double mr = (double)a.maxes[i];
    if (mr > -INFINITY) s += (double)a.sumexps[i] * exp(mr - mx);
    t += (double)a.tgts[i];
  }
  const double lse = s > 0.0 ? mx + log(s) : -INFINITY;
  if (a.lse) a.lse[m] = (float)lse;
  if (a.tgt) a.tgt[m] = (float)t;
  if (a.loss) a.loss[m] = (float)(lse - t);
}

// Sum of v over the 256 threads of the workgroup, the same on every thread
// (fixed reduction tree: the result does not depend on timing).
__device__ __forceinline__ float block_sum256(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int wave = threadIdx.x >> 6;
  __syncthreads();   // red may still be read from a previous call
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// Calls f(std::integral_constant<int, c>) for c = 0 .. CH-1, so that register
// arrays indexed by c keep compile-time indices.
template <typename F, int... C>
__device__ __forceinline__ void for_each_chunk(F&& f, std::integer_sequence<int, C...>) {
  (f(std::integral_constant<int, C>{}), ...);
}

// bf16 element e (0..7) of an 8-column chunk held as 4 raw words.
__device__ __forceinline__ float bf16_at(const u32x4& w, int e) {
  return __uint_as_float((e & 1) ? (w[e >> 1] & 0xffff0000u) : (w[e >> 1] << 16));
}

// The common case of sp_rs_ln_kernel (bf16, N = 2048 CH with CH <= 2 so that
// every thread holds CH whole chunks in ~100 registers, t <= 8): every load
// of the row -- the t partials,
// bias, residual, gamma and beta of all CH chunks -- is issued before any is
// used, so the row costs one round trip to memory; the raw words are kept
// until they are added.  Same arithmetic, in the same order, as the general
// path.  (Absent vectors load partial 0 instead and are not used.)
template <int CH>
__device__ __forceinline__ void sp_rs_ln_row_bf16(const SpLnArgs& a, float* red) {
  const int64_t m = blockIdx.x;
  const int64_t row = a.r0 + m;
  const uint16_t* parts = static_cast<const uint16_t*>(a.parts);
  const uint16_t* bias = static_cast<const uint16_t*>(a.bias);
  const uint16_t* resid = static_cast<const uint16_t*>(a.resid);
  const uint16_t* gamma = static_cast<const uint16_t*>(a.gamma);
  const uint16_t* beta = static_cast<const uint16_t*>(a.beta);
  u32x4 pv[CH][8], bv[CH], rv[CH], gv[CH], ev[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int64_t n = (int64_t)(threadIdx.x + 256 * c) * 8;
    const uint16_t* p0 = parts + row * a.ld + n;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint16_t* pi = p0 + (int64_t)min(i, a.t - 1) * a.part_stride;
      pv[c][i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(pi));
    }
    bv[c] = *reinterpret_cast<const u32x4*>(bias ? bias + n : p0);
    rv[c] = *reinterpret_cast<const u32x4*>(resid ? resid + m * a.ldr + n : p0);
    gv[c] = *reinterpret_cast<const u32x4*>(gamma ? gamma + n : p0);
    ev[c] = *reinterpret_cast<const u32x4*>(beta ? beta + n : p0);
  }
  float h[CH][8];
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < CH; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = bf16_at(pv[c][0], e);
#pragma unroll
      for (int i = 1; i < 8; ++i)
        if (i < a.t) x += bf16_at(pv[c][i], e);
      if (bias) x += bf16_at(bv[c], e);
      if (resid) x += bf16_at(rv[c], e);
      h[c][e] = x;
      s += x;
    }
  const float mean = block_sum256(s, red) / (float)a.N;
  float s2 = 0.f;
#pragma unroll
  for (int c = 0; c < CH; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float d = h[c][e] - mean;
      s2 += d * d;
    }
  const float var = block_sum256(s2, red) / (float)a.N;
  const float rstd = 1.0f / sqrtf(var + a.eps);
  uint16_t* out = static_cast<uint16_t*>(a.out);
  uint16_t* hout = static_cast<uint16_t*>(a.hout);
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int64_t n = (int64_t)(threadIdx.x + 256 * c) * 8;
    if (hout) store8<uint16_t>(hout + m * a.ldh + n, 8, h[c]);
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      y[e] = (h[c][e] - mean) * rstd * (gamma ? bf16_at(gv[c], e) : 1.f) + (beta ? bf16_at(ev[c], e) : 0.f);
    store8<uint16_t>(out + m * a.ldo + n, 8, y);
  }
}

// One workgroup per row of the rank's block; each thread holds CH chunks of 8
// columns in registers (N <= 2048 * CH), so the row is read once.
template <typename T, int CH>
__global__ __launch_bounds__(256) void sp_rs_ln_kernel(const SpLnArgs a) {
  __shared__ float red[4];
  if constexpr (sizeof(T) == 2 && CH <= 2) {
    if (a.N == 2048 * CH && a.t <= 8) {   // uniform: the whole launch takes one path
      sp_rs_ln_row_bf16<CH>(a, red);
      return;
    }
  }
  constexpr auto chunks = std::make_integer_sequence<int, CH>{};
  const int64_t m = blockIdx.x;
  const int64_t row = a.r0 + m;
  const int64_t cpr = (a.N + 7) / 8;
  const T* parts = static_cast<const T*>(a.parts);
  const T* bias = static_cast<const T*>(a.bias);
  const T* resid = static_cast<const T*>(a.resid);
  float h[CH][8];
  float s = 0.f;
  for_each_chunk([&](auto cc) {
    constexpr int c = decltype(cc)::value;
    const int64_t chunk = threadIdx.x + 256 * c;
#pragma unroll
    for (int e = 0; e < 8; ++e) h[c][e] = 0.f;
    if (chunk < cpr) {
      const int64_t n = chunk * 8;
      const int nv = (int)min<int64_t>(8, a.N - n);
      auto body = [&](auto full) {
        constexpr bool FULL = decltype(full)::value;
        // bias and residual are loaded first and added after the partials, in
        // this order; an absent one loads partial 0 instead (no branch around
        // the load) and is not added
        const T* p0 = parts + row * a.ld + n;
        float bv[8], rv[8];
        ld8<FULL>(bias ? bias + n : p0, nv, bv);
        ld8<FULL>(resid ? resid + m * a.ldr + n : p0, nv, rv);
        sum_parts8<FULL, T, 8>(p0, a.part_stride, a.t, nv, h[c]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if (bias) h[c][e] += bv[e];
          if (resid) h[c][e] += rv[e];
          s += h[c][e];   // masked columns hold 0
        }
      };
      if (nv == 8) body(std::true_type{});
      else body(std::false_type{});
    }
  }, chunks);
  const float mean = block_sum256(s, red) / (float)a.N;
  float s2 = 0.f;
  for_each_chunk([&](auto cc) {
    constexpr int c = decltype(cc)::value;
    const int64_t chunk = threadIdx.x + 256 * c;
    if (chunk < cpr) {
      const int nv = (int)min<int64_t>(8, a.N - chunk * 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float d = h[c][e] - mean;
        s2 += e < nv ? d * d : 0.f;
      }
    }
  }, chunks);
  const float var = block_sum256(s2, red) / (float)a.N;
  const float rstd = 1.0f / sqrtf(var + a.eps);
  const T* gamma = static_cast<const T*>(a.gamma);
  const T* beta = static_cast<const T*>(a.beta);
  T* out = static_cast<T*>(a.out);
  T* hout = static_cast<T*>(a.hout);
  for_each_chunk([&](auto cc) {
    constexpr int c = decltype(cc)::value;
    const int64_t chunk = threadIdx.x + 256 * c;
    if (chunk < cpr) {
      const int64_t n = chunk * 8;
      const int nv = (int)min<int64_t>(8, a.N - n);
      if (hout) store8<T>(hout + m * a.ldh + n, nv, h[c]);
      float g[8], b[8], y[8];   // absent gamma / beta: partial 0 is loaded instead, not used
      const T* own = parts + row * a.ld + n;
      if (nv == 8) {
        ld8<true>(gamma ? gamma + n : own, 8, g);
        ld8<true>(beta ? beta + n : own, 8, b);
      } else {
        ld8<false>(gamma ? gamma + n : own, nv, g);
        ld8<false>(beta ? beta + n : own, nv, b);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = (h[c][e] - mean) * rstd * (gamma ? g[e] : 1.f) + (beta ? b[e] : 0.f);
      store8<T>(out + m * a.ldo + n, nv, y);
    }
  }, chunks);
}

}  // namespace

template <typename T>
static void launch_sp_rs_ln_t(const SpLnArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)a.Mr), block(256);
  if (a.N <= 2048) hipLaunchKernelGGL((sp_rs_ln_kernel<T, 1>), grid, block, 0, s, a);
  else if (a.N <= 4096) hipLaunchKernelGGL((sp_rs_ln_kernel<T, 2>), grid, block, 0, s, a);
  else if (a.N <= 8192) hipLaunchKernelGGL((sp_rs_ln_kernel<T, 4>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((sp_rs_ln_kernel<T, kSpLnMaxN / 2048>), grid, block, 0, s, a);
}

hipError_t launch_sp_rs_ln(int is_bf16, const SpLnArgs& a, hipStream_t s) {
  if (a.N < 1 || a.N > kSpLnMaxN) return hipErrorInvalidValue;
  if (a.Mr <= 0) return hipSuccess;
  if (is_bf16) launch_sp_rs_ln_t<uint16_t>(a, s);
  else launch_sp_rs_ln_t<float>(a, s);
  return hipGetLastError();
}

hipError_t launch_act_bwd(int is_bf16, const ActBwdArgs& a, hipStream_t s) {
  dim3 grid((unsigned)((a.M + kColpartRows - 1) / kColpartRows), (unsigned)((a.N + 255) / 256));
#define TPS_ACT_LAUNCH(T)                                                                                     \
  do {                                                                                                        \
    if (a.act == E_SWIGLU) hipLaunchKernelGGL((act_bwd_kernel<T, E_SWIGLU>), grid, dim3(256), 0, s, a);       \
    else if (a.act == E_GELU) hipLaunchKernelGGL((act_bwd_kernel<T, E_GELU>), grid, dim3(256), 0, s, a);      \
    else hipLaunchKernelGGL((act_bwd_kernel<T, E_STORE>), grid, dim3(256), 0, s, a);                          \
  } while (0)
  if (is_bf16) TPS_ACT_LAUNCH(uint16_t);
  else TPS_ACT_LAUNCH(float);
#undef TPS_ACT_LAUNCH
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

hipError_t launch_ce_combine(const CECombineArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(ce_combine_kernel, dim3((unsigned)((a.M + 255) / 256)), dim3(256), 0, s, a);
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
