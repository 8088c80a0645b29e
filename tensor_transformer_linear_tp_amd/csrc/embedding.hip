// Vocab-parallel embedding of one rank: the lookup (rows of the rank's table
// block for the tokens it owns, zero rows for the others) and its backward
// (per-row sums of the owned tokens' output gradients).
//
// The backward groups tokens by table row without atomics on any value:
//   1. emb_order_kernel    one workgroup per 256 table rows counts the owned
//                          tokens of each of its rows (integer LDS counters)
//                          and of all earlier rows, turns them into row starts
//                          and lists each row's tokens in ascending m (a
//                          stable counting sort of the owned tokens);
//   2. emb_bwd_rows_kernel one workgroup per table row sums its tokens'
//                          gradient rows in that order (fp32) and writes the
//                          row once; rows without tokens are written as zeros.
// The result is independent of scheduling: the order of every sum is fixed.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.hpp"
#include "kernels.hpp"

namespace tps {
namespace {

constexpr int kRowsPerBlock = 256;   // table rows per workgroup of the counting kernels

// Row of the rank's block that token id `id` selects, or -1 when not owned.
__device__ __forceinline__ int64_t owned_row(int32_t id, int64_t v0, int64_t Vr) {
  const int64_t r = (int64_t)id - v0;
  return (r >= 0 && r < Vr) ? r : -1;
}

// out[m] = E[ids[m] - v0] for owned tokens, 0 otherwise; raw element copies.
template <typename T>
__global__ __launch_bounds__(256) void emb_fwd_kernel(const EmbArgs a) {
  const int64_t m = blockIdx.x;
  const int64_t r = owned_row(a.ids[m], a.v0, a.Vr);
  const T* src = static_cast<const T*>(a.src) + (r >= 0 ? r : 0) * a.lds;
  T* dst = static_cast<T*>(a.dst) + m * a.ldd;
  constexpr int VEC = 16 / sizeof(T);   // elements per 16-byte vector
  const int64_t full = a.K / VEC;
  for (int64_t j = threadIdx.x; j < full; j += 256) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r >= 0) v = *reinterpret_cast<const u32x4*>(src + j * VEC);
    *reinterpret_cast<u32x4*>(dst + j * VEC) = v;
  }
  const int64_t tail = a.K - full * VEC;
  if (threadIdx.x < tail) {
    const int64_t n = full * VEC + threadIdx.x;
    dst[n] = r >= 0 ? src[n] : T(0);
  }
}

constexpr int kIdBatch = 8;   // ids per thread loaded together (2048 per workgroup)

// Exclusive prefix sum of x over the 256 threads (x >= 0; integers, so the
// result does not depend on the order of the additions); total = the sum
// over all threads.  Each wave scans its 64 values with shuffles, then the
// four wave totals are exchanged through LDS (tmp: 4 entries).
__device__ __forceinline__ int64_t block_excl_scan256(int64_t x, int64_t* tmp, int64_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int64_t v = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t y = __shfl_up(v, o);
    if (lane >= o) v += y;
  }
  if (lane == 63) tmp[wave] = v;
  __syncthreads();
  int64_t before = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) before += w < wave ? tmp[w] : 0;
  total = (tmp[0] + tmp[1]) + (tmp[2] + tmp[3]);
  __syncthreads();   // tmp may be rewritten by the next call
  return before + v - x;
}

// Rows (relative to the block at `base`) of the 8 tokens m0 + threadIdx.x +
// 256 j, or -1 for tokens outside [0, M) or outside the block's rows.  The 8
// id loads are issued together.
__device__ __forceinline__ void block_rows8(const EmbArgs& a, int64_t m0, int64_t base, int32_t (&rr)[kIdBatch]) {
  int32_t id[kIdBatch];
#pragma unroll
  for (int j = 0; j < kIdBatch; ++j) {
    const int64_t m = m0 + threadIdx.x + 256 * j;
    id[j] = a.ids[m < a.M ? m : a.M - 1];
  }
#pragma unroll
  for (int j = 0; j < kIdBatch; ++j) {
    const int64_t m = m0 + threadIdx.x + 256 * j;
    const int64_t r = owned_row(id[j], a.v0, a.Vr) - base;
    rr[j] = (m < a.M && r >= 0 && r < kRowsPerBlock) ? (int32_t)r : -1;
  }
}

// Row starts (start[v], start[Vr] = owned tokens) and the owned tokens listed
// row by row, ascending m within a row.  A first pass over the ids counts
// the tokens of each of the workgroup's rows and the owned tokens of all
// earlier rows (every workgroup reads all ids, so no workgroup waits for
// another).  Then tokens are taken 2048 at a time: an order-preserving
// compaction of the block's tokens into LDS, then each listed token's rank
// among the earlier listed tokens of its row.
__global__ __launch_bounds__(256) void emb_order_kernel(const EmbArgs a, int32_t* start, int32_t* order) {
  constexpr int NB = 256 * kIdBatch;
  __shared__ int64_t tmp[256];
  __shared__ int32_t rstart[kRowsPerBlock];   // first slot of each row of this block
  __shared__ int32_t running[kRowsPerBlock];  // tokens of the row already placed; first the row counts
  __shared__ int32_t lrow[NB], lm[NB], upd[NB];
  __shared__ int32_t wcount[kIdBatch][4];
  const int64_t base = (int64_t)blockIdx.x * kRowsPerBlock;
  const int64_t nrows = min<int64_t>(kRowsPerBlock, a.Vr - base);

  running[threadIdx.x] = 0;
  __syncthreads();
  // Counting pass: 32 ids per thread in flight (8192 ids per round trip).
  constexpr int kCountBatch = 32;
  int64_t before = 0;   // this thread's owned tokens of rows before the block
  for (int64_t m0 = 0; m0 < a.M; m0 += 256 * kCountBatch) {
    int32_t id[kCountBatch];
#pragma unroll
    for (int j = 0; j < kCountBatch; ++j) {
      const int64_t m = m0 + threadIdx.x + 256 * j;
      id[j] = a.ids[m < a.M ? m : a.M - 1];
    }
#pragma unroll
    for (int j = 0; j < kCountBatch; ++j) {
      const int64_t m = m0 + threadIdx.x + 256 * j;
      const int64_t r = owned_row(id[j], a.v0, a.Vr);
      if (m >= a.M || r < 0) continue;
      if (r < base) ++before;
      else if (r < base + kRowsPerBlock) atomicAdd(&running[r - base], 1);   // integer count: order-independent
    }
  }
  __syncthreads();
  int64_t all_before;
  (void)block_excl_scan256(before, tmp, all_before);
  const int64_t own = threadIdx.x < nrows ? running[threadIdx.x] : 0;
  int64_t block_total;
  const int64_t ex = block_excl_scan256(own, tmp, block_total);
  rstart[threadIdx.x] = (int32_t)(all_before + ex);
  running[threadIdx.x] = 0;
  if (threadIdx.x < nrows) start[base + threadIdx.x] = (int32_t)(all_before + ex);
  if (base + nrows == a.Vr && threadIdx.x == 0) start[a.Vr] = (int32_t)(all_before + block_total);
  __syncthreads();

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t below = (1ull << lane) - 1ull;
  for (int64_t m0 = 0; m0 < a.M; m0 += NB) {
    int32_t rr[kIdBatch], inw[kIdBatch];
    block_rows8(a, m0, base, rr);
#pragma unroll
    for (int j = 0; j < kIdBatch; ++j) {
      const uint64_t mask = __ballot(rr[j] >= 0);
      inw[j] = __popcll(mask & below);
      if (lane == 0) wcount[j][wave] = __popcll(mask);
    }
    __syncthreads();
    int k = 0;
#pragma unroll
    for (int j = 0; j < kIdBatch; ++j) {
      int pos = k;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        pos += w < wave ? wcount[j][w] : 0;
        k += wcount[j][w];
      }
      if (rr[j] >= 0) {
        lrow[pos + inw[j]] = rr[j];
        lm[pos + inw[j]] = (int32_t)(m0 + threadIdx.x + 256 * j);
      }
    }
    __syncthreads();
    if (k == 0) continue;   // k is the same on every thread
    for (int p = threadIdx.x; p < k; p += 256) {
      const int32_t r = lrow[p];
      int32_t rank = 0;
      bool last = true;
      for (int i = 0; i < p; ++i) rank += lrow[i] == r ? 1 : 0;
      for (int i = p + 1; i < k; ++i) last = last && lrow[i] != r;
      order[rstart[r] + running[r] + rank] = lm[p];
      upd[p] = last ? rank + 1 : 0;
    }
    __syncthreads();   // every slot computed from the old running counts
    for (int p = threadIdx.x; p < k; p += 256)
      if (upd[p] > 0) running[lrow[p]] += upd[p];   // one entry per row: the row's last token
    __syncthreads();
  }
}

// 8 elements at p as fp32: one 16-byte vector load when FULL (p 16-byte
// aligned), else the first nv elements (the rest 0).
template <bool FULL, typename T>
__device__ __forceinline__ void emb_ld8(const T* p, int nv, float (&x)[8]) {
  if constexpr (FULL && sizeof(T) == 2) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = __uint_as_float(w[e] << 16);
      x[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
  } else if constexpr (FULL) {
    const f32x4 u = *reinterpret_cast<const f32x4*>(p), w = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] = u[e];
      x[4 + e] = w[e];
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if constexpr (sizeof(T) == 2) x[e] = e < nv ? bf2f(p[e]) : 0.f;
      else x[e] = e < nv ? p[e] : 0.f;
    }
  }
}

// acc = sum of g[order[i]] (columns n .. n+7) for i in [s0, s1), ascending i,
// fp32 from 0; the rows are loaded 8 at a time before any is added.
template <bool FULL, typename T>
__device__ __forceinline__ void emb_sum_rows(const T* g, int64_t ldg, const int32_t* order, int32_t s0, int32_t s1,
                                             int64_t n, int nv, float (&acc)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  for (int32_t i0 = s0; i0 < s1; i0 += 8) {
    float x[8][8];
#pragma unroll
    for (int j = 0; j < 8; ++j) emb_ld8<FULL>(g + (int64_t)order[min(i0 + j, s1 - 1)] * ldg + n, nv, x[j]);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (i0 + j < s1) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += x[j][e];
      }
    }
  }
}

// dE[v] = sum over the row's tokens (ascending m) of dout[m]; zeros when none.
template <typename T>
__global__ __launch_bounds__(256) void emb_bwd_rows_kernel(const EmbArgs a, const int32_t* start,
                                                           const int32_t* order) {
  const int64_t v = blockIdx.x;
  const int32_t s0 = start[v], s1 = start[v + 1];
  const T* g = static_cast<const T*>(a.src);
  T* dE = static_cast<T*>(a.dst) + v * a.ldd;
  const int64_t cpr = (a.K + 7) / 8;
  for (int64_t chunk = threadIdx.x; chunk < cpr; chunk += 256) {
    const int64_t n = chunk * 8;
    const int nv = (int)min<int64_t>(8, a.K - n);
    float acc[8];
    if (nv == 8) {
      emb_sum_rows<true, T>(g, a.lds, order, s0, s1, n, 8, acc);
      if constexpr (sizeof(T) == 2) {
        *reinterpret_cast<u32x4*>(dE + n) = u32x4{pack_bf2(acc[0], acc[1]), pack_bf2(acc[2], acc[3]),
                                                  pack_bf2(acc[4], acc[5]), pack_bf2(acc[6], acc[7])};
      } else {
        *reinterpret_cast<f32x4*>(dE + n) = f32x4{acc[0], acc[1], acc[2], acc[3]};
        *reinterpret_cast<f32x4*>(dE + n + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
      }
    } else {
      emb_sum_rows<false, T>(g, a.lds, order, s0, s1, n, nv, acc);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (e < nv) {
          if constexpr (sizeof(T) == 2) dE[n + e] = f2bf(acc[e]);
          else dE[n + e] = acc[e];
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_emb_fwd(int is_bf16, const EmbArgs& a, hipStream_t s) {
  if (is_bf16) hipLaunchKernelGGL(emb_fwd_kernel<uint16_t>, dim3((unsigned)a.M), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(emb_fwd_kernel<float>, dim3((unsigned)a.M), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_emb_bwd(int is_bf16, const EmbArgs& a, int32_t* start, int32_t* order, hipStream_t s) {
  const unsigned nb = (unsigned)((a.Vr + kRowsPerBlock - 1) / kRowsPerBlock);
  hipLaunchKernelGGL(emb_order_kernel, dim3(nb), dim3(256), 0, s, a, start, order);
  if (is_bf16) hipLaunchKernelGGL(emb_bwd_rows_kernel<uint16_t>, dim3((unsigned)a.Vr), dim3(256), 0, s, a, start, order);
  else hipLaunchKernelGGL(emb_bwd_rows_kernel<float>, dim3((unsigned)a.Vr), dim3(256), 0, s, a, start, order);
  return hipGetLastError();
}

}  // namespace tps
