// fp32 GEMM family for gfx950: C = A B on v_mfma_f32_16x16x4_f32 (full fp32
// products and accumulation), with the same layouts and epilogues as the
// bf16 kernels.  Sized for small shards: a 256-thread workgroup owns a 64 x 64
// output tile (SwiGLU: 64 rows x (32 gate + 32 up)), each wave a 32 x 32
// block of four 16 x 16 MFMA tiles; K advances 16 per LDS stage.
#include "device_common.hpp"
#include "kernels.hpp"

namespace tps {
namespace {

constexpr int TB = 64, TK = 16, LDT = TB + 4;

// Per-element bounds-checked loads: this kernel serves small problems.
__device__ __forceinline__ float ldf(const float* p, int64_t r, int64_t c, int64_t ld, int64_t rows, int64_t cols) {
  return (r < rows && c < cols) ? p[r * ld + c] : 0.f;
}

template <int LAYOUT>
__device__ __forceinline__ void load_tiles(const Problem& P, const Seg& S, int64_t m0, int64_t n0, int64_t k0,
                                           float (*As)[LDT], float (*Bs)[LDT]) {
  const int t = threadIdx.x;
  const float* a = static_cast<const float*>(S.a);
  const float* b = static_cast<const float*>(S.b);
  const bool dual = P.epi == E_SWIGLU;
  // A tile -> As[k][m]
  if (LAYOUT != L_TN) {                 // A [M][K]
    const int m = t >> 2, kq = (t & 3) * 4;
#pragma unroll
    for (int e = 0; e < 4; ++e) As[kq + e][m] = ldf(a, m0 + m, k0 + kq + e, S.lda, P.M, S.K);
  } else {                              // A [K][M]
    const int k = t >> 4, mq = (t & 15) * 4;
#pragma unroll
    for (int e = 0; e < 4; ++e) As[k][mq + e] = ldf(a, k0 + k, m0 + mq + e, S.lda, S.K, P.M);
  }
  // B tile -> Bs[k][n]
  if (LAYOUT == L_NT) {                 // B [N][K]
    const int n = t >> 2, kq = (t & 3) * 4;
#pragma unroll
    for (int e = 0; e < 4; ++e) Bs[kq + e][n] = ldf(b, n0 + n, k0 + kq + e, S.ldb, P.N, S.K);
  } else {                              // B [K][N]
    const int k = t >> 4, nq = (t & 15) * 4;
    if (dual) {                         // columns [0,32) gate, [32,64) up
      const bool up = nq >= 32;
      const float* p = up ? static_cast<const float*>(P.b_up) : b;
      const int64_t ld = up ? P.ldb_up : S.ldb;
      const int64_t c = n0 + (nq & 31);
#pragma unroll
      for (int e = 0; e < 4; ++e) Bs[k][nq + e] = ldf(p, k0 + k, c + e, ld, S.K, P.N);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) Bs[k][nq + e] = ldf(b, k0 + k, n0 + nq + e, S.ldb, S.K, P.N);
    }
  }
}

__device__ __forceinline__ void epi4_f32(const Problem& P, int64_t m, int64_t n, float (&v)[4], float (&u)[4]) {
  const int nv = (int)min<int64_t>(4, P.N - n);
  if (P.bias)
    for (int e = 0; e < nv; ++e) v[e] += static_cast<const float*>(P.bias)[n + e];
  float y[4];
  if (P.epi == E_STORE) {
    for (int e = 0; e < 4; ++e) y[e] = v[e];
  } else if (P.epi == E_GELU) {
    float* pre = static_cast<float*>(P.pre) + m * P.ldpre + n;
    for (int e = 0; e < nv; ++e) pre[e] = v[e];
    for (int e = 0; e < 4; ++e) y[e] = gelu_f(v[e]);
  } else {
    if (P.bias2)
      for (int e = 0; e < nv; ++e) u[e] += static_cast<const float*>(P.bias2)[n + e];
    float* pre = static_cast<float*>(P.pre) + m * P.ldpre;
    for (int e = 0; e < nv; ++e) {
      pre[n + e] = v[e];
      pre[P.N + n + e] = u[e];
    }
    for (int e = 0; e < 4; ++e) y[e] = silu_f(v[e]) * u[e];
  }
  float* c = static_cast<float*>(P.c) + m * P.ldc + n;
  for (int e = 0; e < nv; ++e) c[e] = y[e];
}

template <int LAYOUT>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const Problem P) {
  __shared__ float As[TK][LDT];
  __shared__ float Bs[TK][LDT];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wm = wave >> 1, wn = wave & 1;
  const bool dual = P.epi == E_SWIGLU;
  const int64_t m0 = (int64_t)blockIdx.y * TB;
  const int64_t n0 = (int64_t)blockIdx.x * (dual ? TB / 2 : TB);
  f32x4 acc[2][2];
  for (int i = 0; i < 2; ++i)
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < P.nseg; ++s) {
    const Seg& S = s ? P.seg[1] : P.seg[0];
    for (int64_t k0 = 0; k0 < S.K; k0 += TK) {
      load_tiles<LAYOUT>(P, S, m0, n0, k0, As, Bs);
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < TK / 4; ++kk) {
        const int k = 4 * kk + (lane >> 4);
        float a[2], b[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) a[i] = As[k][32 * wm + 16 * i + (lane & 15)];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int bc = dual ? 32 * j + 16 * wn : 32 * wn + 16 * j;
          b[j] = Bs[k][bc + (lane & 15)];
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(b[j], a[i], acc[i][j], 0, 0, 0);
      }
      __syncthreads();
    }
  }
  // lane holds rows m = .. + lane%16, four consecutive columns n = .. + 4*(lane/16) + r
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int64_t m = m0 + 32 * wm + 16 * i + (lane & 15);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (dual && j == 1) continue;
      const int64_t n = n0 + (dual ? 16 * wn : 32 * wn + 16 * j) + 4 * (lane >> 4);
      if (m >= P.M || n >= P.N) continue;
      float v[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
      float u[4] = {acc[i][1][0], acc[i][1][1], acc[i][1][2], acc[i][1][3]};
      epi4_f32(P, m, n, v, u);
    }
  }
}

}  // namespace

hipError_t launch_gemm_f32(GemmLaunch& L, hipStream_t s) {
  for (int i = 0; i < L.nprob; ++i) {
    const Problem& P = L.p[i];
    const int64_t bn = (P.epi == E_SWIGLU) ? TB / 2 : TB;
    dim3 grid((unsigned)((P.N + bn - 1) / bn), (unsigned)((P.M + TB - 1) / TB));
    switch (P.layout) {
      case L_NN: hipLaunchKernelGGL(gemm_f32_kernel<L_NN>, grid, dim3(256), 0, s, P); break;
      case L_NT: hipLaunchKernelGGL(gemm_f32_kernel<L_NT>, grid, dim3(256), 0, s, P); break;
      default: hipLaunchKernelGGL(gemm_f32_kernel<L_TN>, grid, dim3(256), 0, s, P); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace tps
