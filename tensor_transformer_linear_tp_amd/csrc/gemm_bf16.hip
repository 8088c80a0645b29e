// bf16 GEMM family for gfx950 (MI355X): C = A B with fp32 accumulation on
// v_mfma_f32_32x32x16_bf16, LDS-staged double-buffered tiles and fused
// epilogues; plus the vocab-parallel LM-head kernel whose epilogue reduces
// logit tiles to (max, sum exp) partials without writing the logits.
//
// Tiling: a 256-thread workgroup (4 wave64s as 2 x 2) owns a 256 x 256 output
// tile (SwiGLU: 256 rows x (128 gate + 128 up) columns); each wave owns
// 128 x 128 = 4 x 4 MFMA blocks of 32 x 32.  K advances 64 per LDS stage.
//
// LDS layouts.  Operands are copied global -> registers -> LDS in their
// global orientation:
//   * K-contiguous operand (A of NN/NT, B of NT): [256 rows][64 k], read as
//     MFMA fragments with one ds_read_b128 per lane;
//   * MN-contiguous operand (A of TN, B of NN/TN): [64 k][256 cols], read
//     with two ds_read_b64_tr_b16 per lane, which transposes 16-bit elements
//     across each 16-lane group on the way out of LDS.
// Both use an XOR swizzle of the 16-byte chunk index so that fragment reads
// and the staging writes fall into distinct banks.
//
// Accumulator orientation.  The MFMA is issued as (B fragment, A fragment),
// so each lane holds four consecutive output columns of one row per
// register quad; epilogue stores are 8-byte (bf16) vectors.
#include <utility>

#include "device_common.hpp"
#include "kernels.hpp"

namespace tps {
namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int NTHREADS = 256;
constexpr int TILE_BYTES = 256 * BK * 2;      // 32 KiB per operand tile
constexpr int BUF_BYTES = 2 * TILE_BYTES;     // A + B
constexpr int LDS_BYTES = 2 * BUF_BYTES;      // double buffered: 128 KiB
constexpr int GROUP_M = 8;                    // tile rows per L2 group

// ---- LDS address maps ------------------------------------------------------
// K-contiguous [256][64]: 128-byte rows, 8 chunks of 16 bytes each.
__device__ __forceinline__ int kc_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int kc_off(int r, int c) { return r * 128 + ((c ^ kc_swz(r)) << 4); }
// MN-contiguous [64][256]: 512-byte rows, 32 chunks; rows k%4 = 0,1,2,3 XOR the
// chunk index with 0, 6, 10, 12.
__device__ __forceinline__ int mn_swz(int k) { return (0xCA60 >> ((k & 3) * 4)) & 15; }
__device__ __forceinline__ int mn_off(int k, int c) { return k * 512 + ((c ^ mn_swz(k)) << 4); }

__device__ __forceinline__ u32x4 ldg16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }

// Zero the bf16 elements [valid, 8) of a 16-byte chunk.
__device__ __forceinline__ u32x4 mask_tail(u32x4 v, int64_t valid) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    int e0 = 2 * w;
    uint32_t keep = (e0 + 1 < valid) ? 0xffffffffu : (e0 < valid ? 0x0000ffffu : 0u);
    v[w] &= keep;
  }
  return v;
}

// ---- global -> register staging ---------------------------------------------
// K-contiguous operand, tile rows [row0, row0+256), k [k0, k0+64).
__device__ __forceinline__ void load_kc(u32x4 (&r)[8], const uint16_t* p, int64_t ld, int64_t rows,
                                        int64_t row0, int64_t K, int64_t k0) {
  const int t = threadIdx.x;
  const int64_t k = k0 + (t & 7) * 8;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t row = row0 + (t >> 3) + 32 * i;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (row < rows && k < K) {
      v = ldg16(p + row * ld + k);
      if (k + 8 > K) v = mask_tail(v, K - k);
    }
    r[i] = v;
  }
}

// MN-contiguous operand, tile k [k0, k0+64), cols [col0, col0+256).
__device__ __forceinline__ void load_mn(u32x4 (&r)[8], const uint16_t* p, int64_t ld, int64_t cols,
                                        int64_t col0, int64_t K, int64_t k0) {
  const int t = threadIdx.x;
  const int64_t col = col0 + (t & 31) * 8;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t k = k0 + (t >> 5) + 8 * i;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (k < K && col < cols) v = ldg16(p + k * ld + col);
    r[i] = v;
  }
}

// SwiGLU B tile: LDS columns [0,128) from the gate weight, [128,256) from the
// up weight, both at output columns [col0, col0+128).
__device__ __forceinline__ void load_mn_dual(u32x4 (&r)[8], const uint16_t* pg, const uint16_t* pu,
                                             int64_t ldg, int64_t ldu, int64_t cols, int64_t col0,
                                             int64_t K, int64_t k0) {
  const int t = threadIdx.x;
  const int ch = t & 31;
  const bool up = ch >= 16;
  const uint16_t* p = up ? pu : pg;
  const int64_t ld = up ? ldu : ldg;
  const int64_t col = col0 + (ch & 15) * 8;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t k = k0 + (t >> 5) + 8 * i;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (k < K && col < cols) v = ldg16(p + k * ld + col);
    r[i] = v;
  }
}

__device__ __forceinline__ void store_kc(TPS_LDS char* s, const u32x4 (&r)[8]) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 8; ++i) *reinterpret_cast<TPS_LDS u32x4*>(s + kc_off((t >> 3) + 32 * i, t & 7)) = r[i];
}

__device__ __forceinline__ void store_mn(TPS_LDS char* s, const u32x4 (&r)[8]) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 8; ++i) *reinterpret_cast<TPS_LDS u32x4*>(s + mn_off((t >> 5) + 8 * i, t & 31)) = r[i];
}

// ---- LDS -> MFMA fragments ---------------------------------------------------
// Operand fragment of v_mfma_f32_32x32x16_bf16: lane l holds 8 consecutive k
// (k = 8*(l/32) + 0..7 within the 16-deep step) of row/column (l % 32).
__device__ __forceinline__ bf16x8 frag_kc(const TPS_LDS char* s, int rb, int kk) {
  const int lane = threadIdx.x & 63;
  const int r = rb + (lane & 31);
  const int c = 2 * kk + (lane >> 5);
  return *reinterpret_cast<const TPS_LDS bf16x8*>(s + kc_off(r, c));
}

// Same fragment from an MN-contiguous tile.  ds_read_b64_tr_b16: within each
// 16-lane group, lane i receives element (i % 4) of the 8-byte loads of
// source lanes i/4, 4 + i/4, 8 + i/4, 12 + i/4.  Source lane s therefore
// loads row k = base + s/4, columns c + 4*(s % 4) .. +3, and lane i ends up
// with rows base..base+3 of column c + i.
__device__ __forceinline__ bf16x8 frag_mn(const TPS_LDS char* s, int cb, int kk) {
  const int lane = threadIdx.x & 63;
  const int h = lane >> 4, q = lane & 15;
  const int col = cb + 16 * (h & 1) + 4 * (q & 3);
  const int k0 = 16 * kk + 8 * (h >> 1) + (q >> 2);
  const int c = col >> 3, byte_in = (col & 7) * 2;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (TPS_LDS i16x4*)(s + mn_off(k0, c) + byte_in));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (TPS_LDS i16x4*)(s + mn_off(k0 + 4, c) + byte_in));
  typedef __attribute__((ext_vector_type(8))) short i16x8;
  const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// ---- scheduling --------------------------------------------------------------
// Workgroups are dispatched round-robin over the 8 XCDs; give each XCD a
// contiguous range of tile ids so neighbouring tiles share its L2.
__device__ __forceinline__ int xcd_remap(int bid, int total) {
  const int q = total >> 3, r = total & 7;
  const int xcd = bid & 7, slot = bid >> 3;
  return (xcd < r) ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
}

// Grouped order inside a problem: GROUP_M tile rows sweep the tile columns.
__device__ __forceinline__ void tile_coords(int id, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int group = GROUP_M * tiles_n;
  const int g = id / group;
  const int first = g * GROUP_M;
  const int gm = min(tiles_m - first, GROUP_M);
  const int r = id - g * group;
  tm = first + r % gm;
  tn = r / gm;
}

// ---- main loop -------------------------------------------------------------------
template <int LAYOUT>
__device__ __forceinline__ void mainloop(const Problem& P, int64_t m0, int64_t n0, f32x16 (&acc)[4][4],
                                         TPS_LDS char* smem) {
  constexpr bool A_KC = LAYOUT != L_TN;
  constexpr bool B_KC = LAYOUT == L_NT;
  const int wave = threadIdx.x >> 6, wm = wave >> 1, wn = wave & 1;
  const bool dual = (LAYOUT == L_NN) && (P.epi == E_SWIGLU);
  const int nk0 = (int)((P.seg[0].K + BK - 1) / BK);
  const int nk = nk0 + (P.nseg > 1 ? (int)((P.seg[1].K + BK - 1) / BK) : 0);

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{0.f};

  u32x4 ra[8], rb[8];
  auto gload = [&](int kt) {
    const bool s1 = kt >= nk0;
    const Seg& S = s1 ? P.seg[1] : P.seg[0];
    const int64_t k0 = (int64_t)(s1 ? kt - nk0 : kt) * BK;
    const uint16_t* a = static_cast<const uint16_t*>(S.a);
    const uint16_t* b = static_cast<const uint16_t*>(S.b);
    if (A_KC) load_kc(ra, a, S.lda, P.M, m0, S.K, k0);
    else load_mn(ra, a, S.lda, P.M, m0, S.K, k0);
    if (B_KC) load_kc(rb, b, S.ldb, P.N, n0, S.K, k0);
    else if (dual) load_mn_dual(rb, b, static_cast<const uint16_t*>(P.b_up), S.ldb, P.ldb_up, P.N, n0, S.K, k0);
    else load_mn(rb, b, S.ldb, P.N, n0, S.K, k0);
  };
  auto swrite = [&](int buf) {
    TPS_LDS char* as = smem + buf * BUF_BYTES;
    TPS_LDS char* bs = as + TILE_BYTES;
    if (A_KC) store_kc(as, ra); else store_mn(as, ra);
    if (B_KC) store_kc(bs, rb); else store_mn(bs, rb);
  };
  auto compute = [&](int buf) {
    const TPS_LDS char* as = smem + buf * BUF_BYTES;
    const TPS_LDS char* bs = as + TILE_BYTES;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8 af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = A_KC ? frag_kc(as, 128 * wm + 32 * i, kk) : frag_mn(as, 128 * wm + 32 * i, kk);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int bc = dual ? ((j & 2) ? 128 : 0) + 64 * wn + 32 * (j & 1) : 128 * wn + 32 * j;
        bfr[j] = B_KC ? frag_kc(bs, bc, kk) : frag_mn(bs, bc, kk);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
    }
  };

  gload(0);
  swrite(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    compute(buf);
    if (kt + 1 < nk) swrite(buf ^ 1);
    __syncthreads();
  }
}

// ---- GEMM epilogue -------------------------------------------------------------------
// The accumulators leave through LDS one 32-row slice at a time: each wave
// parks its 32 x 128 fp32 slice in a private LDS region, then each lane
// finishes 8 consecutive output columns per step (bias, activation, bf16
// rounding) and writes them with 16-byte stores.  SwiGLU waves hold
// [64 gate | 64 up] columns, so a lane pairs staged columns c and 64 + c.
constexpr int EPI_LD = 132;                      // floats per staged row (128 + 4 padding)
constexpr int EPI_WAVE_FLOATS = 32 * EPI_LD;     // 16.5 KiB per wave

__device__ __forceinline__ void stage_block(TPS_LDS float* w, const f32x16& a, int j) {
  const int lane = threadIdx.x & 63;
  TPS_LDS float* p = w + (lane & 31) * EPI_LD + 32 * j + 4 * (lane >> 5);
#pragma unroll
  for (int r4 = 0; r4 < 4; ++r4)
    *reinterpret_cast<TPS_LDS f32x4*>(p + 8 * r4) = f32x4{a[4 * r4], a[4 * r4 + 1], a[4 * r4 + 2], a[4 * r4 + 3]};
}

__device__ __forceinline__ void store8_bf16(uint16_t* p, const float (&v)[8], int nv) {
  if (nv == 8 && ((reinterpret_cast<uintptr_t>(p) & 15) == 0)) {
    u32x4 w = {pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]), pack_bf2(v[4], v[5]), pack_bf2(v[6], v[7])};
    *reinterpret_cast<u32x4*>(p) = w;
  } else {
    for (int e = 0; e < nv; ++e) p[e] = f2bf(v[e]);
  }
}

// Finish output columns [n, n + nv) of row m (nv <= 8).
__device__ __forceinline__ void epi8(const Problem& P, int64_t m, int64_t n, int nv, float (&v)[8], float (&u)[8]) {
  if (P.bias) {
    const uint16_t* b = static_cast<const uint16_t*>(P.bias) + n;
    for (int e = 0; e < nv; ++e) v[e] += bf2f(b[e]);
  }
  uint16_t* c = static_cast<uint16_t*>(P.c) + m * P.ldc + n;
  if (P.epi == E_STORE) {
    store8_bf16(c, v, nv);
  } else if (P.epi == E_GELU) {
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = gelu_f(v[e]);
    store8_bf16(static_cast<uint16_t*>(P.pre) + m * P.ldpre + n, v, nv);
    store8_bf16(c, y, nv);
  } else {
    if (P.bias2) {
      const uint16_t* b = static_cast<const uint16_t*>(P.bias2) + n;
      for (int e = 0; e < nv; ++e) u[e] += bf2f(b[e]);
    }
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = silu_f(v[e]) * u[e];
    uint16_t* pre = static_cast<uint16_t*>(P.pre) + m * P.ldpre;
    store8_bf16(pre + n, v, nv);
    store8_bf16(pre + P.N + n, u, nv);
    store8_bf16(c, y, nv);
  }
}

// Store the staged 32-row slice i of this wave.
__device__ __forceinline__ void store_slice(const Problem& P, const TPS_LDS float* w, int64_t m0, int64_t n0, int i) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wm = wave >> 1, wn = wave & 1;
  const bool dual = P.epi == E_SWIGLU;
  const int chunks = dual ? 8 : 16;             // 8-column chunks per staged row
  const int64_t mrow = m0 + 128 * wm + 32 * i;
  const int64_t ncol = n0 + (dual ? 64 * wn : 128 * wn);
  for (int idx = lane; idx < 32 * chunks; idx += 64) {
    const int row = idx / chunks, c8 = idx % chunks;
    const int64_t m = mrow + row, n = ncol + 8 * c8;
    if (m >= P.M || n >= P.N) continue;
    const int nv = (int)min<int64_t>(8, P.N - n);
    const TPS_LDS float* src = w + row * EPI_LD + 8 * c8;
    float v[8], u[8];
    const f32x4 v0 = *reinterpret_cast<const TPS_LDS f32x4*>(src);
    const f32x4 v1 = *reinterpret_cast<const TPS_LDS f32x4*>(src + 4);
    f32x4 u0 = {0.f, 0.f, 0.f, 0.f}, u1 = u0;
    if (dual) {
      u0 = *reinterpret_cast<const TPS_LDS f32x4*>(src + 64);
      u1 = *reinterpret_cast<const TPS_LDS f32x4*>(src + 68);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = v0[e];
      v[4 + e] = v1[e];
      u[e] = u0[e];
      u[4 + e] = u1[e];
    }
    epi8(P, m, n, nv, v, u);
  }
}

__device__ __forceinline__ void epilogue(const Problem& P, int64_t m0, int64_t n0, f32x16 (&acc)[4][4],
                                         TPS_LDS char* smem) {
  TPS_LDS float* w = reinterpret_cast<TPS_LDS float*>(smem) + (threadIdx.x >> 6) * EPI_WAVE_FLOATS;
#pragma unroll 1
  for (int i = 0; i < 4; ++i) {
    switch (i) {   // constant indices into acc keep it in registers
      case 0: for (int j = 0; j < 4; ++j) stage_block(w, acc[0][j], j); break;
      case 1: for (int j = 0; j < 4; ++j) stage_block(w, acc[1][j], j); break;
      case 2: for (int j = 0; j < 4; ++j) stage_block(w, acc[2][j], j); break;
      default: for (int j = 0; j < 4; ++j) stage_block(w, acc[3][j], j); break;
    }
    __syncthreads();
    store_slice(P, w, m0, n0, i);
    __syncthreads();
  }
}

// Per-field selection of one of the launch's problems (uniform across the
// workgroup); a runtime index into the kernel-argument array would make the
// compiler copy the whole array to scratch.
__device__ __forceinline__ Problem pick_problem(const GemmLaunch& L, bool s) {
  Problem P;
#define TPS_PICK(f) P.f = s ? L.p[1].f : L.p[0].f
  TPS_PICK(M); TPS_PICK(N);
  TPS_PICK(seg[0].a); TPS_PICK(seg[0].b); TPS_PICK(seg[0].lda); TPS_PICK(seg[0].ldb); TPS_PICK(seg[0].K);
  TPS_PICK(seg[1].a); TPS_PICK(seg[1].b); TPS_PICK(seg[1].lda); TPS_PICK(seg[1].ldb); TPS_PICK(seg[1].K);
  TPS_PICK(nseg); TPS_PICK(layout); TPS_PICK(epi); TPS_PICK(b_up); TPS_PICK(ldb_up);
  TPS_PICK(bias); TPS_PICK(bias2); TPS_PICK(c); TPS_PICK(ldc); TPS_PICK(pre); TPS_PICK(ldpre);
  TPS_PICK(tiles_m); TPS_PICK(tiles_n); TPS_PICK(tile_begin);
#undef TPS_PICK
  return P;
}

// One kernel per (operand layout, epilogue) pair, so each role of the shard
// path is a distinct kernel in traces and gets its own specialised epilogue.
template <int LAYOUT, int EPI>
__global__ __launch_bounds__(NTHREADS, 1) void gemm_bf16_kernel(const GemmLaunch L, int total_tiles) {
  __shared__ __attribute__((aligned(16))) char smem_raw[LDS_BYTES];
  TPS_LDS char* smem = (TPS_LDS char*)smem_raw;
  const int id = xcd_remap(blockIdx.x, total_tiles);
  Problem P = pick_problem(L, L.nprob > 1 && id >= L.p[1].tile_begin);
  P.epi = EPI;
  int tm, tn;
  tile_coords(id - P.tile_begin, P.tiles_m, P.tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM;
  const int64_t n0 = (int64_t)tn * (EPI == E_SWIGLU ? BN / 2 : BN);
  f32x16 acc[4][4];
  mainloop<LAYOUT>(P, m0, n0, acc, smem);
  epilogue(P, m0, n0, acc, smem);
}

// Row statistics of one 32-row slice (I) of a wave's 128 x 128 logit block:
// max and sum exp(z - max) over the valid columns, the target logit if this
// lane holds it, and the per-wave results in LDS for the cross-wave merge.
template <int I>
__device__ __forceinline__ void ce_rows(const CEArgs& a, f32x16 (&acc)[4][4], int64_t m0, int64_t wcol,
                                        int nvalid, float* ws_tgt, TPS_LDS float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5;
  const int rl = 128 * wm + 32 * I + (lane & 31);
  const int64_t m = m0 + rl;
  const int lim = nvalid - 4 * h;     // column c = 32j + 8(r/4) + (r%4) of this lane is valid iff c < lim
  float mx = -INFINITY;
  if (nvalid >= 128) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc[I][j][r]);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int c = 32 * j + 8 * (r >> 2) + (r & 3);
        mx = fmaxf(mx, c < lim ? acc[I][j][r] : -INFINITY);
      }
  }
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  float s = 0.f;
  if (nvalid >= 128) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) s += __expf(acc[I][j][r] - mx);
  } else if (mx > -INFINITY) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int c = 32 * j + 8 * (r >> 2) + (r & 3);
        s += c < lim ? __expf(acc[I][j][r] - mx) : 0.f;
      }
  }
  s += __shfl_xor(s, 32);
  if (m < a.M) {
    const int64_t d64 = (int64_t)a.target[m] - a.v0 - wcol;   // target column relative to the wave
    if (d64 >= 0 && d64 < nvalid) {
      const int dd = (int)d64 - 4 * h;
      float tv = 0.f;
      bool mine = false;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const bool hit = (32 * j + 8 * (r >> 2) + (r & 3)) == dd;
          tv = hit ? acc[I][j][r] : tv;
          mine = mine || hit;
        }
      if (mine) ws_tgt[m] = tv;
    }
  }
  if (h == 0) {
    red[(wn * 256 + rl) * 2 + 0] = mx;
    red[(wn * 256 + rl) * 2 + 1] = s;
  }
}

template <int... Is>
__device__ __forceinline__ void ce_rows_seq(const CEArgs& a, f32x16 (&acc)[4][4], int64_t m0, int64_t wcol,
                                            int nvalid, float* ws_tgt, TPS_LDS float* red,
                                            std::integer_sequence<int, Is...>) {
  (ce_rows<Is>(a, acc, m0, wcol, nvalid, ws_tgt, red), ...);
}

// ---- vocab-parallel LM head: logits tile -> (max, sum exp) partials ---------------------
// Tile (tm, tn) covers tokens [m0, m0+256) and shard vocab columns
// [n0, n0+256).  Writes ws_ms[tn][m] = (tile max, sum exp(z - tile max)) and,
// for the tile holding a token's target, ws_tgt[m] = z[m, target - v0].
__global__ __launch_bounds__(NTHREADS, 1) void ce_tile_kernel(const CEArgs a, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(16))) char smem_raw[LDS_BYTES];
  TPS_LDS char* smem = (TPS_LDS char*)smem_raw;
  const int id = xcd_remap(blockIdx.x, tiles_m * tiles_n);
  int tm, tn;
  tile_coords(id, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  Problem P = {};
  P.M = a.M;
  P.N = a.Vr;
  P.seg[0] = Seg{a.H, a.W, a.ldh, a.ldw, a.K};
  P.nseg = 1;
  P.layout = L_NT;
  P.epi = E_STORE;
  f32x16 acc[4][4];
  mainloop<L_NT>(P, m0, n0, acc, smem);

  const int wn = (threadIdx.x >> 6) & 1;
  const int64_t wcol = n0 + 128 * wn;                 // first column of this wave
  // number of valid columns of this wave, in [0, 128]
  const int nvalid = (int)max<int64_t>(0, min<int64_t>(128, a.Vr - wcol));
  float* ws_ms = a.ws;
  float* ws_tgt = a.ws + 2 * (int64_t)tiles_n * a.M;
  TPS_LDS float* red = (TPS_LDS float*)smem;          // [2][256][2]; the main loop ended on a barrier
  ce_rows_seq(a, acc, m0, wcol, nvalid, ws_tgt, red, std::make_integer_sequence<int, 4>{});
  __syncthreads();
  const int rl = threadIdx.x;
  const int64_t m = m0 + rl;
  if (m < a.M) {
    const float ma = red[rl * 2], sa = red[rl * 2 + 1];
    const float mb = red[(256 + rl) * 2], sb = red[(256 + rl) * 2 + 1];
    const float mm = fmaxf(ma, mb);
    const float ss = sa * __expf(ma - mm) + sb * __expf(mb - mm);
    ws_ms[2 * ((int64_t)tn * a.M + m) + 0] = mm;
    ws_ms[2 * ((int64_t)tn * a.M + m) + 1] = ss;
  }
}

// Combine the per-tile partials of each token in ascending tile order.
__global__ __launch_bounds__(256) void ce_merge_kernel(const CEArgs a, int tiles_n) {
  const int64_t m = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (m >= a.M) return;
  const float* ws_ms = a.ws;
  const float* ws_tgt = a.ws + 2 * (int64_t)tiles_n * a.M;
  float mm = ws_ms[2 * m], ss = ws_ms[2 * m + 1];
  for (int t = 1; t < tiles_n; ++t) {
    const float mt = ws_ms[2 * ((int64_t)t * a.M + m)], st = ws_ms[2 * ((int64_t)t * a.M + m) + 1];
    const float mn = fmaxf(mm, mt);
    ss = ss * __expf(mm - mn) + st * __expf(mt - mn);
    mm = mn;
  }
  const int64_t tg = (int64_t)a.target[m] - a.v0;
  a.out_max[m] = mm;
  a.out_sumexp[m] = ss;
  a.out_tgt[m] = (tg >= 0 && tg < a.Vr) ? ws_tgt[m] : 0.f;
}

}  // namespace

hipError_t launch_gemm_bf16(GemmLaunch& L, hipStream_t s) {
  // Problems of one launch must share the operand layout and the epilogue;
  // otherwise split.  Only L_NN carries activation epilogues.
  if (L.nprob > 1 && (L.p[0].layout != L.p[1].layout || L.p[0].epi != L.p[1].epi)) {
    GemmLaunch a = L, b = L;
    a.nprob = 1;
    b.p[0] = L.p[1];
    b.nprob = 1;
    hipError_t e = launch_gemm_bf16(a, s);
    return e != hipSuccess ? e : launch_gemm_bf16(b, s);
  }
  int total = 0;
  for (int i = 0; i < L.nprob; ++i) {
    Problem& P = L.p[i];
    const int64_t bn = (P.epi == E_SWIGLU) ? BN / 2 : BN;
    P.tiles_m = (int)((P.M + BM - 1) / BM);
    P.tiles_n = (int)((P.N + bn - 1) / bn);
    P.tile_begin = total;
    total += P.tiles_m * P.tiles_n;
  }
  if (total == 0) return hipSuccess;
  const dim3 grid(total), block(NTHREADS);
  const int layout = L.p[0].layout, epi = L.p[0].epi;
  if (layout == L_NN && epi == E_SWIGLU) hipLaunchKernelGGL((gemm_bf16_kernel<L_NN, E_SWIGLU>), grid, block, 0, s, L, total);
  else if (layout == L_NN && epi == E_GELU) hipLaunchKernelGGL((gemm_bf16_kernel<L_NN, E_GELU>), grid, block, 0, s, L, total);
  else if (layout == L_NN) hipLaunchKernelGGL((gemm_bf16_kernel<L_NN, E_STORE>), grid, block, 0, s, L, total);
  else if (layout == L_NT) hipLaunchKernelGGL((gemm_bf16_kernel<L_NT, E_STORE>), grid, block, 0, s, L, total);
  else hipLaunchKernelGGL((gemm_bf16_kernel<L_TN, E_STORE>), grid, block, 0, s, L, total);
  return hipGetLastError();
}

size_t ce_workspace_bytes(int64_t M, int64_t Vr) {
  const int64_t tiles_n = (Vr + BN - 1) / BN;
  return (size_t)(2 * tiles_n * M + M) * sizeof(float);
}

hipError_t launch_ce_partials(const CEArgs& a, hipStream_t s) {
  const int tiles_m = (int)((a.M + BM - 1) / BM);
  const int tiles_n = (int)((a.Vr + BN - 1) / BN);
  hipLaunchKernelGGL(ce_tile_kernel, dim3(tiles_m * tiles_n), dim3(NTHREADS), 0, s, a, tiles_m, tiles_n);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(ce_merge_kernel, dim3((unsigned)((a.M + 255) / 256)), dim3(256), 0, s, a, tiles_n);
  return hipGetLastError();
}

}  // namespace tps
