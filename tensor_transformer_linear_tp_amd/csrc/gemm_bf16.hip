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
constexpr int GROUP_M = 8;                    // tile rows per L2 group

// ---- LDS address maps ------------------------------------------------------
// K-contiguous [256][64]: 128-byte rows, 8 chunks of 16 bytes each.
__device__ __forceinline__ int kc_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int kc_off(int r, int c) { return r * 128 + ((c ^ kc_swz(r)) << 4); }
// MN-contiguous [64][W]: rows of W bf16 (512 or 256 bytes); rows k%4 = 0,1,2,3
// XOR the chunk index with 0, 6, 10, 12.
__device__ __forceinline__ int mn_swz(int k) { return (0xCA60 >> ((k & 3) * 4)) & 15; }
template <int ROWB>
__device__ __forceinline__ int mn_off(int k, int c) { return k * ROWB + ((c ^ mn_swz(k)) << 4); }

// ---- global -> LDS streaming ---------------------------------------------------
// Each operand stage (32 KiB) is copied by 32 wave-level buffer_load_dwordx4
// ... lds instructions, 8 per wave; each writes 1 KiB of LDS contiguously in
// lane order, so a lane's global address is chosen to land its 16 bytes at
// the swizzled position.  Reads past the operand's extent return zero (the
// buffer descriptor's range), which zero-fills rows beyond M/N and, for
// MN-contiguous operands, rows beyond K.  The K tail of K-contiguous operands
// lies inside the extent and is zeroed in LDS afterwards (kc_zero_tail).
struct OpStream {
  const char* base;   // stage-0 origin of this wave's operand (bytes), wave-uniform
  int64_t remain;     // bytes from base to the end of the operand's extent
  int64_t step;       // bytes between K stages
  uint32_t voff[8];   // per-lane byte offsets of this wave's 8 blocks
  int lds_off;        // byte offset of this wave's first block inside the tile
  int lds_stride;     // bytes between this wave's blocks
};

__device__ __forceinline__ int64_t extent_bytes(int64_t rows, int64_t ld, int64_t width) {
  return ((rows - 1) * ld + ((width + 7) & ~int64_t(7))) * 2;
}

// K-contiguous operand: tile rows [row0, row0+256) of a [rows][K] matrix.
__device__ __forceinline__ OpStream stream_kc(const void* p, int64_t ld, int64_t rows, int64_t K, int64_t row0,
                                              int wave) {
  const int lane = threadIdx.x & 63;
  OpStream s;
  s.base = static_cast<const char*>(p) + row0 * ld * 2;
  s.remain = extent_bytes(rows, ld, K) - row0 * ld * 2;
  s.step = BK * 2;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int b = 8 * wave + j;                      // block: rows 8b .. 8b+7
    const int r = 8 * b + (lane >> 3);
    const int c = (lane & 7) ^ kc_swz(r);            // logical chunk stored at physical slot lane&7
    s.voff[j] = (uint32_t)((r * ld + 8 * c) * 2);
  }
  s.lds_off = 8 * wave * 1024;
  s.lds_stride = 1024;
  return s;
}

// MN-contiguous operand: columns [col0, col0 + W) of a [K][cols] matrix,
// W = 256 (512-byte rows, 2 rows per block) or 128 (256-byte rows, 4 rows
// per block; `sub` selects which 16 KiB half of the tile this wave fills).
template <int W>
__device__ __forceinline__ OpStream stream_mn(const void* p, int64_t ld, int64_t cols, int64_t K, int64_t col0,
                                              int wave) {
  const int lane = threadIdx.x & 63;
  constexpr int ROWS_PER_BLOCK = 1024 / (W * 2);
  constexpr int CHUNKS = W / 8;
  OpStream s;
  s.base = static_cast<const char*>(p) + col0 * 2;
  s.remain = extent_bytes(K, ld, cols) - col0 * 2;
  s.step = (int64_t)BK * ld * 2;
  const int wb = (W == 256) ? wave : (wave & 1);     // W = 128: waves {0,1} and {2,3} fill the two halves
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int b = 8 * wb + j;
    const int k = ROWS_PER_BLOCK * b + lane / CHUNKS;
    const int c = (lane % CHUNKS) ^ mn_swz(k);
    s.voff[j] = (uint32_t)((k * ld + 8 * c) * 2);
  }
  s.lds_off = (W == 256) ? 8 * wave * 1024 : (wave >> 1) * 16384 + 8 * wb * 1024;
  s.lds_stride = 1024;
  return s;
}

// Zero k >= kvalid (0 < kvalid < 64) of a K-contiguous [256][64] LDS tile.
__device__ __forceinline__ void kc_zero_tail(TPS_LDS char* tile, int kvalid) {
  const int t = threadIdx.x;
  const int c = t & 7;
  if (8 * c + 8 <= kvalid) return;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = (t >> 3) + 32 * i;
    TPS_LDS u32x4* q = reinterpret_cast<TPS_LDS u32x4*>(tile + kc_off(r, c));
    u32x4 v = *q;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int e0 = 8 * c + 2 * w;
      const uint32_t keep = (e0 + 1 < kvalid) ? 0xffffffffu : (e0 < kvalid ? 0x0000ffffu : 0u);
      v[w] &= keep;
    }
    *q = v;
  }
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
template <int ROWB>
__device__ __forceinline__ bf16x8 frag_mn(const TPS_LDS char* s, int cb, int kk) {
  const int lane = threadIdx.x & 63;
  const int h = lane >> 4, q = lane & 15;
  const int col = cb + 16 * (h & 1) + 4 * (q & 3);
  const int k0 = 16 * kk + 8 * (h >> 1) + (q >> 2);
  const int c = col >> 3, byte_in = (col & 7) * 2;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (TPS_LDS i16x4*)(s + mn_off<ROWB>(k0, c) + byte_in));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (TPS_LDS i16x4*)(s + mn_off<ROWB>(k0 + 4, c) + byte_in));
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
// Two LDS stages held in two distinct __shared__ arrays: while the MFMAs
// consume one stage, the copy engine fills the other.  Because the arrays
// are distinct objects, the compiler can see that reads of one stage do not
// depend on copies into the other and adds no wait for them; the barrier at
// the top of each step (with its vmcnt(0)) makes the step's stage complete
// and visible.  The loop is unrolled by two so each step's stage is static.
template <int LAYOUT, bool DUAL>
struct MainLoop {
  static constexpr bool A_KC = LAYOUT != L_TN;
  static constexpr bool B_KC = LAYOUT == L_NT;

  const Problem& P;
  int64_t m0, n0;
  TPS_LDS char* lds0;
  TPS_LDS char* lds1;
  int wave, wm, wn;
  OpStream sa[2], sb[2];   // per K segment
  int nk0, nk;

  __device__ __forceinline__ void open_segment(int s) {
    // Field-wise selection keeps the problem description in registers.
    const void* pa = s ? P.seg[1].a : P.seg[0].a;
    const void* pb = s ? P.seg[1].b : P.seg[0].b;
    const int64_t lda = s ? P.seg[1].lda : P.seg[0].lda;
    const int64_t ldb = s ? P.seg[1].ldb : P.seg[0].ldb;
    const int64_t K = s ? P.seg[1].K : P.seg[0].K;
    sa[s] = A_KC ? stream_kc(pa, lda, P.M, K, m0, wave) : stream_mn<256>(pa, lda, P.M, K, m0, wave);
    if (B_KC) {
      sb[s] = stream_kc(pb, ldb, P.N, K, n0, wave);
    } else if (DUAL) {   // waves 0,1 stream the gate weight, waves 2,3 the up weight
      const bool up = (wave >> 1) != 0;
      sb[s] = stream_mn<128>(up ? P.b_up : pb, up ? P.ldb_up : ldb, P.N, K, n0, wave);
    } else {
      sb[s] = stream_mn<256>(pb, ldb, P.N, K, n0, wave);
    }
  }

  // Issue the copies of global K stage kt into `dst`; a stage past the end
  // is issued with an empty range (no memory is read, zeros are written).
  __device__ __forceinline__ void issue(int kt, TPS_LDS char* dst) {
    const bool s1 = kt >= nk0;
    const int stage = s1 ? kt - nk0 : kt;
    const bool live = kt < nk;
    issue_one(s1, sa, stage, live, dst);
    issue_one(s1, sb, stage, live, dst + TILE_BYTES);
  }

  static __device__ __forceinline__ void issue_one(bool s1, const OpStream (&st)[2], int stage, bool live,
                                                   TPS_LDS char* tile) {
    const char* base = s1 ? st[1].base : st[0].base;
    const int64_t step = s1 ? st[1].step : st[0].step;
    const int64_t remain = s1 ? st[1].remain : st[0].remain;
    const int64_t off = (int64_t)stage * step;
    const int64_t rem = live ? remain - off : 0;
    const uint32_t nrec = rem <= 0 ? 0u : (rem >= 0xffffffffll ? 0xffffffffu : (uint32_t)rem);
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base + off), (short)0, (int)nrec, 0x00020000);
    const int lds_off = st[0].lds_off;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t v = s1 ? st[1].voff[j] : st[0].voff[j];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (TPS_LDS void*)(tile + lds_off + j * 1024), 16, v, 0, 0, 0);
    }
  }

  // Per-lane LDS byte addresses of the fragments, computed once.  A fragment
  // read is then addr + a compile-time offset (K sub-step, block), which the
  // ds_read instruction's offset field absorbs.
  //   K-contiguous operand: one base per 16-deep K sub-step (the swizzle
  //   mixes k into the chunk index); blocks are +32 rows = +4096 bytes.
  //   MN-contiguous operand: one base per 32-wide block (the swizzle mixes
  //   the column into the chunk index); K sub-steps are +16 rows.
  int adA[4], adB[4];

  __device__ __forceinline__ void init_frag_addr() {
    const int lane = threadIdx.x & 63;
    const int h = lane >> 4, q = lane & 15, hi32 = lane >> 5;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      if (A_KC) {
        const int r = 128 * wm + (lane & 31);
        adA[x] = kc_off(r, 2 * x + hi32);
      } else {
        const int col = 128 * wm + 32 * x + 16 * (h & 1) + 4 * (q & 3);
        const int k = 8 * (h >> 1) + (q >> 2);
        adA[x] = mn_off<512>(k, col >> 3) + (col & 7) * 2;
      }
      if (B_KC) {
        const int r = 128 * wn + (lane & 31);
        adB[x] = TILE_BYTES + kc_off(r, 2 * x + hi32);
      } else if (DUAL) {
        const int col = 64 * wn + 32 * (x & 1) + 16 * (h & 1) + 4 * (q & 3);
        const int k = 8 * (h >> 1) + (q >> 2);
        adB[x] = TILE_BYTES + (x >> 1) * 16384 + mn_off<256>(k, col >> 3) + (col & 7) * 2;
      } else {
        const int col = 128 * wn + 32 * x + 16 * (h & 1) + 4 * (q & 3);
        const int k = 8 * (h >> 1) + (q >> 2);
        adB[x] = TILE_BYTES + mn_off<512>(k, col >> 3) + (col & 7) * 2;
      }
    }
  }

  static __device__ __forceinline__ bf16x8 rd_kc(const TPS_LDS char* p) {
    return *reinterpret_cast<const TPS_LDS bf16x8*>(p);
  }
  static __device__ __forceinline__ bf16x8 rd_mn(const TPS_LDS char* p, int rowb) {
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((TPS_LDS i16x4*)p);
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((TPS_LDS i16x4*)(p + 4 * rowb));
    typedef __attribute__((ext_vector_type(8))) short i16x8;
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }

  // Fragment register sets: sub-step kk of a stage lives in set kk & 1.
  bf16x8 af[2][4], bfr[2][4];

  __device__ __forceinline__ void load(const TPS_LDS char* base, int kk, int r) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      af[r][i] = A_KC ? rd_kc(base + adA[kk] + 4096 * i) : rd_mn(base + adA[i] + 16 * kk * 512, 512);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (B_KC) bfr[r][j] = rd_kc(base + adB[kk] + 4096 * j);
      else if (DUAL) bfr[r][j] = rd_mn(base + adB[j] + 16 * kk * 256, 256);
      else bfr[r][j] = rd_mn(base + adB[j] + 16 * kk * 512, 512);
    }
  }

  __device__ __forceinline__ void mma(int r, f32x16 (&acc)[4][4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[r][j], af[r][i], acc[i][j], 0, 0, 0);
  }

  // Ask the scheduler to alternate one MFMA with one LDS read (and, in the
  // first phase of a step, one global->LDS copy), instead of loading each
  // fragment just before its first use.
  static constexpr int READS = (A_KC ? 4 : 8) + (B_KC ? 4 : 8);
  static __device__ __forceinline__ void interleave(bool with_copies) {
#pragma unroll
    for (int g = 0; g < 16; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // MFMA
      if (g < READS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
      if (with_copies) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0); // VMEM read
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // One 64-deep K step on the stage in `cur`, prefetching stage kt+1 into
  // `nxt`.  Software pipeline: the MFMAs of the previous stage's last
  // sub-step (operands already in registers, set 1) run after the barrier,
  // covering the latency of this stage's first fragment reads.
  __device__ __forceinline__ void step(int kt, TPS_LDS char* cur, TPS_LDS char* nxt, f32x16 (&acc)[4][4]) {
    __syncthreads();                                   // stage kt landed everywhere; stage kt-1 fully read
    const bool s1 = kt >= nk0;
    const int64_t kseg = s1 ? P.seg[1].K : P.seg[0].K;
    const int64_t k0 = (int64_t)(s1 ? kt - nk0 : kt) * BK;
    if ((A_KC || B_KC) && k0 + BK > kseg) {            // K tail of K-contiguous operands
      if (A_KC) kc_zero_tail(cur, (int)(kseg - k0));
      if (B_KC) kc_zero_tail(cur + TILE_BYTES, (int)(kseg - k0));
      __syncthreads();
    }
    __builtin_amdgcn_sched_barrier(0);
    issue(kt + 1, nxt);
    load(cur, 0, 0);
    mma(1, acc);              // previous stage, sub-step 3
    interleave(true);
    load(cur, 1, 1);
    mma(0, acc);
    interleave(false);
    load(cur, 2, 0);
    mma(1, acc);
    interleave(false);
    load(cur, 3, 1);
    mma(0, acc);
    interleave(false);
  }

  __device__ __forceinline__ void run(f32x16 (&acc)[4][4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{0.f};
      af[1][i] = bf16x8{};      // the first step's deferred sub-step multiplies zeros
      bfr[1][i] = bf16x8{};
    }
    wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    wm = wave >> 1;
    wn = wave & 1;
    nk0 = (int)((P.seg[0].K + BK - 1) / BK);
    nk = nk0 + (P.nseg > 1 ? (int)((P.seg[1].K + BK - 1) / BK) : 0);
    init_frag_addr();
    open_segment(0);
    if (P.nseg > 1) open_segment(1);
    else sa[1] = sa[0], sb[1] = sb[0];
    issue(0, lds0);
    int kt = 0;
    for (; kt + 1 < nk; kt += 2) {
      step(kt, lds0, lds1, acc);
      step(kt + 1, lds1, lds0, acc);
    }
    if (kt < nk) step(kt, lds0, lds1, acc);
    mma(1, acc);              // last stage, sub-step 3
    __syncthreads();          // LDS is reused by the epilogue
  }
};

template <int LAYOUT>
__device__ __forceinline__ void mainloop(const Problem& P, int64_t m0, int64_t n0, f32x16 (&acc)[4][4],
                                         TPS_LDS char* lds0, TPS_LDS char* lds1) {
  if (LAYOUT == L_NN && P.epi == E_SWIGLU) {
    MainLoop<L_NN, true> ml{P, m0, n0, lds0, lds1};
    ml.run(acc);
  } else {
    MainLoop<LAYOUT, false> ml{P, m0, n0, lds0, lds1};
    ml.run(acc);
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
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (e < nv) p[e] = f2bf(v[e]);
  }
}

// Finish output columns [n, n + nv) of row m (nv <= 8).
__device__ __forceinline__ void epi8(const Problem& P, int64_t m, int64_t n, int nv, float (&v)[8], float (&u)[8]) {
  if (P.bias) {
    const uint16_t* b = static_cast<const uint16_t*>(P.bias) + n;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (e < nv) v[e] += bf2f(b[e]);
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
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (e < nv) u[e] += bf2f(b[e]);
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
                                         TPS_LDS char* lds0, TPS_LDS char* lds1) {
  const int wave = threadIdx.x >> 6;   // waves 0,1 stage in the first array, 2,3 in the second
  TPS_LDS float* w = reinterpret_cast<TPS_LDS float*>(wave < 2 ? lds0 : lds1) + (wave & 1) * EPI_WAVE_FLOATS;
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
  __shared__ __attribute__((aligned(16))) char lds_a[BUF_BYTES];
  __shared__ __attribute__((aligned(16))) char lds_b[BUF_BYTES];
  TPS_LDS char* lds0 = (TPS_LDS char*)lds_a;
  TPS_LDS char* lds1 = (TPS_LDS char*)lds_b;
  const int id = xcd_remap(blockIdx.x, total_tiles);
  Problem P = pick_problem(L, L.nprob > 1 && id >= L.p[1].tile_begin);
  P.epi = EPI;
  int tm, tn;
  tile_coords(id - P.tile_begin, P.tiles_m, P.tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM;
  const int64_t n0 = (int64_t)tn * (EPI == E_SWIGLU ? BN / 2 : BN);
  f32x16 acc[4][4];
  mainloop<LAYOUT>(P, m0, n0, acc, lds0, lds1);
  epilogue(P, m0, n0, acc, lds0, lds1);
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
  __shared__ __attribute__((aligned(16))) char lds_a[BUF_BYTES];
  __shared__ __attribute__((aligned(16))) char lds_b[BUF_BYTES];
  TPS_LDS char* lds0 = (TPS_LDS char*)lds_a;
  TPS_LDS char* lds1 = (TPS_LDS char*)lds_b;
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
  mainloop<L_NT>(P, m0, n0, acc, lds0, lds1);

  const int wn = (threadIdx.x >> 6) & 1;
  const int64_t wcol = n0 + 128 * wn;                 // first column of this wave
  // number of valid columns of this wave, in [0, 128]
  const int nvalid = (int)max<int64_t>(0, min<int64_t>(128, a.Vr - wcol));
  float* ws_ms = a.ws;
  float* ws_tgt = a.ws + 2 * (int64_t)tiles_n * a.M;
  TPS_LDS float* red = (TPS_LDS float*)lds0;          // [2][256][2]; the main loop ended on a barrier
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
