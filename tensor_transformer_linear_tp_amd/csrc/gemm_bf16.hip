// bf16 GEMM family for gfx950 (MI355X): C = A B with fp32 accumulation on
// v_mfma_f32_16x16x32_bf16, a 4-stage LDS ring filled by direct-to-LDS buffer
// loads, and fused epilogues; plus the vocab-parallel LM-head kernel whose
// epilogue reduces logit tiles to (max, sum exp) partials without writing the
// logits.
//
// Tiling: a 256-thread workgroup (4 wave64s as 2 x 2) owns a 256 x 256 output
// tile (SwiGLU: 256 rows x (128 gate + 128 up) columns); each wave owns
// 128 x 128 = 8 x 8 MFMA blocks of 16 x 16.  K advances 32 per LDS stage,
// one MFMA deep.  (The 16 x 16 x 32 instruction does the same work as the
// 32 x 32 x 16 one at a lower power per FLOP: with random operands held in
// registers the chip sustains a ~16 % higher clock under its power limit.)
//
// LDS layouts.  Operands are copied global -> LDS in their global orientation:
//   * K-contiguous operand (A of NN/NT, B of NT): [256 rows][32 k], read as
//     MFMA fragments with one ds_read_b128 per lane;
//   * MN-contiguous operand (A of TN, B of NN/TN): [32 k][256 cols], read
//     with two ds_read_b64_tr_b16 per lane, which transposes 16-bit elements
//     across each 16-lane group on the way out of LDS.
// Both use an XOR swizzle of the 16-byte chunk index so that fragment reads
// fall into distinct banks.
//
// Accumulator orientation.  The MFMA is issued as (B fragment, A fragment),
// so in each 16 x 16 block a lane holds four consecutive output columns of
// one row: row lane % 16, columns 4 * (lane / 16) .. +3.
#include <algorithm>
#include <climits>
#include <mutex>
#include <utility>

#include "device_common.hpp"
#include "kernels.hpp"

namespace tps {
namespace {

constexpr int BM = 256, BN = 256, BK = 32;
constexpr int NTHREADS = 256;
constexpr int TILE_BYTES = 256 * BK * 2;      // 16 KiB per operand and stage
constexpr int STAGE_BYTES = 2 * TILE_BYTES;   // A + B
constexpr int NSTAGE = 4;                     // LDS ring depth; copies run NSTAGE-1 stages ahead
constexpr int GROUP_M = 8;                    // tile rows per L2 group

// ---- LDS address maps ------------------------------------------------------
// K-contiguous [256][32]: 64-byte rows of 4 chunks of 16 bytes; chunk c of row
// r sits at c ^ kc_swz(r), kc_swz(r) = (r / 2) mod 4.  A fragment read of
// v_mfma_f32_16x16x32_bf16 (ds_read_b128, lane l: row l % 16 of a 16-row
// block, chunk l / 16) with this map measured free of LDS bank conflicts on
// gfx950, like a contiguous read; the map tuned for 32 x 32 fragments (an
// extra flip of chunk bit 0 on rows 8-15) and three other candidates paid
// 0.8 conflict cycles per read.
__device__ __forceinline__ int kc_swz(int r) { return (r >> 1) & 3; }
__device__ __forceinline__ int kc_off(int r, int c) { return r * 64 + ((c ^ kc_swz(r)) << 4); }
// MN-contiguous [32][W]: rows of W bf16 (512 or 256 bytes); row k XORs the
// chunk index with 2 * ((k & 3) | (k & 8) >> 1): a transposing fragment read
// covers 4 consecutive rows in each of two 16-lane groups (rows k..k+3 and
// k+8..k+11, 32 bytes of each), and those 8 rows then hold distinct pairs of
// chunks, all 64 banks once.  Rows k and k + 4 share the swizzle, so the
// second read of a fragment is the first plus 4 rows.
__device__ __forceinline__ int mn_swz(int k) { return 2 * ((k & 3) | ((k & 8) >> 1)); }
template <int ROWB>
__device__ __forceinline__ int mn_off(int k, int c) { return k * ROWB + ((c ^ mn_swz(k)) << 4); }

// The thread index as an opaque value.  The per-tile helpers (copy streams,
// store epilogue) derive per-lane offsets from it; with threadIdx.x itself
// the compiler hoists those out of the tile loop and keeps dozens of them
// live across the K loop, which then spills.  Recomputing them per tile costs
// a few dozen vector instructions.
__device__ __forceinline__ int tid_opaque() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// ---- global -> LDS streaming ---------------------------------------------------
// Each operand stage (16 KiB) is copied by 16 wave-level buffer_load_dwordx4
// ... lds instructions, 4 per wave; each writes 1 KiB of LDS contiguously in
// lane order, so a lane's global address is chosen to land its 16 bytes at
// the swizzled position.  Reads past the operand's extent return zero (the
// buffer descriptor's range), which zero-fills rows beyond M/N and, for
// MN-contiguous operands, rows beyond K.  The K tail of K-contiguous operands
// lies inside the extent and is zeroed in LDS afterwards (kc_zero_tail).
constexpr int DMA_PER_OPERAND = 4;            // copy instructions per wave per operand stage

// Copy stream of one operand of one K segment of one tile: the address of
// the tile's origin, the bytes from there to the end of the operand's extent
// (operands are below 2 GiB, so 32 bits hold every offset), the bytes per K
// stage, and this wave's per-lane byte offsets of its blocks (block j of the
// wave is block 4 w + j of the stage; w = the wave, or for S_MN128 the wave
// within its half).  Everything but the offsets is wave-uniform.
enum StreamKind : int { S_KC = 0, S_MN256 = 1, S_MN128 = 2 };

struct OpStream {
  const char* base;
  uint32_t nrec;
  uint32_t step;
  uint32_t voff[DMA_PER_OPERAND];
};

__device__ __forceinline__ int64_t extent_bytes(int64_t rows, int64_t ld, int64_t width) {
  return ((rows - 1) * ld + ((width + 7) & ~int64_t(7))) * 2;
}

// K-contiguous operand: tile rows [row0, row0+256) of a [rows][K] matrix.
// Block b (16 rows) of the stage: lane L copies row 16b + L/4, logical chunk
// (L%4) ^ kc_swz(row) -- the swizzle only depends on the row's low 4 bits.
template <int NB = DMA_PER_OPERAND>
__device__ __forceinline__ OpStream stream_kc(const void* p, int64_t ld, int64_t rows, int64_t K, int64_t row0,
                                              int wb) {
  const int lane = tid_opaque() & 63;
  OpStream s;
  s.base = static_cast<const char*>(p) + row0 * ld * 2;
  s.nrec = (uint32_t)(extent_bytes(rows, ld, K) - row0 * ld * 2);   // row0 < rows: every tile starts inside
  s.step = BK * 2;
  const int r = lane >> 2;
  const int c = (lane & 3) ^ kc_swz(r);
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int row = 16 * (NB * wb + j) + r;
    s.voff[j] = (uint32_t)((row * ld + 8 * c) * 2);
  }
  return s;
}

// MN-contiguous operand: columns [col0, col0 + W) of a [K][cols] matrix.
// W = 256: block b holds rows 2b, 2b+1 (lane L: row 2b + L/32, chunk L%32);
// W = 128: block b holds rows 4b..4b+3 (lane L: row 4b + L/16, chunk L%16).
// Only the first VALID chunks of each row are wanted (a 192-wide tile kept
// in the 256-wide layout): lanes holding a later chunk are sent past the
// range, so they fetch nothing and fill their LDS slot with zeros.
constexpr uint32_t kDeadLane = 0x80000000u;   // above any extent (< 2 GiB), below 2^32 with any stage offset
template <int W, int VALID = W / 8>
__device__ __forceinline__ OpStream stream_mn(const void* p, int64_t ld, int64_t cols, int64_t K, int64_t col0,
                                              int wb) {
  const int lane = tid_opaque() & 63;
  constexpr int CHUNKS = W / 8;
  constexpr int ROWS = 512 / W;   // rows per block
  OpStream s;
  s.base = static_cast<const char*>(p) + col0 * 2;
  s.nrec = (uint32_t)(extent_bytes(K, ld, cols) - col0 * 2);   // col0 < cols: every tile starts inside
  s.step = (uint32_t)(BK * ld * 2);
#pragma unroll
  for (int j = 0; j < DMA_PER_OPERAND; ++j) {
    const int k = ROWS * (DMA_PER_OPERAND * wb + j) + lane / CHUNKS;
    const int c = (lane % CHUNKS) ^ mn_swz(k);
    s.voff[j] = (VALID < CHUNKS && c >= VALID) ? kDeadLane : (uint32_t)((k * ld + 8 * c) * 2);
  }
  return s;
}

// One 16-byte-per-lane copy into LDS at `ldst` (lane order) from `base` +
// voff (per lane) within a range of nrec bytes (past it: zeros).
__device__ __forceinline__ void copy16(const char* base, uint32_t nrec, uint32_t voff, TPS_LDS char* ldst) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, (int)nrec, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (TPS_LDS void*)ldst, 16, voff, 0, 0, 0);
}

// Zero k >= kvalid (0 < kvalid < 32) of a K-contiguous [256][32] LDS tile.
__device__ __forceinline__ void kc_zero_tail(TPS_LDS char* tile, int kvalid) {
  const int t = threadIdx.x;
  const int c = t & 3;
  if (8 * c + 8 <= kvalid) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (t >> 2) + 64 * i;
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

// s_waitcnt with the given vector-memory and LDS counts (expcnt left free).
template <int VM, int LGKM>
__device__ __forceinline__ void waitcnt() {
  static_assert(VM >= 0 && VM < 64 && LGKM >= 0 && LGKM < 16, "waitcnt range");
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (LGKM << 8));
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

// The LDS ring: NSTAGE distinct arrays (distinct objects, so the compiler
// tracks the copies into each separately).
__shared__ __attribute__((aligned(16))) char lds_ring0[STAGE_BYTES];
__shared__ __attribute__((aligned(16))) char lds_ring1[STAGE_BYTES];
__shared__ __attribute__((aligned(16))) char lds_ring2[STAGE_BYTES];
__shared__ __attribute__((aligned(16))) char lds_ring3[STAGE_BYTES];
static_assert(NSTAGE == 4, "ring_slot enumerates four arrays");

template <int S>
__device__ __forceinline__ TPS_LDS char* ring_slot() {
  if constexpr (S == 0) return (TPS_LDS char*)lds_ring0;
  else if constexpr (S == 1) return (TPS_LDS char*)lds_ring1;
  else if constexpr (S == 2) return (TPS_LDS char*)lds_ring2;
  else return (TPS_LDS char*)lds_ring3;
}

// ---- main loop -------------------------------------------------------------------
// NSTAGE LDS stages held in NSTAGE distinct __shared__ arrays form a ring: the
// copies of stage kt+NSTAGE-1 are issued while the MFMAs consume stage kt.
// Because the arrays are distinct objects, the compiler's own waits on the
// copies are per stage.  Each step waits until only the copies of the later
// in-flight stages are outstanding (vmcnt), drains its LDS reads (so the ring
// slot about to be refilled is no longer being read), and meets the other
// waves at a barrier.  The loop is unrolled NSTAGE times so every step's
// stage is static; a tile's stage count is padded to a multiple of NSTAGE
// with empty (all-zero) stages.
//
// The stage stream continues across the tiles a workgroup processes: the
// last NSTAGE-1 steps of a tile already issue the copies of the next tile's
// first stages, so the next tile starts with a full ring and the current
// tile's epilogue (which does not touch LDS) overlaps those copies.

// Which K-loop copies a kernel carries (Pipe::run_tile).
enum TailMode : int { TM_NONE = 0, TM_TAIL = 1, TM_ANY = 2 };

// Copy streams of one tile: per K segment (0, 1), one stream per operand.
// Plain named members (no arrays of structs) keep all of it in registers.
struct TileStreams {
  OpStream a0, a1, b0, b1;
  int kseg0, kseg1;        // K of each segment
  int nk0;                 // stages of segment 0
  int nk;                  // stages of the tile (0: no tile)
  int rot;                 // the K loop starts at stage rot, wrapping around to 0
  int npad;                // nk rounded up to NSTAGE
  int tail;                // a K-contiguous operand's segment ends inside a stage (K % 32 != 0)
};

// MI, NI: 32-row / 32-column units per wave along M and N (2 x 2 blocks of
// 16 x 16 each); the tile is (64 MI) x (64 NI), MI, NI in {2, 3, 4} (SwiGLU:
// NI = 4).  A K-contiguous operand of 64 MI rows is copied as MI blocks of 16
// rows per wave; an MN-contiguous one always fills the 256-wide LDS layout
// (narrower tiles leave its last columns zero: the lanes of those chunks are
// sent past the range).
template <int LAYOUT, bool DUAL, bool SEG2, int MI = 4, int NI = 4>
struct Pipe {
  static constexpr bool A_KC = LAYOUT != L_TN;
  static constexpr bool B_KC = LAYOUT == L_NT;
  static_assert(MI >= 2 && MI <= 4, "tile heights: 128, 192 or 256");
  static_assert(NI >= 2 && NI <= 4 && (NI == 4 || !DUAL), "tile widths: 128, 192 or 256 (SwiGLU: 256)");
  static constexpr int NBA = A_KC ? MI : DMA_PER_OPERAND;   // A copies per wave per stage
  static constexpr int NBB = B_KC ? NI : DMA_PER_OPERAND;   // B copies per wave per stage
  static constexpr int NCOPY = NBA + NBB;                   // copies per wave per stage
  static constexpr int KA = A_KC ? S_KC : S_MN256;
  static constexpr int KB = B_KC ? S_KC : (DUAL ? S_MN128 : S_MN256);

  int wave, wm, wn;
  int wlds_a, wlds_b;     // this wave's first copy block in the A / B tile (bytes)
  TileStreams cur, nxt;   // nxt.nk == 0: no next tile (its copies are empty)

  __device__ __forceinline__ void init_wave() {
    wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    wm = wave >> 1;
    wn = wave & 1;
    wlds_a = 1024 * NBA * wave;
    wlds_b = TILE_BYTES + (KB == S_MN128 ? (wave >> 1) * (TILE_BYTES / 2) + 1024 * DMA_PER_OPERAND * (wave & 1)
                                          : 1024 * NBB * wave);
    init_frag_addr();
  }

  __device__ __forceinline__ void seg_streams(const Problem& P, int64_t m0, int64_t n0, bool use1, OpStream& sa,
                                              OpStream& sb, int& Kseg) const {
    // Field-wise selection keeps the problem description in registers.
    const void* pa = use1 ? P.seg[1].a : P.seg[0].a;
    const void* pb = use1 ? P.seg[1].b : P.seg[0].b;
    const int64_t lda = use1 ? P.seg[1].lda : P.seg[0].lda;
    const int64_t ldb = use1 ? P.seg[1].ldb : P.seg[0].ldb;
    const int64_t K = use1 ? P.seg[1].K : P.seg[0].K;
    Kseg = (int)K;
    sa = A_KC ? stream_kc<NBA>(pa, lda, P.M, K, m0, wave) : stream_mn<256, 8 * MI>(pa, lda, P.M, K, m0, wave);
    if (B_KC) {
      sb = stream_kc<NBB>(pb, ldb, P.N, K, n0, wave);
    } else if (DUAL) {   // waves 0,1 stream the gate weight, waves 2,3 the up weight
      const bool up = (wave >> 1) != 0;
      sb = stream_mn<128>(up ? P.b_up : pb, up ? P.ldb_up : ldb, P.N, K, n0, wave & 1);
    } else {
      sb = stream_mn<256, 8 * NI>(pb, ldb, P.N, K, n0, wave);
    }
  }

  // Streams of the tile at (m0, n0), its K loop started rot8/8 of the way in.
  __device__ __forceinline__ TileStreams make_streams(const Problem& P, int64_t m0, int64_t n0, int rot8 = 0) const {
    TileStreams T;
    seg_streams(P, m0, n0, false, T.a0, T.b0, T.kseg0);
    if (SEG2) {
      seg_streams(P, m0, n0, true, T.a1, T.b1, T.kseg1);
    } else {
      T.a1 = T.a0;
      T.b1 = T.b0;
      T.kseg1 = T.kseg0;
    }
    T.nk0 = (int)((T.kseg0 + BK - 1) / BK);
    T.nk = T.nk0 + (SEG2 ? (int)((T.kseg1 + BK - 1) / BK) : 0);
    T.rot = (T.nk * rot8) >> 3;
    T.npad = (T.nk + NSTAGE - 1) / NSTAGE * NSTAGE;
    T.tail = (A_KC || B_KC) && ((T.kseg0 % BK) != 0 || (SEG2 && (T.kseg1 % BK) != 0));
    uniform(T);
    return T;
  }

  // The stream records are wave-uniform, but parts of them are computed on
  // the vector ALU (integer division has no scalar form); readfirstlane moves
  // them to scalar registers once per tile, so the per-stage descriptor
  // arithmetic is scalar.
  static __device__ __forceinline__ uint32_t sgpr(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }
  static __device__ __forceinline__ int sgpr(int v) { return __builtin_amdgcn_readfirstlane(v); }
  static __device__ __forceinline__ void uniform(OpStream& o) {
    const uint64_t a = reinterpret_cast<uint64_t>(o.base);
    o.base = reinterpret_cast<const char*>(((uint64_t)sgpr((uint32_t)(a >> 32)) << 32) | sgpr((uint32_t)a));
    o.nrec = sgpr(o.nrec);
    o.step = sgpr(o.step);
  }
  static __device__ __forceinline__ void uniform(TileStreams& T) {
    uniform(T.a0);
    uniform(T.b0);
    if (SEG2) {
      uniform(T.a1);
      uniform(T.b1);
    }
    T.kseg0 = sgpr(T.kseg0);
    T.kseg1 = sgpr(T.kseg1);
    T.nk0 = sgpr(T.nk0);
    T.nk = sgpr(T.nk);
    T.rot = sgpr(T.rot);
    T.npad = sgpr(T.npad);
    T.tail = sgpr(T.tail);
  }

  __device__ __forceinline__ void no_next() {
    nxt = cur;
    nxt.nk = 0;
    nxt.rot = 0;
    nxt.npad = 0;
  }

  // Tile stage of step r; live == false past the tile's last stage.
  static __device__ __forceinline__ int stage_of(const TileStreams& T, int r, bool& live) {
    int t = r + T.rot;
    t = t >= T.nk ? t - T.nk : t;
    live = r < T.nk;
    return t;
  }

  // The copy source of step r: the current tile's step r or, past its
  // padded end, the next tile's step r - npad (the next tile's first stages
  // load during this tile's last steps and its epilogue).  Selected
  // field-wise at run time -- scalars once per step, one vector select per
  // copy -- so that the K loop is one uniform body (a separate block for the
  // last steps made the register allocator move accumulators around it).
  struct CopySrc {
    const char* basea;      // the stage's first byte of each operand (the tile origin + the stage offset)
    const char* baseb;
    uint32_t nreca, nrecb;  // bytes from there to the operand's end; 0 past the tile's end (zeros)
    int nx, s1;             // masks (-1 / 0): the next tile's streams, the second K segment's
  };
  template <class F>
  __device__ __forceinline__ static auto pick4(int nx, int s1, F c0, F c1, F n0, F n1) {
    if constexpr (SEG2) return nx ? (s1 ? n1 : n0) : (s1 ? c1 : c0);
    else return nx ? n0 : c0;
  }
  // Its computation in NCALC small steps of a few scalar instructions each,
  // so that the K loop can spread the next step's over as many MFMAs (one
  // wave per SIMD issues about one instruction per 4 cycles, so only a few
  // fit in the shadow of each MFMA; a run of a few dozen stalls them).  Each
  // step ends with an empty asm statement that takes its results and the
  // next-tile mask as read-write operands.  The compiler keeps those
  // statements in order with the loop's MFMA statements, and a step's
  // arithmetic depends on the previous statement's mask and feeds its own,
  // so it stays between the two (left alone, the compiler gathers all
  // selects on one condition into one run).  Flags are sign-splat masks,
  // x >> sh with sh = 31 held in a register: with a literal 31 the compiler
  // turns the shift back into a compare, whose integer value it forms on
  // the vector unit.
  struct CopyCalc {
    int sh;                     // 31
    int rr, cnt, t, live;       // live: -1 for a stage inside the tile, else 0
    uint32_t stage, oa, ob;
    CopySrc c;
  };
  static constexpr int NCALC = 12;
  // (readfirstlane: where the compiler has kept a uniform value in a vector
  // register, one instruction moves it to a scalar one; elsewhere it folds.)
  static __device__ __forceinline__ int sg(int x) { return __builtin_amdgcn_readfirstlane(x); }
  static __device__ __forceinline__ uint32_t sg(uint32_t x) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)x); }
  static __device__ __forceinline__ const char* sg(const char* x) { return x; }
  template <class T>
  static __device__ __forceinline__ void pin(T& x, int& nx) {
    x = sg(x);
    nx = sg(nx);
    asm volatile("" : "+s"(x), "+s"(nx));
  }
  __device__ __forceinline__ void calc_init(CopyCalc& w) const {
    w.sh = 31;
    w.c.nx = 0;
    pin(w.sh, w.c.nx);
  }
  template <int I>
  __device__ __forceinline__ void calc(CopyCalc& w, int r) const {
    CopySrc& c = w.c;
    if constexpr (I == 0) {
      c.nx = ~((r - cur.npad) >> w.sh);   // r >= npad
      w.rr = r;
      pin(w.rr, c.nx);
    } else if constexpr (I == 1) {
      w.rr -= cur.npad & c.nx;
      pin(w.rr, c.nx);
    } else if constexpr (I == 2) {
      w.cnt = c.nx ? nxt.nk : cur.nk;
      pin(w.cnt, c.nx);
    } else if constexpr (I == 3) {
      w.t = w.rr + (c.nx ? nxt.rot : cur.rot);
      pin(w.t, c.nx);
    } else if constexpr (I == 4) {
      w.live = (w.rr - w.cnt) >> w.sh;   // rr < cnt
      pin(w.live, c.nx);
    } else if constexpr (I == 5) {
      const int st = w.t - (w.cnt & ~((w.t - w.cnt) >> w.sh));   // t >= cnt: wrap
      if constexpr (SEG2) {
        const int nk0 = c.nx ? nxt.nk0 : cur.nk0;
        c.s1 = ~((st - nk0) >> w.sh);   // st >= nk0
        w.stage = (uint32_t)(st - (nk0 & c.s1));
        pin(c.s1, c.nx);
      } else {
        c.s1 = 0;
        w.stage = (uint32_t)st;
      }
      pin(w.stage, c.nx);
    } else if constexpr (I == 6) {
      w.oa = w.stage * pick4(c.nx, c.s1, cur.a0.step, cur.a1.step, nxt.a0.step, nxt.a1.step);
      pin(w.oa, c.nx);
    } else if constexpr (I == 7) {
      c.basea = pick4(c.nx, c.s1, cur.a0.base, cur.a1.base, nxt.a0.base, nxt.a1.base) + w.oa;
      pin(c.basea, c.nx);
    } else if constexpr (I == 8) {   // a stage past the tile's end reads past the range: zeros
      c.nreca = (pick4(c.nx, c.s1, cur.a0.nrec, cur.a1.nrec, nxt.a0.nrec, nxt.a1.nrec) - w.oa) & (uint32_t)w.live;
      pin(c.nreca, c.nx);
    } else if constexpr (I == 9) {
      w.ob = w.stage * pick4(c.nx, c.s1, cur.b0.step, cur.b1.step, nxt.b0.step, nxt.b1.step);
      pin(w.ob, c.nx);
    } else if constexpr (I == 10) {
      c.baseb = pick4(c.nx, c.s1, cur.b0.base, cur.b1.base, nxt.b0.base, nxt.b1.base) + w.ob;
      pin(c.baseb, c.nx);
    } else if constexpr (I == 11) {
      c.nrecb = (pick4(c.nx, c.s1, cur.b0.nrec, cur.b1.nrec, nxt.b0.nrec, nxt.b1.nrec) - w.ob) & (uint32_t)w.live;
      pin(c.nrecb, c.nx);
    }
  }
  template <int... Is>
  __device__ __forceinline__ void calc_all(CopyCalc& w, int r, std::integer_sequence<int, Is...>) const {
    (calc<Is>(w, r), ...);
  }
  __device__ __forceinline__ CopySrc copy_src(int r) const {
    CopyCalc w;
    calc_init(w);
    calc_all(w, r, std::make_integer_sequence<int, NCALC>{});
    return w.c;
  }

  // Copy C of a step into `dst`: copies [0, NBA) are A's blocks, [NBA, NCOPY)
  // B's.  Each writes 1 KiB of LDS in lane order at the wave's block.
  template <int C>
  __device__ __forceinline__ void issue1(const CopySrc& c, TPS_LDS char* dst) {
    if constexpr (C < NBA) {
      const uint32_t v = pick4(c.nx, c.s1, cur.a0.voff[C], cur.a1.voff[C], nxt.a0.voff[C], nxt.a1.voff[C]);
      copy16(c.basea, c.nreca, v, dst + wlds_a + 1024 * C);
    } else {
      constexpr int J = C - NBA;
      const uint32_t v = pick4(c.nx, c.s1, cur.b0.voff[J], cur.b1.voff[J], nxt.b0.voff[J], nxt.b1.voff[J]);
      copy16(c.baseb, c.nrecb, v, dst + wlds_b + 1024 * J);
    }
  }
  template <int... Cs>
  __device__ __forceinline__ void issue_all(const CopySrc& c, TPS_LDS char* dst, std::integer_sequence<int, Cs...>) {
    (issue1<Cs>(c, dst), ...);
  }
  __device__ __forceinline__ void issue(int r, TPS_LDS char* dst) {
    issue_all(copy_src(r), dst, std::make_integer_sequence<int, NCOPY>{});
  }

  // 16 x 16 MFMA blocks per wave along M and N; acc[i][j] is block (i, j).
  static constexpr int BI = 2 * MI, BJ = 2 * NI;
  typedef f32x4 Acc[BI][BJ];

  // Per-lane LDS byte addresses of the fragments, computed once.  A fragment
  // of v_mfma_f32_16x16x32_bf16: lane l holds 8 consecutive k (k = 8 (l/16)
  // .. +7 of the 32-deep stage) of row/column l % 16 of its 16-wide block.
  //   K-contiguous operand: one ds_read_b128 (row l % 16 of the block, chunk
  //   l / 16); block b is +16 rows = +1024 bytes (the row swizzle repeats
  //   every 16 rows), so one base address.
  //   MN-contiguous operand: two ds_read_b64_tr_b16 (rows k and k + 4); one
  //   address per block (the swizzle mixes the column into the chunk index).
  //   Within each 16-lane group the transposing read gives lane i element
  //   i % 4 of the 8-byte loads of source lanes i/4, 4 + i/4, 8 + i/4,
  //   12 + i/4: source lane s loads row k0 + s/4, columns c + 4 (s % 4) .. +3,
  //   and lane i ends up with rows k0 .. k0+3 of column c + i.
  int adA[A_KC ? 1 : BI], adB[B_KC ? 1 : BJ];

  __device__ __forceinline__ void init_frag_addr() {
    const int lane = threadIdx.x & 63;
    const int h = lane >> 4, q = lane & 15;
    const int k = 8 * h + (q >> 2);   // first row of this lane's transposing read
    if constexpr (A_KC) {
      adA[0] = kc_off(32 * MI * wm + q, h);
    } else {
#pragma unroll
      for (int i = 0; i < (A_KC ? 1 : BI); ++i) {
        const int col = 32 * MI * wm + 16 * i + 4 * (q & 3);
        adA[i] = mn_off<512>(k, col >> 3) + (col & 7) * 2;
      }
    }
    if constexpr (B_KC) {
      adB[0] = TILE_BYTES + kc_off(32 * NI * wn + q, h);
    } else {
#pragma unroll
      for (int j = 0; j < (B_KC ? 1 : BJ); ++j) {
        if (DUAL) {   // blocks 0-3: gate columns 64 wn .. +63, blocks 4-7: the same up columns
          const int col = 64 * wn + 16 * (j & 3) + 4 * (q & 3);
          adB[j] = TILE_BYTES + (j >> 2) * (TILE_BYTES / 2) + mn_off<256>(k, col >> 3) + (col & 7) * 2;
        } else {
          const int col = 32 * NI * wn + 16 * j + 4 * (q & 3);
          adB[j] = TILE_BYTES + mn_off<512>(k, col >> 3) + (col & 7) * 2;
        }
      }
    }
  }

  static __device__ __forceinline__ bf16x8 rd_kc(const TPS_LDS char* p) {
    return *reinterpret_cast<const TPS_LDS bf16x8*>(p);
  }
  static __device__ __forceinline__ i16x4 rd_tr(const TPS_LDS char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((TPS_LDS i16x4*)p);
  }

  // Fragment registers.  B: one set per stage parity (the loop is unrolled
  // over an even number of ring slots, so the parity is static): the
  // previous stage's second half still multiplies its B while this stage's
  // is read.  A: one set -- its first half is read after the previous stage's
  // first half has run, its second half after the previous second half.
  // MN-contiguous fragments are kept as their two transposed halves.
  bf16x8 akc[BI], bkc[2][BJ];
  i16x4 amn[BI][2], bmn[2][BJ][2];

  __device__ __forceinline__ bf16x8 fragA(int i) const {
    if constexpr (A_KC) return akc[i];
    else return __builtin_bit_cast(bf16x8, __builtin_shufflevector(amn[i][0], amn[i][1], 0, 1, 2, 3, 4, 5, 6, 7));
  }
  template <int P>
  __device__ __forceinline__ bf16x8 fragB(int j) const {
    if constexpr (B_KC) return bkc[P][j];
    else return __builtin_bit_cast(bf16x8, __builtin_shufflevector(bmn[P][j][0], bmn[P][j][1], 0, 1, 2, 3, 4, 5, 6, 7));
  }

  // LDS read R of a stage (one instruction): the A fragments of block rows
  // [I0, I1) first (MN: two reads each), then, when WITH_B, all of B.
  static constexpr int RA_PER = A_KC ? 1 : 2, RB_PER = B_KC ? 1 : 2;
  template <int P, int I0, int I1, bool WITH_B, int R>
  __device__ __forceinline__ void read_op(const TPS_LDS char* base) {
    constexpr int NRA = (I1 - I0) * RA_PER;
    if constexpr (R < NRA) {
      constexpr int i = I0 + R / RA_PER, h = R % RA_PER;
      if constexpr (A_KC) akc[i] = rd_kc(base + adA[0] + 1024 * i);
      else amn[i][h] = rd_tr(base + adA[A_KC ? 0 : i] + h * 4 * 512);
    } else if constexpr (WITH_B) {
      constexpr int j = (R - NRA) / RB_PER, h = (R - NRA) % RB_PER;
      if constexpr (B_KC) bkc[P][j] = rd_kc(base + adB[0] + 1024 * j);
      else bmn[P][j][h] = rd_tr(base + adB[B_KC ? 0 : j] + h * 4 * (DUAL ? 256 : 512));
    }
  }

  // One MFMA of the stage with parity P, accumulating in place: an asm
  // statement ties the accumulator to one register tuple for the whole loop.
  // (Written with the compiler builtin, the 16 x 16 accumulators were renamed
  // and copied between registers every step.)  Operands as (B, A): the lane
  // holds output row lane % 16, columns 4 (lane / 16) .. +3.
  template <int P, int I, int J>
  __device__ __forceinline__ void mma1(Acc& acc) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0"
                 : "+a"(acc[I][J])
                 : "v"(fragB<P>(J)), "v"(fragA(I)));
  }

  __device__ __forceinline__ void zero_set1() {
#pragma unroll
    for (int i = 0; i < BI; ++i) {
      akc[i] = bf16x8{};
      amn[i][0] = amn[i][1] = i16x4{};
    }
#pragma unroll
    for (int j = 0; j < BJ; ++j) {
      bkc[1][j] = bf16x8{};
      bmn[1][j][0] = bmn[1][j][1] = i16x4{};
    }
  }

  // Group G of a phase: MFMA G of the half H of the stage with parity PM
  // (block row H*BI/2 + G/BJ, column G % BJ), then LDS read G (of the reads
  // of block rows [I0, I1) of A and, WITH_B, all of B, for parity PR), then,
  // with copies, copy G/2 after every second MFMA; fenced so the scheduler
  // keeps this order.
  static constexpr int HALF_MFMA = (BI / 2) * BJ;
  // COPIES: phase 1 issues the copies described by w.c; otherwise (phase 2)
  // groups [CALC_AT, CALC_AT + NCALC) compute the next step's copy source
  // into w, one small step each.  Phase 1's fences let scalar instructions
  // through (the copies' M0 set-up); phase 2's let nothing through, so that
  // the scheduler cannot gather the copy-source steps into one run.
  static constexpr int READS2 = (BI - BI / 2) * RA_PER;
  static constexpr int CALC_AT = READS2;
  template <int PM, int H, int PR, int I0, int I1, bool WITH_B, int NREAD, bool COPIES, int G>
  __device__ __forceinline__ void group(Acc& acc, const TPS_LDS char* rbase, CopyCalc& w, TPS_LDS char* cdst,
                                        int rnext) {
    if constexpr (G < HALF_MFMA) mma1<PM, H * (BI / 2) + G / BJ, G % BJ>(acc);
    if constexpr (G < NREAD) read_op<PR, I0, I1, WITH_B, G>(rbase);
    if constexpr (COPIES && G % COPY_EVERY == 0 && G / COPY_EVERY < NCOPY) issue1<G / COPY_EVERY>(w.c, cdst);
    if constexpr (!COPIES && G >= CALC_AT && G < CALC_AT + NCALC) calc<G - CALC_AT>(w, rnext);
    __builtin_amdgcn_sched_barrier(COPIES ? 0x0004 : 0);
  }
  template <int PM, int H, int PR, int I0, int I1, bool WITH_B, int NREAD, bool COPIES, int... Gs>
  __device__ __forceinline__ void phase(Acc& acc, const TPS_LDS char* rbase, CopyCalc& w, TPS_LDS char* cdst,
                                        int rnext, std::integer_sequence<int, Gs...>) {
    (group<PM, H, PR, I0, I1, WITH_B, NREAD, COPIES, Gs>(acc, rbase, w, cdst, rnext), ...);
  }
  static constexpr int READS1 = (BI / 2) * RA_PER + BJ * RB_PER;
  static constexpr int COPY_EVERY = HALF_MFMA >= 4 * NCOPY ? 4 : 2;   // MFMAs per copy in phase 1
  static constexpr int GROUPS1 = std::max(std::max(HALF_MFMA, READS1), COPY_EVERY * NCOPY);
  static constexpr int GROUPS2 = std::max(HALF_MFMA, CALC_AT + NCALC);

  // One 32-deep K step on ring slot S (step kt of the current tile).
  // Software pipeline: phase 1 runs the second half of the previous stage's
  // MFMAs (operands already in registers) while this stage's first-half A
  // and all its B are read and the copies of step kt + NSTAGE - 1 are issued;
  // phase 2 runs this stage's first half while its second-half A is read.
  // w.c: the copy source of this step (step kt + NSTAGE - 1 of the tile),
  // replaced during phase 2 by the next step's.
  template <int S, bool TAIL>
  __device__ __forceinline__ void step(int kt, Acc& acc, CopyCalc& w) {
    TPS_LDS char* cur_slot = ring_slot<S>();
    // Stage kt's copies are complete once only the later NSTAGE-2 stages'
    // copies (NCOPY each) remain outstanding; lgkmcnt(0)
    // retires this wave's reads of the slot that is refilled below.
    waitcnt<(NSTAGE - 2) * NCOPY, 0>();
    __builtin_amdgcn_s_barrier();
    if constexpr (TAIL) {   // K tail of K-contiguous operands: zero k past the segment's end
      bool kt_live;
      const int ka = stage_of(cur, kt, kt_live);   // stage within the tile
      const bool s1 = SEG2 && ka >= cur.nk0;
      const int kseg = s1 ? cur.kseg1 : cur.kseg0;
      const int k0 = (s1 ? ka - cur.nk0 : ka) * BK;
      if (kt_live && k0 + BK > kseg) {
        if (A_KC) kc_zero_tail(cur_slot, kseg - k0);
        if (B_KC) kc_zero_tail(cur_slot + TILE_BYTES, kseg - k0);
        waitcnt<63, 0>();
        __builtin_amdgcn_s_barrier();
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    constexpr int PC = S & 1, PP = (S + 1) & 1;   // this stage's and the previous stage's parity
    TPS_LDS char* cdst = ring_slot<(S + NSTAGE - 1) % NSTAGE>();
    phase<PP, 1, PC, 0, BI / 2, true, READS1, true>(acc, cur_slot, w, cdst, 0,
                                                   std::make_integer_sequence<int, GROUPS1>{});
    phase<PC, 0, PC, BI / 2, BI, false, READS2, false>(acc, cur_slot, w, cdst, kt + NSTAGE,
                                                      std::make_integer_sequence<int, GROUPS2>{});
  }

  // The last stage's second half, after the loop: written with the compiler
  // builtin, which the compiler's hazard checks see (outside the loop it may
  // move accumulators between register files, and a register copy right next
  // to an asm MFMA would be a hazard it does not know about).
  template <int P, int H, int... Gs>
  __device__ __forceinline__ void mma_half(Acc& acc, std::integer_sequence<int, Gs...>) {
    ((acc[H * (BI / 2) + Gs / BJ][Gs % BJ] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          fragB<P>(Gs % BJ), fragA(H * (BI / 2) + Gs / BJ), acc[H * (BI / 2) + Gs / BJ][Gs % BJ], 0, 0, 0)),
     ...);
  }

  // Run the current tile.  The copies of its first NSTAGE-1 stages must
  // already be issued, and nxt set (the next tile, or no_next()): the
  // tile's last NSTAGE-1 steps issue the next tile's first stages.
  // `init` sets the accumulators' starting values.  Tiles whose
  // K-contiguous operands end inside a stage (cur.tail) run a copy of the
  // loop that zeroes those tails; TM says which copies a kernel carries:
  // TM_NONE (the caller never passes such tiles), TM_TAIL (only such
  // tiles), TM_ANY (both copies, chosen per tile).  A test inside the loop
  // would split its body into blocks, and the compiler sinks the scalar copy
  // bookkeeping across such splits to just after the barrier, where it
  // stalls the MFMAs; two copies in one kernel hold about twice the vector
  // registers, which the persistent kernels cannot spare without spilling.
  template <int TM, class InitFn>
  __device__ __forceinline__ void run_tile(Acc& acc, InitFn&& init) {
    if constexpr (TM == TM_ANY) {
      if ((A_KC || B_KC) && cur.tail) run_loop<A_KC || B_KC>(acc, init);
      else run_loop<false>(acc, init);
    } else {
      run_loop<TM == TM_TAIL && (A_KC || B_KC)>(acc, init);
    }
  }
  template <bool TAIL, class InitFn>
  __device__ __forceinline__ void run_loop(Acc& acc, InitFn&& init) {
    static_assert(NSTAGE % 2 == 0, "the fragment set of a stage is its parity");
    init(acc);
    zero_set1();              // the first step's deferred half multiplies zeros
    // The loop's asm MFMAs read the accumulators as written by ordinary code
    // (the starting values) and leave them to ordinary code, neither of which
    // sees them as MFMAs: wait states on both sides of the loop (the hazards
    // of a register write before an MFMA reads it, and of an MFMA's result
    // before a register read, last a few passes).
    asm volatile("s_nop 4" ::: "memory");
    CopyCalc w;
    calc_init(w);
    calc_all(w, NSTAGE - 1, std::make_integer_sequence<int, NCALC>{});
    for (int kt = 0; kt < cur.npad; kt += NSTAGE) {
      step<0, TAIL>(kt, acc, w);
      step<1, TAIL>(kt + 1, acc, w);
      step<2, TAIL>(kt + 2, acc, w);
      step<3, TAIL>(kt + 3, acc, w);
    }
    asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");
    mma_half<(NSTAGE - 1) & 1, 1>(acc, std::make_integer_sequence<int, HALF_MFMA>{});   // last stage, second half
  }

  __device__ __forceinline__ void prologue() {
    issue(0, ring_slot<0>());
    issue(1, ring_slot<1>());
    issue(2, ring_slot<2>());
  }
};

template <int MI, int NI = 4>
__device__ __forceinline__ void zero_acc(f32x4 (&acc)[2 * MI][2 * NI]) {
#pragma unroll
  for (int i = 0; i < 2 * MI; ++i)
#pragma unroll
    for (int j = 0; j < 2 * NI; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// ---- GEMM epilogue -------------------------------------------------------------------
// In a 16 x 16 accumulator block a lane holds row (lane % 16) and the four
// consecutive columns 4 (lane / 16) .. +3.  SwiGLU waves hold gate blocks
// 0-3 and the matching up blocks 4-7 (same columns).
//
// Fast path (16-byte aligned rows; the persistent kernels; a column bias is
// already in the accumulators, see TileInit): blocks are finished in pairs (j, j + 1) of
// adjacent 16-column blocks -- values in fp32, packed to bf16 pairs, then
// one v_permlane16_swap per packed register trades half of them between the
// lanes of adjacent 16-lane rows, so that every lane holds eight consecutive
// columns, written with one 16-byte store.  No LDS: the ring is already
// filling with the next tile's stages.
//
// Generic path (edge tiles, unaligned outputs, bias outside NN products;
// one tile per workgroup): see generic_epilogue.

// p: the lane's packed block-j values (two registers), q: block j + 1's.
// v_permlane16_swap swaps the odd 16-lane rows of its first operand with the
// even rows of its second: afterwards a lane of row 0 or 2 holds {p, q} =
// block j columns 4g .. 4g+7, a lane of row 1 or 3 block j+1 columns
// 4(g-1) .. 4g+3 (g = lane / 16).
__device__ __forceinline__ void swap_pair(uint32_t (&p)[2], uint32_t (&q)[2]) {
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const auto r = __builtin_amdgcn_permlane16_swap(p[w], q[w], false, false);
    p[w] = r[0];
    q[w] = r[1];
  }
}

__device__ __forceinline__ void store_pq(uint16_t* p, const uint32_t (&a)[2], const uint32_t (&b)[2]) {
  *reinterpret_cast<u32x4*>(p) = u32x4{a[0], a[1], b[0], b[1]};
}

// A lane's output position in a tile's fast epilogue, computed once per
// tile: block row I, column pair JP of its 8-column chunk lies at
// c + I * rc + 32 JP elements (16 rows per block row; the pair step fits the
// store's immediate offset), so the per-pair address work is one add per
// block row.  Kept small (two pointers, two counts): the epilogue runs
// beside the accumulators and the fragment registers of the K loop.
template <int EPI>
struct EpiLane {
  uint16_t* c;     // output at the lane's row of block row 0, first column of its chunk in pair 0
  uint16_t* pre;   // pre-activation output at the same position (GeLU, SwiGLU)
  int64_t rc, rp;  // 16 rows of c / pre, in elements (wave-uniform)
  int rl, cl;      // rows below / columns right of that position inside the output (clamped to 2^30)
  bool whole;      // the tile lies inside the output: no per-lane bounds (wave-uniform)
  int64_t m, cg;   // E_CE_GRAD: the lane's row, first column of its 4-column group in block 0
};

template <int EPI, int MI, int NI>
__device__ __forceinline__ EpiLane<EPI> epi_lane(const Problem& P, int64_t m0, int64_t n0) {
  constexpr bool dual = EPI == E_SWIGLU;
  const int tid = tid_opaque(), lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
  const int g = lane >> 4;
  EpiLane<EPI> e;
  const int64_t m = m0 + 32 * MI * wm + (lane & 15);
  const int64_t cj = n0 + (dual ? 64 * wn : 32 * NI * wn);   // first column of the wave's block 0
  const int64_t n = cj + 16 * (g & 1) + 4 * (g & 2);        // this lane's 8 columns
  const int64_t bw = dual ? BN / 2 : 64 * NI;
  e.whole = m0 + 64 * MI <= P.M && n0 + bw <= P.N;
  e.rl = (int)min<int64_t>(P.M - m, int64_t(1) << 30);
  e.cl = (int)min<int64_t>(P.N - n, int64_t(1) << 30);
  e.c = static_cast<uint16_t*>(P.c) + m * P.ldc + n;
  e.rc = 16 * P.ldc;
  if (EPI == E_GELU || EPI == E_SWIGLU) {
    e.pre = static_cast<uint16_t*>(P.pre) + m * P.ldpre + n;
    e.rp = 16 * P.ldpre;
  } else {
    e.pre = nullptr;
    e.rp = 0;
  }
  if (EPI == E_CE_GRAD) {
    e.m = m;
    e.cg = cj + 4 * g;
  } else {
    e.m = e.cg = 0;
  }
  return e;
}

// Blocks (I, 2 JP) and (I, 2 JP + 1) of the wave (a, b); for SwiGLU also the
// up blocks (I, 2 JP + 4), (I, 2 JP + 5) (ua, ub).  A tile may overhang the
// matrix (rows past M; columns past N when N is a multiple of 8): unless
// the tile is whole, each lane's 8-column chunk is stored only inside it.
template <int EPI, int MI, int NI, int I, int JP>
__device__ __forceinline__ void fast_pair(const Problem& P, const EpiLane<EPI>& e, const f32x4& a, const f32x4& b,
                                          const f32x4& ua, const f32x4& ub) {
  constexpr bool dual = EPI == E_SWIGLU;
  float ce_l = 0.f, ce_g = 0.f;
  int64_t ce_t = 0;
  if (EPI == E_CE_GRAD) {   // per-row loss terms; the target column relative to this lane's block-2JP columns
    const int64_t m = e.m + 16 * I;
    const int64_t mr = m < P.M ? m : P.M - 1;
    ce_l = P.lse[mr];
    ce_g = P.gscale ? P.gscale[mr] : 1.0f;
    ce_t = (int64_t)P.target[mr] - P.v0 - (e.cg + 32 * JP);
  }
  uint32_t py[2], qy[2], pg[2], qg[2], pu[2], qu[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {   // packed register h: elements 2h, 2h + 1
    const float a0 = a[2 * h], a1 = a[2 * h + 1], b0 = b[2 * h], b1 = b[2 * h + 1];
    if (EPI == E_STORE) {
      py[h] = pack_bf2(a0, a1);
      qy[h] = pack_bf2(b0, b1);
    } else if (EPI == E_CE_GRAD) {
      py[h] = pack_bf2(ce_g * (__expf(a0 - ce_l) - (ce_t == 2 * h ? 1.0f : 0.0f)),
                       ce_g * (__expf(a1 - ce_l) - (ce_t == 2 * h + 1 ? 1.0f : 0.0f)));
      qy[h] = pack_bf2(ce_g * (__expf(b0 - ce_l) - (ce_t == 16 + 2 * h ? 1.0f : 0.0f)),
                       ce_g * (__expf(b1 - ce_l) - (ce_t == 17 + 2 * h ? 1.0f : 0.0f)));
    } else if (EPI == E_GELU) {
      pg[h] = pack_bf2(a0, a1);
      qg[h] = pack_bf2(b0, b1);
      py[h] = pack_bf2(gelu_f(a0), gelu_f(a1));
      qy[h] = pack_bf2(gelu_f(b0), gelu_f(b1));
    } else {
      const float u0 = ua[2 * h], u1 = ua[2 * h + 1], v0 = ub[2 * h], v1 = ub[2 * h + 1];
      pg[h] = pack_bf2(a0, a1);
      qg[h] = pack_bf2(b0, b1);
      pu[h] = pack_bf2(u0, u1);
      qu[h] = pack_bf2(v0, v1);
      py[h] = pack_bf2(silu_f(a0) * u0, silu_f(a1) * u1);
      qy[h] = pack_bf2(silu_f(b0) * v0, silu_f(b1) * v1);
    }
  }
  swap_pair(py, qy);
  if (EPI == E_GELU || EPI == E_SWIGLU) swap_pair(pg, qg);
  if (dual) swap_pair(pu, qu);
  if (e.whole || (16 * I < e.rl && 32 * JP < e.cl)) {
    store_pq(e.c + I * e.rc + 32 * JP, py, qy);
    if (EPI == E_GELU || EPI == E_SWIGLU) store_pq(e.pre + I * e.rp + 32 * JP, pg, qg);
    if (dual) store_pq(e.pre + I * e.rp + P.N + 32 * JP, pu, qu);
  }
}

template <int EPI, int MI, int NI, int... Is>
__device__ __forceinline__ void fast_epilogue(const Problem& P, int64_t m0, int64_t n0,
                                              f32x4 (&acc)[2 * MI][2 * NI], std::integer_sequence<int, Is...>) {
  constexpr int NP = EPI == E_SWIGLU ? 2 : NI;   // block pairs per block row
  constexpr int UP = EPI == E_SWIGLU ? 4 : 0;    // SwiGLU: block j's up values are block j + 4
  const EpiLane<EPI> e = epi_lane<EPI, MI, NI>(P, m0, n0);
  ((fast_pair<EPI, MI, NI, Is / NP, Is % NP>(P, e, acc[Is / NP][2 * (Is % NP)], acc[Is / NP][2 * (Is % NP) + 1],
                                             acc[Is / NP][2 * (Is % NP) + UP], acc[Is / NP][2 * (Is % NP) + 1 + UP]),
    __builtin_amdgcn_sched_barrier(0)),
   ...);
}

// Generic path: the ring is drained, and each wave stages 32-row slices of
// its 128 x 128 accumulator (two block rows) in its own ring slot, then
// finishes eight columns at a time with every bound checked.
constexpr int EPI_LD = 132;                       // floats per staged row (128 + 4 padding)

template <int SL>
__device__ __forceinline__ void stage_slice(TPS_LDS float* w, const f32x4 (&acc)[8][8]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int j = 0; j < 8; ++j)
      *reinterpret_cast<TPS_LDS f32x4*>(w + (16 * rb + (lane & 15)) * EPI_LD + 16 * j + 4 * (lane >> 4)) =
          acc[2 * SL + rb][j];
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
  } else if (P.epi == E_CE_GRAD) {
    const float l = P.lse[m], g = P.gscale ? P.gscale[m] : 1.0f;
    const int64_t t = (int64_t)P.target[m] - P.v0 - n;   // target column relative to n
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = g * (__expf(v[e] - l) - (t == e ? 1.0f : 0.0f));
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

// The ring must be drained (no copies in flight) and every wave past its
// last fragment read.
__device__ __forceinline__ void generic_epilogue(const Problem& P, int64_t m0, int64_t n0, f32x4 (&acc)[8][8]) {
  const int wave = threadIdx.x >> 6;   // wave w stages in ring slot w (16.5 KiB of 32 KiB)
  TPS_LDS float* w = reinterpret_cast<TPS_LDS float*>(
      wave < 2 ? (wave == 0 ? ring_slot<0>() : ring_slot<1>()) : (wave == 2 ? ring_slot<2>() : ring_slot<3>()));
#pragma unroll 1
  for (int i = 0; i < 4; ++i) {
    switch (i) {   // constant indices into acc keep it in registers
      case 0: stage_slice<0>(w, acc); break;
      case 1: stage_slice<1>(w, acc); break;
      case 2: stage_slice<2>(w, acc); break;
      default: stage_slice<3>(w, acc); break;
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's staging writes are done
    store_slice(P, w, m0, n0, i);
    __builtin_amdgcn_s_waitcnt(0xc07f);   // reads done before the next slice overwrites
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
  TPS_PICK(lse); TPS_PICK(gscale); TPS_PICK(target); TPS_PICK(v0);
  TPS_PICK(tiles_m); TPS_PICK(tiles_n); TPS_PICK(tile_begin);
  TPS_PICK(edge_only); TPS_PICK(full_m); TPS_PICK(full_n);
  TPS_PICK(ksplit); TPS_PICK(c32);
#undef TPS_PICK
  return P;
}

// Tile of a launch: its problem (selected field-wise) and its origin; tiles
// are (64 MI) x (64 NI) (SwiGLU: 128 columns of Y).
// SPLIT: the launch may hold split-contraction problems (the two-layout kernel).
template <bool EDGE, int MI = 4, int NI = 4, bool SPLIT = false>
__device__ __forceinline__ void locate(const GemmLaunch& L, int id, int epi, Problem& P, int64_t& m0, int64_t& n0) {
  P = pick_problem(L, L.nprob > 1 && id >= L.p[1].tile_begin);
  P.epi = epi;
  int local = id - P.tile_begin;
  if (SPLIT && P.ksplit > 1) {   // part-major: part j's tiles cover K range [j K/ks, (j+1) K/ks); ks is 2 or 4
    const int nt = P.tiles_m * P.tiles_n;
    const int j = (local >= nt) + (local >= 2 * nt) + (local >= 3 * nt);
    local -= j * nt;
    const int64_t kl = P.ksplit == 4 ? P.seg[0].K >> 2 : P.seg[0].K >> 1, k0 = (int64_t)j * kl;
    const int64_t da = P.layout == L_TN ? k0 * P.seg[0].lda : k0;   // elements along A's K
    const int64_t db = P.layout == L_NT ? k0 : k0 * P.seg[0].ldb;   // and along B's
    P.seg[0].a = static_cast<const uint16_t*>(P.seg[0].a) + da;
    P.seg[0].b = static_cast<const uint16_t*>(P.seg[0].b) + db;
    P.seg[0].K = kl;
    P.c32 += (int64_t)j * P.M * P.N;
  }
  int tm, tn;
  if (EDGE && P.edge_only) {   // right strip (whole-tile rows, ragged columns), then the bottom strip
    const int rn = P.tiles_n - P.full_n;
    const int right = P.full_m * rn;
    if (local < right) {
      tm = local / rn;
      tn = P.full_n + local % rn;
    } else {
      tm = P.full_m + (local - right) / P.tiles_n;
      tn = (local - right) % P.tiles_n;
    }
  } else {
    tile_coords(local, P.tiles_m, P.tiles_n, tm, tn);
  }
  m0 = (int64_t)tm * (64 * MI);
  n0 = (int64_t)tn * (epi == E_SWIGLU ? BN / 2 : 64 * NI);
}

// ---- schedule of the fast kernels ---------------------------------------------------------
// Workgroup g of G (one per CU) runs the whole tiles [g T / G, (g+1) T / G)
// of the launch's T tiles, with the K-stage stream running on from tile to
// tile.  Workgroup g sits on XCD g / (G / 8), so the tiles that run at the
// same time on one XCD are neighbours in the grouped tile order and share
// operand panels in its L2.
__device__ __forceinline__ int range_begin(int g, int T, int G) { return (int)((int64_t)g * T / G); }

// Whole tiles [t0, t0 + count) of a launch spread over G workgroups; this is
// workgroup g.  The K-stage stream runs on from tile to tile.  Tiles start
// their K loop (xcd/8) of the way in, wrapping around.
// Tile `tile` of a whole-tile launch.  In a half-tile tail launch
// (L.half_tail, MI == 2) the launch's tiles are the two 128-row halves of
// the 256-row tiles from L.half_base on; otherwise the problems' tile grids
// are in (64 MI) x (64 NI) tiles.
template <int MI, int NI, bool SPLIT = false>
__device__ __forceinline__ void locate_mi(const GemmLaunch& L, int tile, int epi, Problem& P, int64_t& m0,
                                          int64_t& n0) {
  if (MI == 2 && NI == 4 && L.half_tail) {
    locate<false>(L, L.half_base + (tile >> 1), epi, P, m0, n0);
    m0 += (tile & 1) * (BM / 2);
  } else {
    locate<false, MI, NI, SPLIT>(L, tile, epi, P, m0, n0);
  }
}

// Starting accumulator values of a fast-kernel tile: zeros, or with a column
// bias the bias of each lane's four columns in every block (alike for all
// rows; SwiGLU: the gate bias in gate blocks 0-3, the up bias in up blocks
// 4-7).  The fp32 accumulators then hold x W + b, the bias summed first.
// Columns past N (tiles overhanging the output, N a multiple of 8, so a
// lane's four columns are all inside or all outside) start at zero.
template <int EPI, int MI, int NI>
struct TileInit {
  f32x4 bj[2 * NI];
  __device__ __forceinline__ void operator()(f32x4 (&acc)[2 * MI][2 * NI]) const {
#pragma unroll
    for (int i = 0; i < 2 * MI; ++i)
#pragma unroll
      for (int j = 0; j < 2 * NI; ++j) acc[i][j] = bj[j];
  }
};

template <int EPI, int MI, int NI>
__device__ __forceinline__ TileInit<EPI, MI, NI> tile_init() {
  TileInit<EPI, MI, NI> t;
#pragma unroll
  for (int j = 0; j < 2 * NI; ++j) t.bj[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  return t;
}

template <int EPI, int MI, int NI>
__device__ __forceinline__ TileInit<EPI, MI, NI> tile_init(const Problem& P, int64_t n0) {
  constexpr bool dual = EPI == E_SWIGLU;
  TileInit<EPI, MI, NI> t;
  const int tid = tid_opaque(), lane = tid & 63, wn = (tid >> 6) & 1, g = lane >> 4;
#pragma unroll
  for (int j = 0; j < 2 * NI; ++j) {
    t.bj[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint16_t* b = static_cast<const uint16_t*>(dual && j >= 4 ? P.bias2 : P.bias);
    const int64_t col = n0 + (dual ? 64 * wn + 16 * (j & 3) : 32 * NI * wn + 16 * j) + 4 * g;
    if (b && col < P.N) {
      const uint2 w = *reinterpret_cast<const uint2*>(b + col);
      t.bj[j] = f32x4{bf2f((uint16_t)(w.x & 0xffffu)), bf2f((uint16_t)(w.x >> 16)), bf2f((uint16_t)(w.y & 0xffffu)),
                      bf2f((uint16_t)(w.y >> 16))};
    }
  }
  return t;
}

// A split-contraction part's tile: the fp32 accumulators straight to its
// partial plane (a lane's four consecutive columns of each block are one
// 16-byte store; N is a multiple of 8, so a group is all inside or all
// past the right edge).
template <int MI, int NI>
__device__ __forceinline__ void f32_epilogue(const Problem& P, int64_t m0, int64_t n0,
                                             const f32x4 (&acc)[2 * MI][2 * NI]) {
  const int tid = tid_opaque(), lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
  const int64_t m = m0 + 32 * MI * wm + (lane & 15);
  const int64_t n = n0 + 32 * NI * wn + 4 * (lane >> 4);
  float* c = P.c32 + m * P.N + n;
  const bool whole = m0 + 64 * MI <= P.M && n0 + 64 * NI <= P.N;
#pragma unroll
  for (int i = 0; i < 2 * MI; ++i)
#pragma unroll
    for (int j = 0; j < 2 * NI; ++j)
      if (whole || (m + 16 * i < P.M && n + 16 * j < P.N))
        *reinterpret_cast<f32x4*>(c + 16 * i * P.N + 16 * j) = acc[i][j];
}

// The fused store epilogues of the GEMM kernels (the default of tile_loop).
template <int EPI, int MI, int NI>
struct StoreEpilogue {
  __device__ __forceinline__ void operator()(const Problem& P, int64_t m0, int64_t n0,
                                            f32x4 (&acc)[2 * MI][2 * NI]) const {
    fast_epilogue<EPI, MI, NI>(P, m0, n0, acc,
                               std::make_integer_sequence<int, 2 * MI * (EPI == E_SWIGLU ? 2 : NI)>{});
  }
};

// The two-layout launch's epilogue: bf16 stores, or a split part's fp32 plane.
template <int MI, int NI>
struct DualEpilogue {
  __device__ __forceinline__ void operator()(const Problem& P, int64_t m0, int64_t n0,
                                            f32x4 (&acc)[2 * MI][2 * NI]) const {
    if (P.ksplit > 1) f32_epilogue<MI, NI>(P, m0, n0, acc);
    else fast_epilogue<E_STORE, MI, NI>(P, m0, n0, acc, std::make_integer_sequence<int, 2 * MI * NI>{});
  }
};

// Strided (STRIDED or L.strided): workgroup g runs tiles t0 + g,
// t0 + g + G, ... instead of a contiguous range, so that the tiles running
// at one time are neighbours in the grouped order (share operand panels in
// L2) however many tiles each workgroup runs; for launches of many tiles per
// workgroup.
template <int LAYOUT, int EPI, bool SEG2, int MI = 4, int NI = 4, bool STRIDED = false, int TM = TM_NONE,
          class Epi = StoreEpilogue<EPI, MI, NI>, bool SPLIT = false>
__device__ __forceinline__ void tile_loop(const GemmLaunch& L, int t0, int count, int g, int G, int xcd,
                                          const Epi& epilogue = Epi{}) {
  const bool strided = STRIDED || L.strided;
  const int ta = strided ? t0 + g : t0 + range_begin(g, count, G);
  const int tb = strided ? t0 + count : t0 + range_begin(g + 1, count, G);
  const int stride = strided ? G : 1;
  if (ta >= tb) return;
  constexpr bool DUAL = LAYOUT == L_NN && EPI == E_SWIGLU;
  const bool any_bias = L.p[0].bias || L.p[0].bias2 || (L.nprob > 1 && (L.p[1].bias || L.p[1].bias2));
  Pipe<LAYOUT, DUAL, SEG2, MI, NI> pipe;
  pipe.init_wave();
  int tile = ta;
  {
    Problem P;
    int64_t m0, n0;
    locate_mi<MI, NI, SPLIT>(L, tile, EPI, P, m0, n0);
    pipe.cur = pipe.make_streams(P, m0, n0, xcd);
  }
  pipe.prologue();
  for (;;) {
    const bool more = tile + stride < tb;
    if (more) {
      Problem Pn;
      int64_t m0n, n0n;
      locate_mi<MI, NI, SPLIT>(L, tile + stride, EPI, Pn, m0n, n0n);
      pipe.nxt = pipe.make_streams(Pn, m0n, n0n, xcd);
    } else {
      pipe.no_next();
    }
    f32x4 acc[2 * MI][2 * NI];
    if constexpr (LAYOUT == L_NN && EPI != E_CE_GRAD) {   // only column-parallel forwards take a bias
      // (One run_tile call: each call site inlines its own copy of the K loop.)
      TileInit<EPI, MI, NI> init = tile_init<EPI, MI, NI>();
      if (any_bias) {
        Problem P;
        int64_t m0, n0;
        locate_mi<MI, NI, SPLIT>(L, tile, EPI, P, m0, n0);
        init = tile_init<EPI, MI, NI>(P, n0);
      }
      pipe.template run_tile<TM>(acc, init);
    } else {
      pipe.template run_tile<TM>(acc, zero_acc<MI, NI>);
    }
    {
      Problem P;
      int64_t m0, n0;
      locate_mi<MI, NI, SPLIT>(L, tile, EPI, P, m0, n0);
      epilogue(P, m0, n0, acc);
    }
    if (!more) break;
    tile += stride;
    pipe.cur = pipe.nxt;
  }
  waitcnt<0, 0>();   // trailing (empty) copies retire before the workgroup ends
}

// Workgroup index with the workgroups of one XCD numbered consecutively (the
// hardware hands workgroup b to XCD b % 8), and the XCD.
__device__ __forceinline__ int wg_index(int& xcd) {
  const int G = gridDim.x;
  xcd = blockIdx.x & 7;
  return (G % 8 == 0) ? (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3) : blockIdx.x;
}

// Fast kernels: one per (operand layout, epilogue, K segments), so each role
// of the shard path is a distinct kernel in traces.  Tiles overhanging the
// matrix are masked at the stores (rows; columns in 8-wide chunks);
// aligned outputs; one workgroup per CU.  Starting the K loops of the
// XCDs at different points keeps the workgroups of one XCD in step (their
// shared operand panels stay in its L2).
template <int LAYOUT, int EPI, bool SEG2, int MI, int NI = 4>
__global__ __launch_bounds__(NTHREADS, 1) void gemm_bf16_kernel(const GemmLaunch L) {
  int xcd;
  const int g = wg_index(xcd);
  tile_loop<LAYOUT, EPI, SEG2, MI, NI>(L, 0, L.tiles, g, gridDim.x, xcd);
}

// Between two tile loops of different shapes in one workgroup: the first
// loop's last steps still issue (empty) copies into the ring, and the second
// loop splits the ring between the waves differently (a 128-row A tile is 2
// copy blocks per wave, a 256-row one 4), so every wave's copies must have
// landed before any wave issues the second loop's first ones.
__device__ __forceinline__ void ring_handover() {
  waitcnt<0, 0>();
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// Whole tiles, then the 128-row halves of the last round, in one launch: each
// workgroup runs its whole tiles (F) and then its half tile (H, at most one
// per workgroup), so it starts the half tile as soon as its own whole tiles
// (and its waves' last copies) are done.
template <int LAYOUT, int EPI>
__global__ __launch_bounds__(NTHREADS, 1) void gemm_bf16_tail_kernel(const GemmLaunch F, const GemmLaunch H) {
  int xcd;
  const int g = wg_index(xcd);
  tile_loop<LAYOUT, EPI, false, 4, 4>(F, 0, F.tiles, g, gridDim.x, xcd);
  ring_handover();
  tile_loop<LAYOUT, EPI, false, 2, 4>(H, 0, H.tiles, g, gridDim.x, xcd);
}

// Two problems of different operand layouts in one launch: workgroups
// [0, g0) run problem 0's tiles, the rest problem 1's (plain stores), each
// problem in its own tile shape.  Used when one problem alone cannot fill the
// CUs, e.g. the row-parallel backward, whose weight gradient has few, long
// tiles and whose input gradient has more, shorter ones.
template <int LA, int LB, int MIA = 4, int NIA = 4, int MIB = 4, int NIB = 4>
__global__ __launch_bounds__(NTHREADS, 1) void gemm_bf16_dual_kernel(const GemmLaunch L) {
  int xcd;
  const int g = wg_index(xcd);
  const int t1 = L.p[1].tile_begin;
  if (g < L.g0)
    tile_loop<LA, E_STORE, false, MIA, NIA, false, TM_NONE, DualEpilogue<MIA, NIA>, true>(L, 0, t1, g, L.g0, xcd);
  else
    tile_loop<LB, E_STORE, false, MIB, NIB, false, TM_NONE, DualEpilogue<MIB, NIB>, true>(
        L, t1, L.tiles - t1, g - L.g0, (int)gridDim.x - L.g0, xcd);
}

// Sum of a split problem's fp32 partial planes, in ascending part order, to
// bf16 (round to nearest even): thread i takes 8 consecutive columns of one
// row.  Both problems of a two-layout launch in one grid: rows of problem 0,
// then of problem 1 (n8[q] = N / 8 groups per row, g[q] groups in all).
struct SplitReduce {
  const float* c32[2];
  uint16_t* out[2];
  int64_t N[2], ldo[2], n8[2], groups[2];
  int ks[2];
};

template <int KS>
__device__ __forceinline__ void splitk_sum(const float* p, int64_t plane, f32x4& lo, f32x4& hi) {
  f32x4 l[KS], h[KS];
#pragma unroll
  for (int j = 0; j < KS; ++j) {   // all loads first: KS x 32 bytes in flight per lane
    l[j] = *reinterpret_cast<const f32x4*>(p + j * plane);
    h[j] = *reinterpret_cast<const f32x4*>(p + j * plane + 4);
  }
  lo = l[0];
  hi = h[0];
#pragma unroll
  for (int j = 1; j < KS; ++j) {
    lo += l[j];
    hi += h[j];
  }
}

__global__ __launch_bounds__(256) void splitk_reduce_kernel(const SplitReduce r) {
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int q = i >= r.groups[0] ? 1 : 0;
  if (q) i -= r.groups[0];
  if (i >= r.groups[q]) return;
  const int64_t n8 = q ? r.n8[1] : r.n8[0], N = q ? r.N[1] : r.N[0];
  const int64_t m = i / n8, n = (i - m * n8) * 8;
  const int64_t plane = (q ? r.groups[1] : r.groups[0]) * 8;
  const float* p = (q ? r.c32[1] : r.c32[0]) + m * N + n;
  f32x4 lo, hi;
  const int ks = q ? r.ks[1] : r.ks[0];
  if (ks == 4) splitk_sum<4>(p, plane, lo, hi);
  else splitk_sum<2>(p, plane, lo, hi);
  uint16_t* o = (q ? r.out[1] : r.out[0]) + m * (q ? r.ldo[1] : r.ldo[0]) + n;
  *reinterpret_cast<u32x4*>(o) = u32x4{pack_bf2(lo[0], lo[1]), pack_bf2(lo[2], lo[3]), pack_bf2(hi[0], hi[1]),
                                       pack_bf2(hi[2], hi[3])};
}

// Generic kernels: one tile per workgroup, any shape, bias, alignment.
template <int LAYOUT, int EPI, bool SEG2>
__global__ __launch_bounds__(NTHREADS, 1) void gemm_bf16_edge_kernel(const GemmLaunch L, int total_tiles) {
  const int id = xcd_remap(blockIdx.x, total_tiles);
  constexpr bool DUAL = LAYOUT == L_NN && EPI == E_SWIGLU;
  Problem P;
  int64_t m0, n0;
  locate<true>(L, id, EPI, P, m0, n0);
  f32x4 acc[8][8];
  Pipe<LAYOUT, DUAL, SEG2> pipe;
  pipe.init_wave();
  pipe.cur = pipe.make_streams(P, m0, n0);
  pipe.prologue();
  pipe.no_next();
  pipe.template run_tile<TM_ANY>(acc, zero_acc<4>);
  waitcnt<0, 0>();   // trailing (empty) copies land before the LDS is reused
  __syncthreads();
  generic_epilogue(P, m0, n0, acc);
}

// Row statistics of one 16-row block (I) of a wave's (32 MI) x 128 logit
// block: max and sum exp(z - max) over the valid columns (a lane holds 32 of
// its row's columns, 16 j + 4 (lane / 16) + e; the four 16-lane rows of the
// wave hold the rest), the target logit if this lane holds it, and the
// per-wave results in LDS for the cross-wave merge.
template <int I, int MI>
__device__ __forceinline__ void ce_rows(const CEArgs& a, f32x4 (&acc)[2 * MI][8], int64_t m0, int64_t wcol,
                                        int nvalid, float* ws_tgt, TPS_LDS float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wm = wave >> 1, wn = wave & 1;
  const int g = lane >> 4;
  const int rl = 32 * MI * wm + 16 * I + (lane & 15);
  const int64_t m = m0 + rl;
  const int lim = nvalid - 4 * g;     // column 16 j + 4 g + e of this lane is valid iff 16 j + e < lim
  float mx = -INFINITY;
  if (nvalid >= 128) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) mx = fmaxf(mx, acc[I][j][e]);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) mx = fmaxf(mx, 16 * j + e < lim ? acc[I][j][e] : -INFINITY);
  }
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  float s = 0.f;
  if (nvalid >= 128) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) s += __expf(acc[I][j][e] - mx);
  } else if (mx > -INFINITY) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) s += 16 * j + e < lim ? __expf(acc[I][j][e] - mx) : 0.f;
  }
  s += __shfl_xor(s, 16);
  s += __shfl_xor(s, 32);
  if (m < a.M) {
    const int64_t d64 = (int64_t)a.target[m] - a.v0 - wcol;   // target column relative to the wave
    if (d64 >= 0 && d64 < nvalid) {
      const int dd = (int)d64 - 4 * g;
      float tv = 0.f;
      bool mine = false;
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool hit = 16 * j + e == dd;
          tv = hit ? acc[I][j][e] : tv;
          mine = mine || hit;
        }
      if (mine) ws_tgt[m] = tv;
    }
  }
  if (g == 0) {
    red[(wn * 256 + rl) * 2 + 0] = mx;
    red[(wn * 256 + rl) * 2 + 1] = s;
  }
}

template <int MI, int... Is>
__device__ __forceinline__ void ce_rows_seq(const CEArgs& a, f32x4 (&acc)[2 * MI][8], int64_t m0, int64_t wcol,
                                            int nvalid, float* ws_tgt, TPS_LDS float* red,
                                            std::integer_sequence<int, Is...>) {
  (ce_rows<Is, MI>(a, acc, m0, wcol, nvalid, ws_tgt, red), ...);
}

// Cross-wave merge buffer of the CE epilogue, [2 column waves][256 rows][max,
// sum].  Its own array: in the persistent kernel the LDS ring is already
// filling with the next tile's stages while the epilogue runs.
__shared__ __attribute__((aligned(16))) float ce_red[2 * 256 * 2];

// LDS-only workgroup barrier: this wave's LDS accesses are complete
// (lgkmcnt(0)), the global->LDS copies of later stages stay in flight.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ---- vocab-parallel LM head: logits tile -> (max, sum exp) partials ---------------------
// Epilogue of the logit tile (tm, tn): tokens [m0, m0 + 64 MI) and shard
// vocab columns [n0, n0 + 256).  Writes ws_ms[tn][m] = (tile max, sum
// exp(z - tile max)) and, for the tile holding a token's target,
// ws_tgt[m] = z[m, target - v0].  The logits never leave the registers.
template <int MI>
struct CeEpilogue {
  CEArgs a;
  int tiles_n;
  __device__ __forceinline__ void operator()(const Problem&, int64_t m0, int64_t n0, f32x4 (&acc)[2 * MI][8]) const {
    const int wn = (threadIdx.x >> 6) & 1;
    const int64_t wcol = n0 + 128 * wn;                 // first column of this wave
    // number of valid columns of this wave, in [0, 128]
    const int nvalid = (int)max<int64_t>(0, min<int64_t>(128, a.Vr - wcol));
    float* ws_ms = a.ws;
    float* ws_tgt = a.ws + 2 * (int64_t)tiles_n * a.M;
    TPS_LDS float* red = (TPS_LDS float*)ce_red;
    ce_rows_seq<MI>(a, acc, m0, wcol, nvalid, ws_tgt, red, std::make_integer_sequence<int, 2 * MI>{});
    lds_barrier();
    const int rl = threadIdx.x;
    const int64_t m = m0 + rl;
    const int64_t tn = n0 / BN;
    if (rl < 64 * MI && m < a.M) {
      const float ma = red[rl * 2], sa = red[rl * 2 + 1];
      const float mb = red[(256 + rl) * 2], sb = red[(256 + rl) * 2 + 1];
      const float mm = fmaxf(ma, mb);
      const float ss = sa * __expf(ma - mm) + sb * __expf(mb - mm);
      ws_ms[2 * (tn * a.M + m) + 0] = mm;
      ws_ms[2 * (tn * a.M + m) + 1] = ss;
    }
    lds_barrier();   // red is rewritten by the next tile's epilogue
  }
};

// Persistent logit-tile kernel: workgroup g of G runs the tiles g, g + G,
// ... of the launch (about 9 per workgroup for an 8192 x 18992 shard), the
// next tile's first stages loading during this tile's epilogue (MI = 2: the
// 128-row halves of a half-tile tail launch).  KTAIL: the hidden size ends
// inside a 32-deep stage (the loop that zeroes its tail).
template <int MI, bool KTAIL>
__global__ __launch_bounds__(NTHREADS, 1) void ce_tile_kernel(const GemmLaunch L, const CEArgs a, int tiles_n) {
  int xcd;
  const int g = wg_index(xcd);
  tile_loop<L_NT, E_STORE, false, MI, 4, true, KTAIL ? TM_TAIL : TM_NONE>(L, 0, L.tiles, g, gridDim.x, xcd,
                                                                        CeEpilogue<MI>{a, tiles_n});
}

// The whole tiles (F) and then the 128-row halves of the last round (H) in
// one launch, as gemm_bf16_tail_kernel does for the GEMMs.
template <bool KTAIL>
__global__ __launch_bounds__(NTHREADS, 1) void ce_tile_tail_kernel(const GemmLaunch F, const GemmLaunch H,
                                                                   const CEArgs a, int tiles_n) {
  constexpr int TM = KTAIL ? TM_TAIL : TM_NONE;
  int xcd;
  const int g = wg_index(xcd);
  tile_loop<L_NT, E_STORE, false, 4, 4, true, TM>(F, 0, F.tiles, g, gridDim.x, xcd, CeEpilogue<4>{a, tiles_n});
  ring_handover();
  tile_loop<L_NT, E_STORE, false, 2, 4, false, TM>(H, 0, H.tiles, g, gridDim.x, xcd, CeEpilogue<2>{a, tiles_n});
}

// Combine the per-tile partials of each token: 8 lanes per token, lane j
// folding tiles j, j + 8, ... in ascending order, then the lanes' pairs
// combined by a butterfly over lane ^ 1, ^ 2, ^ 4.  Max and the two-term sum
// are commutative, so every lane ends with the same bits and the result is
// fixed (it does not depend on scheduling).
__device__ __forceinline__ void lse_fold(float& m, float& s, float mt, float st) {
  const float mn = fmaxf(m, mt);
  s = mn == -INFINITY ? 0.f : s * __expf(m - mn) + st * __expf(mt - mn);
  m = mn;
}

__global__ __launch_bounds__(256) void ce_merge_kernel(const CEArgs a, int tiles_n) {
  const int64_t m = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 3;
  const int j = threadIdx.x & 7;
  const int64_t mr = m < a.M ? m : a.M - 1;   // past the end: a repeat, kept in the shuffles, not written
  const float* ws_ms = a.ws;
  const float* ws_tgt = a.ws + 2 * (int64_t)tiles_n * a.M;
  float mm = -INFINITY, ss = 0.f;
  for (int t = j; t < tiles_n; t += 8) {
    const float* p = ws_ms + 2 * ((int64_t)t * a.M + mr);
    lse_fold(mm, ss, p[0], p[1]);
  }
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) {
    const float mo = __shfl_xor(mm, o), so = __shfl_xor(ss, o);
    lse_fold(mm, ss, mo, so);
  }
  if (m >= a.M || j != 0) return;
  const int64_t tg = (int64_t)a.target[m] - a.v0;
  a.out_max[m] = mm;
  a.out_sumexp[m] = ss;
  a.out_tgt[m] = (tg >= 0 && tg < a.Vr) ? ws_tgt[m] : 0.f;
}

}  // namespace

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// The tiles of this problem may take the fast kernel (16-byte aligned
// outputs and, with a bias, an NN product with 8-byte aligned bias vectors;
// K-contiguous operands ending on a 32-deep stage: the fast kernels carry no
// K-tail code).
bool fast_ok(const Problem& P) {
  if ((P.bias || P.bias2) && (P.layout != L_NN || P.epi == E_CE_GRAD)) return false;
  if ((reinterpret_cast<uintptr_t>(P.bias) & 7) || (reinterpret_cast<uintptr_t>(P.bias2) & 7)) return false;
  for (int i = 0; i < P.nseg; ++i)
    if (P.layout != L_TN && P.seg[i].K % BK != 0) return false;
  if (!aligned16(P.c) || (P.ldc & 7)) return false;
  if (P.epi != E_STORE && (!aligned16(P.pre) || (P.ldpre & 7))) return false;
  if (P.epi == E_SWIGLU && (P.N & 7)) return false;
  return true;
}

// FAST: the fast kernel's tiles; else edge tiles.
template <bool FAST>
hipError_t dispatch(const GemmLaunch& L, int total, int grid, hipStream_t s) {
  const dim3 g(grid), block(NTHREADS);
  const int layout = L.p[0].layout, epi = L.p[0].epi;
  const bool seg2 = L.p[0].nseg > 1 || (L.nprob > 1 && L.p[1].nseg > 1);
#define TPS_LAUNCH(LY, EP, S2)                                                                      \
  do {                                                                                              \
    if constexpr (FAST) {                                                                           \
      hipLaunchKernelGGL((gemm_bf16_kernel<LY, EP, S2, 4>), g, block, 0, s, L);                     \
    } else {                                                                                        \
      hipLaunchKernelGGL((gemm_bf16_edge_kernel<LY, EP, S2>), g, block, 0, s, L, total);            \
    }                                                                                               \
  } while (0)
  if (layout == L_NN && epi == E_SWIGLU) TPS_LAUNCH(L_NN, E_SWIGLU, false);
  else if (layout == L_NN && epi == E_GELU) TPS_LAUNCH(L_NN, E_GELU, false);
  else if (layout == L_NN) TPS_LAUNCH(L_NN, E_STORE, false);
  else if (layout == L_NT && epi == E_CE_GRAD) TPS_LAUNCH(L_NT, E_CE_GRAD, false);
  else if (layout == L_NT && seg2) TPS_LAUNCH(L_NT, E_STORE, true);
  else if (layout == L_NT) TPS_LAUNCH(L_NT, E_STORE, false);
  else TPS_LAUNCH(L_TN, E_STORE, false);
#undef TPS_LAUNCH
  return hipGetLastError();
}

}  // namespace

// Stages of a problem's tile rounded up to the ring depth (its MFMA time).
int64_t tile_stages(const Problem& P) {
  int64_t nk = (P.seg[0].K + BK - 1) / BK;
  if (P.nseg > 1) nk += (P.seg[1].K + BK - 1) / BK;
  return (nk + NSTAGE - 1) / NSTAGE * NSTAGE;
}

// (64 mi) x (64 ni) tiles covering a problem's output (the last row and
// column of tiles may overhang it).
int64_t tiles_of(const Problem& P, int mi, int ni) {
  const int64_t bm = 64 * mi, bn = 64 * ni;
  return (P.M + bm - 1) / bm * ((P.N + bn - 1) / bn);
}

// Problem 0 on g0 workgroups and problem 1 on the rest of `cus`, one launch:
// the best g0 (the smallest of the best) and its makespan (in units of a
// tile's cost).  Problem 0's rounds times its tile cost, f0(g), never grows
// with g and problem 1's, f1(g), never shrinks, so the best g is the first
// one with f0 <= f1 or the one before it; on a run of equal makespans below
// that point the makespan is f0, and a second search finds the run's start.
int64_t dual_split(int64_t t0, int64_t s0, int64_t t1, int64_t s1, int cus, int& g0) {
  g0 = 1;
  if (cus < 2) return INT64_MAX;
  auto f0 = [&](int64_t g) { return (t0 + g - 1) / g * s0; };
  auto f1 = [&](int64_t g) { return (t1 + cus - g - 1) / (cus - g) * s1; };
  int lo = 1, hi = cus - 1;
  while (lo < hi) {   // first g in [1, cus - 1] with f0(g) <= f1(g) (cus - 1 if none)
    const int mid = (lo + hi) / 2;
    if (f0(mid) <= f1(mid)) hi = mid;
    else lo = mid + 1;
  }
  int64_t best = std::max(f0(lo), f1(lo));
  g0 = lo;
  if (lo > 1 && f0(lo - 1) <= best) {   // below lo the makespan is f0, never growing with g
    best = f0(lo - 1);
    int a = 1, b = lo - 1;   // first g with f0(g) == best
    while (a < b) {
      const int mid = (a + b) / 2;
      if (f0(mid) <= best) b = mid;
      else a = mid + 1;
    }
    g0 = a;
  }
  return best;
}

// Tile pairings of the one-launch row backward: (MI, NI) of problem 0, then of problem 1.
constexpr int kGeoN = 7;
constexpr int kGeo[kGeoN][4] = {{4, 4, 4, 4}, {3, 4, 4, 3}, {3, 3, 2, 3}, {2, 2, 2, 3},
                                {2, 2, 4, 4}, {2, 3, 4, 3}, {2, 3, 2, 3}};

// Cost model of the two-layout launch, in shader cycles.  A 32-deep stage of a
// (64 MI) x (64 NI) tile: 64 cycles per 16 x 16 MFMA block and wave, 47/4 per
// KiB it copies (a TN tile copies both 256-wide MN-contiguous panels, 32 KiB,
// whatever its width; an NT tile 4 KiB per 16-row block of either operand),
// and 100 of fixed work (waits, barrier); no stage takes under 900 cycles,
// the time the four-stage ring needs to cover a load's latency (small tiles
// hit that floor: a 128 x 128 tile's stages take ~30% longer than their MFMA
// and copy counts say).  A tile's epilogue: 8800 cycles for
// a 256 x 256 tile's bf16 stores, 13200 for a split part's fp32 plane, scaled
// by area.  Fit to per-step and per-tile timestamps (s_memtime) of the 256 x
// 256 kernels (~1.5 k cycles per stage, ~8.8 k per epilogue); the copy term
// is what makes narrow TN tiles dearer than their MFMA count says (they run
// the full panels' copies for fewer MFMAs).  Split contractions add the
// reduction launch: its planes read and its output written at ~5 TB/s (2439
// bytes per cycle at ~2.05 GHz), plus ~2 us for the launch.  Parts must hold
// whole 32-deep stages.
constexpr int64_t EPI_BF16 = 8800, EPI_F32 = 13200;
constexpr int64_t REDUCE_LAUNCH = 4200;
constexpr int64_t REDUCE_BYTES_PER_CYCLE = 2439;
constexpr int64_t STAGE_FLOOR = 900;

int64_t stage_cycles(bool tn, int mi, int ni) {
  const int64_t kib = tn ? 32 : 4 * (mi + ni);
  return std::max<int64_t>(64 * mi * ni + kib * 47 / 4 + 100, STAGE_FLOOR);
}
int64_t epi_cycles(bool f32, int mi, int ni) { return (f32 ? EPI_F32 : EPI_BF16) * mi * ni / 16; }

size_t split_bytes(const Problem& P, int ks) {
  return ks > 1 ? ((size_t)ks * (size_t)P.M * (size_t)P.N * 4 + 255) / 256 * 256 : 0;
}

int dual_plan(const GemmLaunch& L, int cus, int& g0, int64_t& t0, int64_t& t1, int& ks0, int& ks1,
              size_t& split_need) {
  ks0 = ks1 = 1;
  split_need = 0;
  if (!(L.nprob == 2 && L.p[0].layout == L_TN && L.p[1].layout == L_NT && L.p[0].epi == E_STORE &&
        L.p[1].epi == E_STORE && L.p[0].nseg == 1 && L.p[1].nseg == 1 && fast_ok(L.p[0]) && fast_ok(L.p[1]) &&
        (L.p[0].N & 7) == 0 && (L.p[1].N & 7) == 0 && cus % 8 == 0))
    return -1;
  const int64_t s0 = tile_stages(L.p[0]), s1 = tile_stages(L.p[1]);
  const int64_t n0 = tiles_of(L.p[0], 4, 4), n1 = tiles_of(L.p[1], 4, 4);
  const int64_t apart = (n0 + cus - 1) / cus * (s0 * stage_cycles(true, 4, 4) + epi_cycles(false, 4, 4)) +
                        (n1 + cus - 1) / cus * (s1 * stage_cycles(false, 4, 4) + epi_cycles(false, 4, 4));
  const bool can_split = L.split_ws != nullptr && (reinterpret_cast<uintptr_t>(L.split_ws) & 15) == 0;
  int best = -1;
  int64_t best_cost = apart, best_tiles = 0;
  for (int k0 = 1; k0 <= 4; k0 *= 2) {
    for (int k1 = 1; k1 <= 4; k1 *= 2) {
      const bool split = k0 > 1 || k1 > 1;
      if (split && !can_split) continue;
      if ((k0 > 1 && L.p[0].seg[0].K % (BK * k0) != 0) || (k1 > 1 && L.p[1].seg[0].K % (BK * k1) != 0)) continue;
      const size_t need = split_bytes(L.p[0], k0) + split_bytes(L.p[1], k1);
      if (split && need > L.split_bytes) continue;
      const int64_t ss0 = (s0 / k0 + NSTAGE - 1) / NSTAGE * NSTAGE, ss1 = (s1 / k1 + NSTAGE - 1) / NSTAGE * NSTAGE;
      int64_t red = 0;
      if (split) {
        for (int q = 0; q < 2; ++q) {
          const int k = q ? k1 : k0;
          if (k > 1) red += (int64_t)((4 * k + 2) * L.p[q].M * L.p[q].N / REDUCE_BYTES_PER_CYCLE);
        }
        red += REDUCE_LAUNCH;
      }
      for (int c = 0; c < kGeoN; ++c) {
        const int64_t a = tiles_of(L.p[0], kGeo[c][0], kGeo[c][1]) * k0;
        const int64_t b = tiles_of(L.p[1], kGeo[c][2], kGeo[c][3]) * k1;
        if (a + b >= INT_MAX) continue;
        int g = 1;
        const int64_t w0 = ss0 * stage_cycles(true, kGeo[c][0], kGeo[c][1]) + epi_cycles(k0 > 1, kGeo[c][0], kGeo[c][1]);
        const int64_t w1 = ss1 * stage_cycles(false, kGeo[c][2], kGeo[c][3]) + epi_cycles(k1 > 1, kGeo[c][2], kGeo[c][3]);
        const int64_t m = dual_split(a, w0, b, w1, cus, g) + red;
        // Costs within 2% of each other are a tie (the model's resolution: it puts 128 x 128
        // weight-gradient tiles beside 256 x 256 level with 128 x 192 beside 256 x 192 for the
        // attention output projection's backward, which measure 106 and 97 us); a tie goes to
        // the plan with fewer tiles.
        bool take = m < best_cost;
        if (best >= 0 && (m > best_cost ? m - best_cost : best_cost - m) * 50 <= best_cost)
          take = a + b < best_tiles || (a + b == best_tiles && m < best_cost);
        if (take) {
          best_cost = m;
          best_tiles = a + b;
          best = c;
          g0 = g;
          t0 = a;
          t1 = b;
          ks0 = k0;
          ks1 = k1;
          split_need = need;
        }
      }
    }
  }
  return best;
}

int dual_plan(const GemmLaunch& L, int cus, int& g0, int64_t& t0, int64_t& t1) {
  GemmLaunch U = L;
  U.split_ws = nullptr;
  U.split_bytes = 0;
  int ks0 = 1, ks1 = 1;
  size_t need = 0;
  return dual_plan(U, cus, g0, t0, t1, ks0, ks1, need);
}

hipError_t launch_gemm_bf16(GemmLaunch& L, hipStream_t s) {
  int dev = 0, cus = 256;
  {
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
  }
  // The row-parallel backward pair (TN weight gradient, NT input gradient) in
  // one launch, when sharing the CUs beats running them one after the other.
  // Tile shapes per problem, from a short list: 256 x 256 for both; 192 x 256
  // weight-gradient tiles beside 256 x 192 input-gradient tiles (for
  // 1536 x 4096 over 8192 tokens and 8192 x 1536 over 4096: 128 + 256 tiles
  // that give every CU the same work, where 96 + 192 256 x 256 tiles leave a
  // quarter of the CU-time idle); 192 x 192 beside 128 x 192 (for a narrow
  // 512 x 4096 weight gradient over 8192 tokens: 66 tiles instead of 32).
  // Tiles may overhang the outputs (masked stores; N a multiple of 8).  A
  // tile's cost is its stages' cycles plus its epilogue's (the cycle model
  // above).  (128 x 256 input-gradient tiles beside 192 x 256 balance the
  // first case too but ran slower: a stage's barrier and copies then serve
  // half the MFMAs.)
  {
    int g0 = 1, ks[2] = {1, 1};
    int64_t t0 = 0, t1 = 0;
    size_t need = 0;
    const int best = dual_plan(L, cus, g0, t0, t1, ks[0], ks[1], need);
    if (best >= 0) {
      GemmLaunch D = L;
      float* part = L.split_ws;
      for (int i = 0; i < 2; ++i) {
        const int64_t bm = 64 * kGeo[best][2 * i], bn = 64 * kGeo[best][2 * i + 1];
        D.p[i].tiles_m = (int)((L.p[i].M + bm - 1) / bm);
        D.p[i].tiles_n = (int)((L.p[i].N + bn - 1) / bn);
        D.p[i].edge_only = 0;
        D.p[i].ksplit = ks[i];
        D.p[i].c32 = ks[i] > 1 ? part : nullptr;
        if (ks[i] > 1) part += split_bytes(L.p[i], ks[i]) / sizeof(float);
      }
      D.p[0].tile_begin = 0;
      D.p[1].tile_begin = (int)t0;
      D.tiles = (int)(t0 + t1);
      D.g0 = g0;
      D.half_tail = 0;
      D.strided = 1;   // measured faster here (one-problem launches of two tiles per CU ran slower strided)
      if (best == 0)
        hipLaunchKernelGGL((gemm_bf16_dual_kernel<L_TN, L_NT>), dim3(cus), dim3(NTHREADS), 0, s, D);
      else if (best == 1)
        hipLaunchKernelGGL((gemm_bf16_dual_kernel<L_TN, L_NT, 3, 4, 4, 3>), dim3(cus), dim3(NTHREADS), 0, s, D);
      else if (best == 2)
        hipLaunchKernelGGL((gemm_bf16_dual_kernel<L_TN, L_NT, 3, 3, 2, 3>), dim3(cus), dim3(NTHREADS), 0, s, D);
      else if (best == 3)
        hipLaunchKernelGGL((gemm_bf16_dual_kernel<L_TN, L_NT, 2, 2, 2, 3>), dim3(cus), dim3(NTHREADS), 0, s, D);
      else if (best == 4)
        hipLaunchKernelGGL((gemm_bf16_dual_kernel<L_TN, L_NT, 2, 2, 4, 4>), dim3(cus), dim3(NTHREADS), 0, s, D);
      else if (best == 5)
        hipLaunchKernelGGL((gemm_bf16_dual_kernel<L_TN, L_NT, 2, 3, 4, 3>), dim3(cus), dim3(NTHREADS), 0, s, D);
      else
        hipLaunchKernelGGL((gemm_bf16_dual_kernel<L_TN, L_NT, 2, 3, 2, 3>), dim3(cus), dim3(NTHREADS), 0, s, D);
      if (ks[0] > 1 || ks[1] > 1) {
        SplitReduce r = {};
        for (int i = 0; i < 2; ++i) {
          r.ks[i] = ks[i];
          r.c32[i] = D.p[i].c32;
          r.out[i] = static_cast<uint16_t*>(D.p[i].c);
          r.N[i] = D.p[i].N;
          r.ldo[i] = D.p[i].ldc;
          r.n8[i] = D.p[i].N / 8;
          r.groups[i] = ks[i] > 1 ? D.p[i].M * r.n8[i] : 0;
        }
        if (r.groups[0] == 0) {   // problem 1 only: its rows first
          std::swap(r.ks[0], r.ks[1]);
          std::swap(r.c32[0], r.c32[1]);
          std::swap(r.out[0], r.out[1]);
          std::swap(r.N[0], r.N[1]);
          std::swap(r.ldo[0], r.ldo[1]);
          std::swap(r.n8[0], r.n8[1]);
          std::swap(r.groups[0], r.groups[1]);
        }
        const int64_t total = r.groups[0] + r.groups[1];
        hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, r);
      }
      return hipGetLastError();
    }
  }
  // Otherwise problems of one launch must share the operand layout and the
  // epilogue; else split.  Only L_NN carries activation epilogues.
  if (L.nprob > 1 && (L.p[0].layout != L.p[1].layout || L.p[0].epi != L.p[1].epi)) {
    GemmLaunch a = L, b = L;
    a.nprob = 1;
    b.p[0] = L.p[1];
    b.nprob = 1;
    hipError_t e = launch_gemm_bf16(a, s);
    return e != hipSuccess ? e : launch_gemm_bf16(b, s);
  }
  bool fast = true;
  for (int i = 0; i < L.nprob; ++i) fast = fast && fast_ok(L.p[i]);
  // Narrower tiles for plain-store launches whose 256 x 256 tiles would
  // leave CUs idle: weight gradients (TN) in 256 x 192 or 192 x 192 tiles,
  // NN / NT products in 128 x 192 tiles.  A launch's cost is taken as its
  // rounds times (MFMA blocks per wave + 2), the 2 standing for a K stage's
  // fixed barrier and copy work (256 x 256: 18; 256 x 192: 14; 192 x 192: 11;
  // 128 x 192: 8; a 256 x 256 launch whose last round runs as 128-row halves:
  // 18 per whole round + 10).  Examples: a SwiGLU column backward with two
  // 4096 x 1536 weight gradients, 192 whole tiles (75 % of 256 CUs) or 256
  // tiles of 256 x 192 in one round; an 8192 x 768 projection, 96 whole tiles
  // or 256 tiles of 128 x 192.  Every tile then takes the fast kernel
  // (columns past N are masked in 8-column chunks).
  if (fast && L.p[0].epi == E_STORE && L.p[0].nseg == 1 && (L.nprob == 1 || L.p[1].nseg == 1)) {
    const int lay = L.p[0].layout;
    static constexpr int kTN[2][2] = {{4, 3}, {3, 3}};
    static constexpr int kAK[1][2] = {{2, 3}};   // K-contiguous A (NN, NT)
    const int ncand = lay == L_TN ? 2 : 1;
    bool n8 = true, half_ok = lay != L_TN;
    int64_t n44 = 0;
    for (int i = 0; i < L.nprob; ++i) {
      const Problem& P = L.p[i];
      n8 = n8 && (P.N & 7) == 0;
      half_ok = half_ok && P.M % BM == 0;
      n44 += (P.M + BM - 1) / BM * ((P.N + BN - 1) / BN);
    }
    const int64_t rem44 = n44 % cus;
    int64_t best_cost = (half_ok && n44 > cus && rem44 > 0 && 2 * rem44 <= cus) ? n44 / cus * 18 + 10
                                                                                 : (n44 + cus - 1) / cus * 18;
    int best = -1;
    for (int c = 0; c < ncand && n8; ++c) {
      const int mi = lay == L_TN ? kTN[c][0] : kAK[c][0], ni = lay == L_TN ? kTN[c][1] : kAK[c][1];
      int64_t n = 0;
      for (int i = 0; i < L.nprob; ++i)
        n += (L.p[i].M + 64 * mi - 1) / (64 * mi) * ((L.p[i].N + 64 * ni - 1) / (64 * ni));
      const int64_t cost = (n + cus - 1) / cus * (mi * ni + 2);
      if (n < INT_MAX && cost < best_cost) {
        best_cost = cost;
        best = c;
      }
    }
    if (best >= 0) {
      const int mi = lay == L_TN ? kTN[best][0] : kAK[best][0], ni = lay == L_TN ? kTN[best][1] : kAK[best][1];
      GemmLaunch G = L;
      int nt = 0;
      for (int i = 0; i < L.nprob; ++i) {
        G.p[i].tiles_m = (int)((L.p[i].M + 64 * mi - 1) / (64 * mi));
        G.p[i].tiles_n = (int)((L.p[i].N + 64 * ni - 1) / (64 * ni));
        G.p[i].tile_begin = nt;
        G.p[i].edge_only = 0;
        nt += G.p[i].tiles_m * G.p[i].tiles_n;
      }
      G.tiles = nt;
      G.half_tail = 0;
      G.strided = nt >= 3 * cus;
      const dim3 grid(std::min(nt, cus)), block(NTHREADS);
      if (lay == L_TN && mi == 4)
        hipLaunchKernelGGL((gemm_bf16_kernel<L_TN, E_STORE, false, 4, 3>), grid, block, 0, s, G);
      else if (lay == L_TN)
        hipLaunchKernelGGL((gemm_bf16_kernel<L_TN, E_STORE, false, 3, 3>), grid, block, 0, s, G);
      else if (lay == L_NN)
        hipLaunchKernelGGL((gemm_bf16_kernel<L_NN, E_STORE, false, 2, 3>), grid, block, 0, s, G);
      else
        hipLaunchKernelGGL((gemm_bf16_kernel<L_NT, E_STORE, false, 2, 3>), grid, block, 0, s, G);
      return hipGetLastError();
    }
  }
  GemmLaunch F = L, E = L;   // fast-kernel tiles, remaining tiles (generic kernel)
  int nf = 0, ne = 0;
  for (int i = 0; i < L.nprob; ++i) {
    const Problem& P = L.p[i];
    const int64_t bn = (P.epi == E_SWIGLU) ? BN / 2 : BN;
    const int tm = (int)((P.M + BM - 1) / BM), tn = (int)((P.N + bn - 1) / bn);
    // The fast kernel masks rows past M, and columns past N in whole 8-column
    // chunks: every tile row, and the last tile column when N % 8 == 0.
    const int fm = fast ? tm : 0, fn = fast ? ((P.N & 7) == 0 ? tn : (int)(P.N / bn)) : 0;
    F.p[i].tiles_m = fm;
    F.p[i].tiles_n = fn;
    F.p[i].tile_begin = nf;
    F.p[i].edge_only = 0;
    nf += fm * fn;
    E.p[i].tiles_m = tm;
    E.p[i].tiles_n = tn;
    E.p[i].full_m = fm;
    E.p[i].full_n = fn;
    E.p[i].edge_only = fast ? 1 : 0;
    E.p[i].tile_begin = ne;
    ne += tm * tn - fm * fn;
  }
  if (nf > 0) {
    // A last round that would leave over half the CUs idle runs as 128-row
    // half tiles instead (layouts with a K-contiguous A and one segment; M a
    // multiple of 256, so that no half tile starts past the last row).
    bool half_ok = L.p[0].layout != L_TN && L.p[0].nseg == 1 && (L.nprob == 1 || L.p[1].nseg == 1);
    for (int i = 0; i < L.nprob; ++i) half_ok = half_ok && L.p[i].M % BM == 0;
    const int rem = nf % cus;
    const int tail = (half_ok && nf > cus && rem > 0 && 2 * rem <= cus) ? rem : 0;
    F.tiles = nf - tail;
    F.half_tail = 0;
    F.strided = F.tiles >= 3 * cus;   // many tiles per workgroup: keep the running tiles adjacent
    if (tail > 0) {   // F.tiles >= cus: the combined launch has one workgroup per CU
      GemmLaunch H = F;
      H.tiles = 2 * tail;
      H.half_base = nf - tail;
      H.half_tail = 1;
      H.strided = 0;
      const int layout = L.p[0].layout, epi = L.p[0].epi;
      const dim3 grid(cus), block(NTHREADS);
      if (layout == L_NN && epi == E_SWIGLU)
        hipLaunchKernelGGL((gemm_bf16_tail_kernel<L_NN, E_SWIGLU>), grid, block, 0, s, F, H);
      else if (layout == L_NN && epi == E_GELU)
        hipLaunchKernelGGL((gemm_bf16_tail_kernel<L_NN, E_GELU>), grid, block, 0, s, F, H);
      else if (layout == L_NN)
        hipLaunchKernelGGL((gemm_bf16_tail_kernel<L_NN, E_STORE>), grid, block, 0, s, F, H);
      else if (epi == E_CE_GRAD)
        hipLaunchKernelGGL((gemm_bf16_tail_kernel<L_NT, E_CE_GRAD>), grid, block, 0, s, F, H);
      else
        hipLaunchKernelGGL((gemm_bf16_tail_kernel<L_NT, E_STORE>), grid, block, 0, s, F, H);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    } else {
      hipError_t e = dispatch<true>(F, F.tiles, std::min(F.tiles, cus), s);
      if (e != hipSuccess) return e;
    }
  }
  if (ne > 0) return dispatch<false>(E, ne, ne, s);
  return hipSuccess;
}

}  // namespace tps

// Scratch of the allocation-free CE entry point: the per-tile (max, sum exp)
// pairs and target logits that tp_vocab_ce_partials keeps in the caller's
// workspace.  Each GPU the library runs on holds its own copy until the
// process ends.  Host code never uses this name as an address (on the host it
// is only a stand-in for the symbol): the device address comes from
// hipGetSymbolAddress, once per device.
static __device__ __align__(256) char scratch[tps::kCeScratchBytes];

namespace tps {

hipError_t ce_scratch(float** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* ptrs[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));   // with `dev` current: this device's copy
    if (e != hipSuccess) return e;
    ptrs[dev] = p;
  }
  *out = static_cast<float*>(ptrs[dev]);
  return hipSuccess;
}

size_t ce_workspace_bytes(int64_t M, int64_t Vr) {
  const int64_t tiles_n = (Vr + BN - 1) / BN;
  return (size_t)(2 * tiles_n * M + M) * sizeof(float);
}

hipError_t launch_ce_partials(const CEArgs& a, hipStream_t s) {
  int dev = 0, cus = 256;
  {
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
  }
  const int tiles_m = (int)((a.M + BM - 1) / BM);
  const int tiles_n = (int)((a.Vr + BN - 1) / BN);
  GemmLaunch L = {};
  L.nprob = 1;
  Problem& P = L.p[0];
  P.M = a.M;
  P.N = a.Vr;
  P.seg[0] = Seg{a.H, a.W, a.ldh, a.ldw, a.K};
  P.nseg = 1;
  P.layout = L_NT;
  P.epi = E_STORE;
  P.tiles_m = tiles_m;
  P.tiles_n = tiles_n;
  const int nt = tiles_m * tiles_n;
  // A last round that would leave over half the CUs idle runs as 128-row
  // half tiles (M a multiple of 256, so that no half tile starts past the
  // last row).
  const int rem = nt % cus;
  const int tail = (a.M % BM == 0 && nt > cus && rem > 0 && 2 * rem <= cus) ? rem : 0;
  const bool ktail = a.K % BK != 0;
  L.tiles = nt - tail;
  if (tail > 0) {   // L.tiles >= cus: one workgroup per CU runs its whole tiles, then at most one half
    GemmLaunch H = L;
    H.tiles = 2 * tail;
    H.half_base = nt - tail;
    H.half_tail = 1;
    if (ktail)
      hipLaunchKernelGGL(ce_tile_tail_kernel<true>, dim3(cus), dim3(NTHREADS), 0, s, L, H, a, tiles_n);
    else
      hipLaunchKernelGGL(ce_tile_tail_kernel<false>, dim3(cus), dim3(NTHREADS), 0, s, L, H, a, tiles_n);
  } else {
    const dim3 grid(std::min(L.tiles, cus));
    if (ktail) hipLaunchKernelGGL((ce_tile_kernel<4, true>), grid, dim3(NTHREADS), 0, s, L, a, tiles_n);
    else hipLaunchKernelGGL((ce_tile_kernel<4, false>), grid, dim3(NTHREADS), 0, s, L, a, tiles_n);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(ce_merge_kernel, dim3((unsigned)((a.M + 31) / 32)), dim3(256), 0, s, a, tiles_n);
  return hipGetLastError();
}

}  // namespace tps
