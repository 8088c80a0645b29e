// Backward of the attention core (gfx950), without atomics:
//
//   attn_bwd_prep_kernel     per (token, head): lse in the log2 domain and
//                            D = sum_d dO * O (= sum_j P dP of that row);
//   attn_bwd_dq_kernel       query-major, like the forward: for each key tile
//                            S^T = K Q^T and dP^T = V dO^T are recomputed,
//                            P^T = 2^(S^T c - lse2), dS^T = P^T (dP^T - D), and
//                            dQ^T += K^T dS^T;
//   attn_bwd_dkv_kernel      key-major: a workgroup owns 128 keys of one KV
//                            head and takes the query tiles of one query head:
//                            S = Q K^T, dP = dO V^T, P, dS as above,
//                            dV^T += dO^T P and dK^T += Q^T dS;
//   *_combine kernels        ordered sums of the partial results (key chunks
//                            for dQ; query heads and query chunks for dK, dV).
//
// Fragments and lane layouts are those of the forward kernel
// (attention_common.hpp); P and dS enter their products as bf16, every sum is
// fp32 and runs in a fixed order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <climits>
#include <type_traits>

#include "attention_common.hpp"
#include "attention_order.hpp"
#include "device_common.hpp"
#include "kernels.hpp"

namespace tps {
namespace {

using namespace attn;

constexpr int KT = 64;                   // keys per tile (dQ kernel)
constexpr int KTILE = KT * HD * 2;       // 16 KiB
constexpr int QT = 32;                   // queries per tile (dK/dV kernel)
constexpr int QTILE = QT * HD * 2;       // 8 KiB
constexpr int QSTAGE = 2 * QTILE + 512;  // Q tile, dO tile, 32 (lse2, D) pairs (+ pad)
constexpr int64_t DQ_SLOT = 128 * 128;   // fp32 partial dQ^T rows of one query block
constexpr int64_t KV_SLOT = 128 * 256;   // fp32 partial [dK | dV] rows of one key block

struct Geo {
  int group, hpw, tq, nquad;
  int64_t nqb;
};

__device__ __forceinline__ Geo geo_of(const AttnArgs& a) {
  Geo q;
  q.group = a.n_q / a.n_kv;
  q.hpw = q.group < 4 ? q.group : 4;
  q.tq = 32 * (4 / q.hpw);
  q.nquad = q.group / q.hpw;
  q.nqb = (a.S + q.tq - 1) / q.tq;
  return q;
}

// ---- prep ---------------------------------------------------------------------
// 16 lanes per row, 8 of its 128 elements each (one 16-byte load of O and of
// dO: a wave reads four whole rows per load), then a fixed butterfly over the
// 16 lanes.
__global__ __launch_bounds__(256) void attn_bwd_prep_kernel(const AttnBwdArgs p) {
  const AttnArgs& a = p.f;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t rows = a.B * a.n_q * a.S;
  const int64_t i = t >> 4;                    // (b, h, token) flattened
  const int c = (int)(t & 15);                 // this lane's 8 elements: 8 c .. 8 c + 7
  const bool live = i < rows;
  const int64_t ir = live ? i : rows - 1;      // past the end: a repeat, kept in the shuffles, not written
  const int64_t tok = ir % a.S, bh = ir / a.S;
  const int h = (int)(bh % a.n_q);
  const int64_t b = bh / a.n_q;
  const uint16_t* o = static_cast<const uint16_t*>(a.o) + (b * a.S + tok) * a.ldo + (int64_t)h * HD + 8 * c;
  const uint16_t* g = static_cast<const uint16_t*>(p.dout) + (b * a.S + tok) * p.ldg + (int64_t)h * HD + 8 * c;
  const u32x4 x = *reinterpret_cast<const u32x4*>(o);
  const u32x4 y = *reinterpret_cast<const u32x4*>(g);
  float d = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    d += __uint_as_float(x[e] << 16) * __uint_as_float(y[e] << 16);
    d += __uint_as_float(x[e] & 0xffff0000u) * __uint_as_float(y[e] & 0xffff0000u);
  }
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) d += __shfl_xor(d, off);
  if (live && c == 0) reinterpret_cast<f32x2_t*>(p.ld)[i] = f32x2_t{a.lse[i] * LOG2E, d};
}

// ---- dQ ---------------------------------------------------------------------------
__shared__ __attribute__((aligned(1024))) char bq_ring[2 * 2 * KTILE];

__device__ __forceinline__ TPS_LDS char* bq_k(int st) { return (TPS_LDS char*)bq_ring + st * 2 * KTILE; }
__device__ __forceinline__ TPS_LDS char* bq_v(int st) { return bq_k(st) + KTILE; }

__device__ __forceinline__ int key_tiles(const AttnArgs& a, const Geo& q, int64_t qb) {
  const int64_t kv_end = a.causal ? min<int64_t>(a.S, qb * q.tq + q.tq) : a.S;
  return (int)((kv_end + KT - 1) / KT);
}

__device__ __forceinline__ float* dq_slot(const AttnBwdArgs& p, const Geo& q, int64_t qb, int chunk) {
  const int64_t idx = (((int64_t)blockIdx.z * gridDim.y + blockIdx.y) * q.nqb + qb) * p.f.max_chunks + chunk;
  return p.dq_ws + idx * DQ_SLOT;
}

__global__ __launch_bounds__(256, 2) void attn_bwd_dq_kernel(const AttnBwdArgs p) {
  const AttnArgs& a = p.f;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const Geo geo = geo_of(a);
  const int chunk = (int)(blockIdx.x / geo.nqb);
  const int64_t qb = geo.nqb - 1 - (int64_t)(blockIdx.x % geo.nqb);
  const int nt_all = key_tiles(a, geo, qb);
  const int nchunks = (nt_all + a.chunk_tiles - 1) / a.chunk_tiles;
  if (chunk >= nchunks) return;
  const int t_begin = chunk * a.chunk_tiles;
  const int nt = min(nt_all, t_begin + a.chunk_tiles) - t_begin;
  const int g = (int)blockIdx.y / geo.nquad, quad = (int)blockIdx.y % geo.nquad;
  const int64_t b = blockIdx.z;
  const int head = g * geo.group + quad * geo.hpw + (wave % geo.hpw);
  const int64_t tok0 = qb * geo.tq + 32 * (wave / geo.hpw);
  const int64_t row0 = b * a.S;
  const int64_t my_tok = tok0 + (lane & 31);
  const int64_t tc = min<int64_t>(my_tok, a.S - 1);

  // Q and dO rows of this lane's query (B operands of S^T and dP^T)
  bf16x8 qf[8], gf[8];
  {
    const uint16_t* q = static_cast<const uint16_t*>(a.q) + (row0 + tc) * a.ldq + (int64_t)head * HD + 8 * (lane >> 5);
    const uint16_t* gg = static_cast<const uint16_t*>(p.dout) + (row0 + tc) * p.ldg + (int64_t)head * HD +
                         8 * (lane >> 5);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      qf[kk] = *reinterpret_cast<const bf16x8*>(q + 16 * kk);
      gf[kk] = *reinterpret_cast<const bf16x8*>(gg + 16 * kk);
    }
  }
  const f32x2_t ldv = reinterpret_cast<const f32x2_t*>(p.ld)[((int64_t)b * a.n_q + head) * a.S + tc];
  const float lse2 = ldv[0], Dv = ldv[1];

  const char* kbase = static_cast<const char*>(a.k) + (row0 * a.ldk + (int64_t)g * HD) * 2;
  const char* vbase = static_cast<const char*>(a.v) + (row0 * a.ldv + (int64_t)g * HD) * 2;
  const __amdgpu_buffer_rsrc_t kr = rsrc(kbase, (uint32_t)(((a.S - 1) * a.ldk + HD) * 2));
  const __amdgpu_buffer_rsrc_t vr = rsrc(vbase, (uint32_t)(((a.S - 1) * a.ldv + HD) * 2));
  uint32_t kvo[4], vvo[4];
  tile_voffs<LAY_BOTH, 4>(a.ldk, kvo);   // K: read as rows (S^T) and as columns (dQ)
  tile_voffs<LAY_ROW, 4>(a.ldv, vvo);    // V: read as rows (dP^T)
  const uint32_t kstep = (uint32_t)(KT * a.ldk * 2), vstep = (uint32_t)(KT * a.ldv * 2);
  issue_tile(kr, kvo, (uint32_t)t_begin * kstep, bq_k(0));
  issue_tile(vr, vvo, (uint32_t)t_begin * vstep, bq_v(0));

  f32x16 dq[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) dq[i] = f32x16{0.f};
  const float c = a.scale * LOG2E;

  for (int t = 0; t < nt; ++t) {
    wait_vm<0>();
    __syncthreads();
    if (t + 1 < nt) {
      issue_tile(kr, kvo, (uint32_t)(t_begin + t + 1) * kstep, bq_k((t + 1) & 1));
      issue_tile(vr, vvo, (uint32_t)(t_begin + t + 1) * vstep, bq_v((t + 1) & 1));
    }
    const TPS_LDS char* ks = bq_k(t & 1);
    const TPS_LDS char* vs = bq_v(t & 1);

    const int64_t key0 = (int64_t)(t_begin + t) * KT;
    const bool need_mask = (key0 + KT > a.S) || (a.causal && key0 + KT - 1 > tok0);
    const int kmax = need_mask ? (int)min<int64_t>(a.causal ? my_tok - key0 : INT_MAX, a.S - 1 - key0) : INT_MAX;
    uint32_t pk[2][8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {   // one 32-key block at a time (register budget)
      f32x16 st = f32x16{0.f}, dp = f32x16{0.f};
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_rows<LAY_BOTH>(ks, 32 * kb, kk), qf[kk], st, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_rows<LAY_ROW>(vs, 32 * kb, kk), gf[kk], dp, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        float ds[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int key = 32 * kb + 8 * ((r + e) >> 2) + 4 * (lane >> 5) + ((r + e) & 3);
          const float pr = __builtin_amdgcn_exp2f(key > kmax ? -INFINITY : __builtin_fmaf(st[r + e], c, -lse2));
          ds[e] = pr * (dp[r + e] - Dv);
        }
        pk[kb][r >> 1] = pack_bf2(ds[0], ds[1]);
      }
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const bf16x8 df = pk_frag(pk[s >> 1], s & 1);
#pragma unroll
      for (int db = 0; db < 4; ++db)
        dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_cols<LAY_BOTH>(ks, 32 * db, s), df, dq[db], 0, 0, 0);
    }
  }

  if (nchunks > 1) {
    const int row = 32 * wave + (lane & 31);
    store_rows_f32(dq, 1.f, dq_slot(p, geo, qb, chunk) + row * 128);
    return;
  }
  uint16_t* out = static_cast<uint16_t*>(p.dq) + (row0 + tc) * p.lddq + (int64_t)head * HD;
  store_rows_bf16(dq, a.scale, out, my_tok < a.S);
}

// Ordered sum of the key chunks of every split query block, times scale: a
// workgroup takes 8 rows of one block (32 threads per row, 4 columns each) and
// loads 8 chunks' values before adding them.
__global__ __launch_bounds__(256) void attn_bwd_dq_combine_kernel(const AttnBwdArgs p) {
  const AttnArgs& a = p.f;
  const Geo geo = geo_of(a);
  const int64_t qb = blockIdx.x >> 4;
  const int nchunks = (key_tiles(a, geo, qb) + a.chunk_tiles - 1) / a.chunk_tiles;
  if (nchunks <= 1) return;
  const int g = (int)blockIdx.y / geo.nquad, quad = (int)blockIdx.y % geo.nquad;
  const int64_t b = blockIdx.z;
  const int d4 = 4 * (threadIdx.x & 31);
  const int row = 8 * (blockIdx.x & 15) + (threadIdx.x >> 5);
  const int w = row >> 5;
  const int head = g * geo.group + quad * geo.hpw + (w % geo.hpw);
  const int64_t tok = qb * geo.tq + 32 * (w / geo.hpw) + (row & 31);
  if (tok >= a.S) return;
  const float* s0 = dq_slot(p, geo, qb, 0) + row * 128 + d4;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < nchunks; c0 += 8) {
    f32x4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = *reinterpret_cast<const f32x4*>(s0 + min(c0 + j, nchunks - 1) * DQ_SLOT);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (c0 + j < nchunks) {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] += v[j][e];
      }
  }
  uint16_t* out = static_cast<uint16_t*>(p.dq) + (b * a.S + tok) * p.lddq + (int64_t)head * HD + d4;
  *reinterpret_cast<u32x2*>(out) =
      u32x2{pack_bf2(acc[0] * a.scale, acc[1] * a.scale), pack_bf2(acc[2] * a.scale, acc[3] * a.scale)};
}

// ---- dK, dV -------------------------------------------------------------------------
// Ring of 32-query tiles.  Iteration t finishes tile t (dV, dK) and forms tile t + 1's S and
// dP; while its MFMAs run, it reads from LDS the operands of iteration t + 1 (tile t + 2's row
// fragments, tile t + 1's (lse2, D)), so that every iteration starts on operands already in
// registers.  The waves meet at a barrier every KV_WIN = 2
// iterations: at the barrier of an even t, tiles up to t + 3 have landed (the window reads up
// to tile t + 3), tiles t - 2 and t - 1 are finished, and their stages take tiles t + 6, t + 7.
constexpr int KV_NSTAGE = 8;
constexpr int KV_WIN = 2;

__shared__ __attribute__((aligned(1024))) char bkv_ring[KV_NSTAGE * QSTAGE];

__device__ __forceinline__ TPS_LDS char* bkv_q(int st) { return (TPS_LDS char*)bkv_ring + st * QSTAGE; }
__device__ __forceinline__ TPS_LDS char* bkv_g(int st) { return bkv_q(st) + QTILE; }
__device__ __forceinline__ TPS_LDS char* bkv_l(int st) { return bkv_q(st) + 2 * QTILE; }

// First query and query tiles of key block kbk (queries before the block see none of its keys
// under the causal mask).
__device__ __forceinline__ int64_t kv_q_begin(const AttnArgs& a, int64_t kbk) { return a.causal ? 128 * kbk : 0; }
__device__ __forceinline__ int query_tiles(const AttnArgs& a, int64_t kbk) {
  return (int)((a.S - kv_q_begin(a, kbk) + QT - 1) / QT);
}

using attn_order::KvItem;
using attn_order::kv_item;

__device__ __forceinline__ float* kv_slot(const AttnBwdArgs& p, int64_t b, int g, int64_t kbk, int hg, int chunk) {
  const AttnArgs& a = p.f;
  const int group = a.n_q / a.n_kv;
  const int64_t nkb = (a.S + 127) / 128;
  const int64_t idx = ((((b * a.n_kv + g) * nkb + kbk) * group + hg) * p.kv_max_chunks) + chunk;
  return p.kv_ws + idx * KV_SLOT;
}

__global__ __launch_bounds__(256, 1) void attn_bwd_dkv_kernel(const AttnBwdArgs p) {
  const AttnArgs& a = p.f;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  KvItem item;
  if (!kv_item(a.S, a.causal != 0, a.n_q, p.kv_chunk_tiles, blockIdx.x, item)) return;
  const int chunk = item.chunk;
  const int64_t kbk = item.kbk;
  const int nqt_all = query_tiles(a, kbk);
  const int nchunks = (nqt_all + p.kv_chunk_tiles - 1) / p.kv_chunk_tiles;
  if (chunk >= nchunks) return;
  const int t_begin = chunk * p.kv_chunk_tiles;
  const int nt = min(nqt_all, t_begin + p.kv_chunk_tiles) - t_begin;
  const int h = item.h;
  const int group = a.n_q / a.n_kv;
  const int g = h / group;
  const int64_t b = blockIdx.z;
  const int64_t row0 = b * a.S;
  const int64_t key_w = 128 * kbk + 32 * wave;           // this wave's first key
  const int64_t my_key = key_w + (lane & 31);
  const int64_t kc = min<int64_t>(my_key, a.S - 1);
  const int64_t q_begin = kv_q_begin(a, kbk);

  const char* qbase = static_cast<const char*>(a.q) + (row0 * a.ldq + (int64_t)h * HD) * 2;
  const char* gbase = static_cast<const char*>(p.dout) + (row0 * p.ldg + (int64_t)h * HD) * 2;
  const char* lbase = reinterpret_cast<const char*>(p.ld + 2 * (((int64_t)b * a.n_q + h) * a.S));
  const __amdgpu_buffer_rsrc_t qr = rsrc(qbase, (uint32_t)(((a.S - 1) * a.ldq + HD) * 2));
  const __amdgpu_buffer_rsrc_t gr = rsrc(gbase, (uint32_t)(((a.S - 1) * p.ldg + HD) * 2));
  const __amdgpu_buffer_rsrc_t lr = rsrc(lbase, (uint32_t)(a.S * 8));
  uint32_t qvo[2], gvo[2];
  tile_voffs<LAY_BOTH, 2>(a.ldq, qvo);
  tile_voffs<LAY_BOTH, 2>(p.ldg, gvo);
  const uint32_t qstep = (uint32_t)(QT * a.ldq * 2), gstep = (uint32_t)(QT * p.ldg * 2);

  auto issue = [&](int t, int st) {
    const int64_t qt = q_begin + (int64_t)(t_begin + t) * QT;   // first query of the tile
    const uint32_t tq = (uint32_t)(qt / QT);
    issue_tile(qr, qvo, tq * qstep, bkv_q(st));
    issue_tile(gr, gvo, tq * gstep, bkv_g(st));
    // 32 (lse2, D) pairs: 256 bytes, 4 per lane.  Every wave issues the same copy (identical
    // bytes to the same place), so that every wave counts 5 copies per tile.
    lds_copy4(lr, (uint32_t)(qt * 8 + 4 * lane), bkv_l(st));
  };
  for (int t = 0; t < 4 && t < nt; ++t) issue(t, t);
  // K and V rows of this lane's key (B operands of S = Q K^T and dP = dO V^T)
  bf16x8 kf[8], vf[8];
  {
    const uint16_t* kp = static_cast<const uint16_t*>(a.k) + (row0 + kc) * a.ldk + (int64_t)g * HD + 8 * (lane >> 5);
    const uint16_t* vp = static_cast<const uint16_t*>(a.v) + (row0 + kc) * a.ldv + (int64_t)g * HD + 8 * (lane >> 5);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      kf[kk] = *reinterpret_cast<const bf16x8*>(kp + 16 * kk);
      vf[kk] = *reinterpret_cast<const bf16x8*>(vp + 16 * kk);
    }
  }
  // Tiles 0 .. 3 and the K, V rows; waited for here, explicitly, so that the compiler's own
  // wait for the K, V registers does not also wait for the copies queued after them.
  wait_vm<0>();
  for (int t = 4; t < KV_NSTAGE && t < nt; ++t) issue(t, t);

  f32x16 dk[4], dv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    dk[i] = f32x16{0.f};
    dv[i] = f32x16{0.f};
  }
  const float c = a.scale * LOG2E;

  // Row fragments of the tile in ring stage st: A operands of S = Q K^T and dP = dO V^T.
  auto load_rows = [&](int st, bf16x8 (&qa)[8], bf16x8 (&ga)[8]) {
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      qa[kk] = frag_rows<LAY_BOTH>(bkv_q(st), 0, kk);
      ga[kk] = frag_rows<LAY_BOTH>(bkv_g(st), 0, kk);
    }
  };
  // Column fragments of k-step ss: A operands of dV += dO^T P and dK += Q^T dS.
  auto load_cols = [&](int st, int ss, bf16x8 (&cq)[4], bf16x8 (&cg)[4]) {
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      cg[db] = frag_cols<LAY_BOTH>(bkv_g(st), 32 * db, ss);
      cq[db] = frag_cols<LAY_BOTH>(bkv_q(st), 32 * db, ss);
    }
  };
  // (lse2, D) of this lane's 16 queries: pairs 8 q + 4 (lane / 32) + 0..3 as two f32x4 per q
  auto load_ld = [&](int st, f32x4 (&lv)[8]) {
    const TPS_LDS float* ls = (const TPS_LDS float*)bkv_l(st);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int qi = 8 * q + 4 * (lane >> 5);
      lv[2 * q] = *reinterpret_cast<const TPS_LDS f32x4*>(ls + 2 * qi);
      lv[2 * q + 1] = *reinterpret_cast<const TPS_LDS f32x4*>(ls + 2 * qi + 4);
    }
  };

  __syncthreads();   // tiles 0 .. 3 visible to every wave
  // Operands rotate through registers: at the top of iteration t, ra, rg hold tile t + 1's row
  // fragments and lv tile t's (lse2, D).
  // Reads of tiles past the chunk's end hit stale ring stages; those values are never used.
  bf16x8 ra[8], rg[8], cq0[4], cg0[4];
  f32x4 lv[8];
  f32x16 s_cur = f32x16{0.f}, dp_cur = f32x16{0.f};
  load_rows(0, ra, rg);
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    s_cur = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[kk], kf[kk], s_cur, 0, 0, 0);
    dp_cur = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rg[kk], vf[kk], dp_cur, 0, 0, 0);
  }
  load_rows(1, ra, rg);
  load_ld(0, lv);

  for (int t = 0; t < nt; ++t) {
    if (t > 0 && t % KV_WIN == 0) {
      // tiles up to t + 5 issued (5 copies each); tiles up to t + 3 must have landed
      switch (max(0, min(nt, t + 6) - (t + 4))) {
        case 0: wait_vm<0>(); break;
        case 1: wait_vm<5>(); break;
        default: wait_vm<10>(); break;
      }
      __syncthreads();
      if (t + 6 < nt) issue(t + 6, (t + 6) % KV_NSTAGE);
      if (t + 7 < nt) issue(t + 7, (t + 7) % KV_NSTAGE);
    }
    const int st = t % KV_NSTAGE;
    __builtin_amdgcn_sched_barrier(0);

    // lane: key my_key, queries qt + 8 (r / 4) + 4 (lane / 32) + r % 4.  Every pair of the
    // tile is live when its queries lie inside the sequence, the wave's keys do, and (causal)
    // its first query is not before the wave's last key; otherwise mask per element.
    // (positions fit in 32 bits: a bf16 operand holds under 2^30 elements, so B S < 2^23)
    const int qt = (int)q_begin + (t_begin + t) * QT;
    const int S32 = (int)a.S, kw = (int)key_w;
    const bool full = qt + QT <= S32 && kw + 32 <= S32 && (!a.causal || qt >= kw + 31);
    const int lim = S32 - 1 - qt;                           // last query, tile-relative
    const int first = a.causal ? (int)my_key - qt : INT_MIN;  // first query that sees my_key
    const bool key_ok = my_key < a.S;
    uint32_t pp[8], pd[8];
    f32x16 s_nxt = f32x16{0.f}, dp_nxt = f32x16{0.f};
    // S and dP of tile t + 1 on the matrix cores while the vector unit forms tile t's
    // P = 2^(S c - lse2) (masked pairs: 2^-inf = 0) and dS = P (dP - D); two straight-line
    // versions, chosen per tile, so that unmasked tiles carry no per-element tests
    auto step = [&](auto masked) {
      load_cols(st, 0, cq0, cg0);   // this tile's first column fragments, needed after the step
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        s_nxt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[kk], kf[kk], s_nxt, 0, 0, 0);
        dp_nxt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rg[kk], vf[kk], dp_nxt, 0, 0, 0);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int qi = 8 * q + 4 * (lane >> 5);
        const f32x4 l01 = lv[2 * q], l23 = lv[2 * q + 1];
        const float lse2[4] = {l01[0], l01[2], l23[0], l23[2]};
        const float dd[4] = {l01[1], l01[3], l23[1], l23[3]};
        float pv[4], dsv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * q + e;
          if constexpr (decltype(masked)::value) {
            // the mask acts on the operands (S -> -inf, dP -> D), so that neither path shares
            // an instruction with the other that the compiler would hoist out of the MFMA mix
            const bool ok = (qi + e) <= lim && (qi + e) >= first && key_ok;
            pv[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(ok ? s_cur[r] : -INFINITY, c, -lse2[e]));
            dsv[e] = pv[e] * ((ok ? dp_cur[r] : dd[e]) - dd[e]);
          } else {
            pv[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[r], c, -lse2[e]));
            dsv[e] = pv[e] * (dp_cur[r] - dd[e]);
          }
        }
        pp[2 * q] = pack_bf2(pv[0], pv[1]);
        pp[2 * q + 1] = pack_bf2(pv[2], pv[3]);
        pd[2 * q] = pack_bf2(dsv[0], dsv[1]);
        pd[2 * q + 1] = pack_bf2(dsv[2], dsv[3]);
      }
      // one MFMA, then a slice of the vector work, so that the vector unit runs while the
      // matrix core is busy (one wave per SIMD: nothing else would fill those cycles)
      // (group masks: 0x008 MFMA, 0x002 | 0x400 vector ALU and transcendental, 0x100 LDS read)
      if constexpr (decltype(masked)::value) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x402, 8, 0);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x402, 5, 0);
        }
      }
    };
    if (full) step(std::false_type{});
    else step(std::true_type{});
    __builtin_amdgcn_sched_barrier(0);

    // dV, dK in two k-steps of 8 MFMAs; under each, the LDS reads for what comes next: the
    // second column fragments and the next iteration's (lse2, D), then its rows
    bf16x8 cq1[4], cg1[4];
    {
      const bf16x8 pf = pk_frag(pp, 0), df = pk_frag(pd, 0);
      load_cols(st, 1, cq1, cg1);
      load_ld((t + 1) % KV_NSTAGE, lv);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cg0[db], pf, dv[db], 0, 0, 0);
        dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cq0[db], df, dk[db], 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    {
      const bf16x8 pf = pk_frag(pp, 1), df = pk_frag(pd, 1);
      load_rows((t + 2) % KV_NSTAGE, ra, rg);   // the next iteration's S, dP operands
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cg1[db], pf, dv[db], 0, 0, 0);
        dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cq1[db], df, dk[db], 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    s_cur = s_nxt;
    dp_cur = dp_nxt;
  }

  float* slot = kv_slot(p, b, g, kbk, h % group, chunk) + (32 * wave + (lane & 31)) * 256;
  store_rows_f32(dk, a.scale, slot);
  store_rows_f32(dv, 1.f, slot + 128);
}

// dK, dV rows of every key block: ordered sum over the query heads of the group
// and their query chunks (head-major), rounded to bf16.  A workgroup takes 4
// rows (64 threads per row, 4 of the 256 [dK | dV] columns each) and loads 8
// partials before adding them.
__global__ __launch_bounds__(256) void attn_bwd_dkv_combine_kernel(const AttnBwdArgs p) {
  const AttnArgs& a = p.f;
  const int64_t kbk = blockIdx.x >> 5;
  const int g = (int)blockIdx.y;
  const int64_t b = blockIdx.z;
  const int group = a.n_q / a.n_kv;
  const int nchunks = (query_tiles(a, kbk) + p.kv_chunk_tiles - 1) / p.kv_chunk_tiles;
  const int col = 4 * (threadIdx.x & 63);   // 0..252 over [dK | dV]
  const int row = 4 * (blockIdx.x & 31) + (threadIdx.x >> 6);
  const int64_t key = 128 * kbk + row;
  if (key >= a.S) return;
  const int n = group * nchunks;            // partial j = (head j / nchunks, chunk j % nchunks)
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < n; j0 += 8) {
    f32x4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int jj = min(j0 + j, n - 1);
      v[j] = *reinterpret_cast<const f32x4*>(kv_slot(p, b, g, kbk, jj / nchunks, jj % nchunks) + row * 256 + col);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j0 + j < n) {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] += v[j][e];
      }
  }
  const bool is_k = col < 128;
  uint16_t* out = is_k ? static_cast<uint16_t*>(p.dk) + (b * a.S + key) * p.lddk + (int64_t)g * HD + col
                       : static_cast<uint16_t*>(p.dv) + (b * a.S + key) * p.lddv + (int64_t)g * HD + (col - 128);
  *reinterpret_cast<u32x2*>(out) = u32x2{pack_bf2(acc[0], acc[1]), pack_bf2(acc[2], acc[3])};
}

}  // namespace

// Key chunks of the dQ pass follow the forward's chunking; the dK/dV pass takes
// 4096 queries (128 tiles) per workgroup: with the longest-first launch order,
// fewer and longer items beat 2048 queries (8192 tokens, 4 heads: 327 against
// 335 µs for the whole backward; 6144 and 8192 queries ran slower), and the
// partials the merge reads shrink with the item count.
constexpr int KV_CHUNK_TILES = 128;
static_assert(KV_CHUNK_TILES % 4 == 0, "the causal item order steps query tiles by 4 per key block");
static_assert(attn_order::kQT == QT, "the item order counts the pass's query tiles");


void attn_bwd_layout(int64_t B, int64_t S, int n_q, int n_kv, int causal, AttnBwdLayout& L) {
  attn_chunking(B, S, n_q, n_kv, causal, L.chunk_tiles, L.max_chunks);
  const int group = n_q / n_kv;
  const int hpw = group < 4 ? group : 4;
  const int tq = 32 * (4 / hpw);
  const int64_t nqb = (S + tq - 1) / tq;
  const int64_t nkb = (S + 127) / 128;
  const int64_t nqt = (S + QT - 1) / QT;
  L.kv_chunk_tiles = KV_CHUNK_TILES;
  L.kv_max_chunks = (int)((nqt + KV_CHUNK_TILES - 1) / KV_CHUNK_TILES);
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  L.ld_bytes = al((size_t)(B * n_q * S) * 8);
  L.dq_bytes = L.max_chunks > 1 ? al((size_t)(B * n_kv * (group / hpw) * nqb * L.max_chunks * DQ_SLOT) * 4) : 0;
  L.kv_bytes = al((size_t)(B * n_kv * nkb * group * L.kv_max_chunks * KV_SLOT) * 4);
}

hipError_t launch_attn_bwd(const AttnBwdArgs& p, hipStream_t s) {
  const AttnArgs& a = p.f;
  const int group = a.n_q / a.n_kv;
  const int hpw = group < 4 ? group : 4;
  const int tq = 32 * (4 / hpw);
  const int64_t nqb = (a.S + tq - 1) / tq;
  const int64_t nkb = (a.S + 127) / 128;
  const unsigned gy = (unsigned)(a.n_kv * (group / hpw));
  const int64_t rows = a.B * a.n_q * a.S;
  hipLaunchKernelGGL(attn_bwd_prep_kernel, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, s, p);
  hipLaunchKernelGGL(attn_bwd_dq_kernel, dim3((unsigned)(nqb * a.max_chunks), gy, (unsigned)a.B), dim3(256), 0, s, p);
  if (a.max_chunks > 1)
    hipLaunchKernelGGL(attn_bwd_dq_combine_kernel, dim3((unsigned)(nqb * 16), gy, (unsigned)a.B), dim3(256), 0, s, p);
  const int64_t items = attn_order::kv_items(a.S, a.causal != 0, a.n_q, KV_CHUNK_TILES);
  hipLaunchKernelGGL(attn_bwd_dkv_kernel, dim3((unsigned)items, 1, (unsigned)a.B), dim3(256), 0, s, p);
  hipLaunchKernelGGL(attn_bwd_dkv_combine_kernel, dim3((unsigned)(nkb * 32), (unsigned)a.n_kv, (unsigned)a.B),
                     dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace tps
