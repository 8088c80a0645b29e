// Attention core of one tensor-parallel rank's heads on gfx950: scaled
// dot-product attention with an online (streaming) softmax, GQA (several query
// heads read one KV head), optional causal mask, head dim 128, bf16 in, fp32
// softmax and accumulation.
//
// Work split.  A 256-thread workgroup (4 wave64s) takes one KV head and 128
// query rows that all read it: 32 tokens x 4 query heads when 4 or more query
// heads share the KV head (one head per wave), else 32 x 4/group tokens of
// each of its `group` heads.  Every wave owns 32 query rows, so the KV tiles
// staged in LDS are read by 128 query rows.
//
// Orientation.  Scores are computed transposed, S^T = K Q^T, as
// v_mfma_f32_32x32x16_bf16 with K as the A operand: a lane then holds one
// query row (lane % 32) and 32 of the 64 keys of a tile, so the row max and
// row sum are in-lane plus one exchange with lane ^ 32.  The output is
// accumulated transposed too, O^T += V^T P^T (V as the MN-contiguous A
// operand read with ds_read_b64_tr_b16, P^T as the B operand after one
// v_permlane32_swap per register pair puts each lane's keys in MFMA order).
//
// KV tiles of 64 keys (K 16 KiB + V 16 KiB) go global -> LDS with
// buffer_load_dwordx4 ... lds into a 2-stage ring; rows past the sequence read
// as zero and are masked.
//
// Split KV.  Under the causal mask the work of a query block grows with its
// position, so a block's key range is cut into chunks of chunk_tiles tiles,
// each run by its own workgroup (two fit on a CU).  A block with one chunk
// writes O and lse directly; otherwise every chunk writes its unnormalized
// O, running max and sum (fp32) to the workspace and attn_combine_kernel
// merges the chunks in ascending order (a fixed order: the result does not
// depend on scheduling).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <climits>

#include "attention_common.hpp"
#include "device_common.hpp"
#include "kernels.hpp"

namespace tps {
namespace {

using namespace attn;

constexpr int AT_D = HD;
constexpr int AT_KT = 64;                       // keys per tile
constexpr int AT_TILE = AT_KT * AT_D * 2;       // bytes of one K or V tile (16 KiB)
constexpr int AT_NSTAGE = 2;
constexpr float AT_LOG2E = LOG2E;

__device__ __forceinline__ uint32_t pack2(float lo, float hi) { return pack_bf2(lo, hi); }

// LDS ring: stage s holds the K tile at s * 2 * AT_TILE and the V tile after it.
__shared__ __attribute__((aligned(1024))) char at_ring[AT_NSTAGE * 2 * AT_TILE];

__device__ __forceinline__ TPS_LDS char* ring_k(int stage) { return (TPS_LDS char*)at_ring + stage * 2 * AT_TILE; }
__device__ __forceinline__ TPS_LDS char* ring_v(int stage) { return ring_k(stage) + AT_TILE; }

// Query-block geometry shared by the attention kernels.
struct AttnGeo {
  int group, hpw, tq, nquad;
  int64_t nqb;
};

__device__ __forceinline__ AttnGeo attn_geo(const AttnArgs& a) {
  AttnGeo q;
  q.group = a.n_q / a.n_kv;
  q.hpw = q.group < 4 ? q.group : 4;   // query heads per workgroup
  q.tq = 32 * (4 / q.hpw);             // tokens per workgroup
  q.nquad = q.group / q.hpw;
  q.nqb = (a.S + q.tq - 1) / q.tq;
  return q;
}

// Key tiles of query block qb, and the chunks they are cut into.
__device__ __forceinline__ int attn_tiles(const AttnArgs& a, const AttnGeo& q, int64_t qb) {
  const int64_t kv_end = a.causal ? min<int64_t>(a.S, qb * q.tq + q.tq) : a.S;
  return (int)((kv_end + AT_KT - 1) / AT_KT);
}

// Workspace slot of one chunk: O [128 rows][128] then m [128] and l [128], fp32.
constexpr int64_t AT_SLOT = 128 * 128 + 2 * 128;

__device__ __forceinline__ float* attn_slot(const AttnArgs& a, const AttnGeo& q, int64_t qb, int chunk) {
  const int64_t idx = (((int64_t)blockIdx.z * gridDim.y + blockIdx.y) * q.nqb + qb) * a.max_chunks + chunk;
  return a.ws + idx * AT_SLOT;
}

__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(const AttnArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const AttnGeo geo = attn_geo(a);
  const int group = geo.group, hpw = geo.hpw, tq = geo.tq, nquad = geo.nquad;
  const int64_t nqb = geo.nqb;
  const int chunk = (int)(blockIdx.x / nqb);
  const int64_t qb = nqb - 1 - (int64_t)(blockIdx.x % nqb);   // longest causal blocks first
  const int nt_all = attn_tiles(a, geo, qb);
  const int nchunks = (nt_all + a.chunk_tiles - 1) / a.chunk_tiles;
  if (chunk >= nchunks) return;                                // (uniform: before any barrier)
  const int t_begin = chunk * a.chunk_tiles;
  const int nt = min(nt_all, t_begin + a.chunk_tiles) - t_begin;
  const int g = (int)blockIdx.y / nquad, quad = (int)blockIdx.y % nquad;
  const int64_t b = blockIdx.z;
  const int head = g * group + quad * hpw + (wave % hpw);
  const int64_t tok0 = qb * tq + 32 * (wave / hpw);    // this wave's first token
  const int64_t row0 = b * a.S;                        // the sequence's first row

  // Q fragments (B operand of S^T): row tok0 + lane % 32, d = 16 kk + 8 (lane / 32) .. +7
  bf16x8 qf[8];
  {
    const int64_t t = min<int64_t>(tok0 + (lane & 31), a.S - 1);
    const uint16_t* q = static_cast<const uint16_t*>(a.q) + (row0 + t) * a.ldq + (int64_t)head * AT_D + 8 * (lane >> 5);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qf[kk] = *reinterpret_cast<const bf16x8*>(q + 16 * kk);
  }

  // copy streams (descriptor at the head's first row)
  const char* kbase = static_cast<const char*>(a.k) + (row0 * a.ldk + (int64_t)g * AT_D) * 2;
  const char* vbase = static_cast<const char*>(a.v) + (row0 * a.ldv + (int64_t)g * AT_D) * 2;
  const uint32_t knrec = (uint32_t)(((a.S - 1) * a.ldk + AT_D) * 2);
  const uint32_t vnrec = (uint32_t)(((a.S - 1) * a.ldv + AT_D) * 2);
  const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(kbase), (short)0, (int)knrec,
                                                                      0x00020000);
  const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(vbase), (short)0, (int)vnrec,
                                                                      0x00020000);
  uint32_t kvo[4], vvo[4];
  tile_voffs<LAY_ROW, 4>(a.ldk, kvo);   // K: read as rows
  tile_voffs<LAY_COL, 4>(a.ldv, vvo);   // V: read transposed
  const uint32_t kstep = (uint32_t)(AT_KT * a.ldk * 2), vstep = (uint32_t)(AT_KT * a.ldv * 2);

  issue_tile(kr, kvo, (uint32_t)t_begin * kstep, ring_k(0));
  issue_tile(vr, vvo, (uint32_t)t_begin * vstep, ring_v(0));

  f32x16 o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32x16{0.f};
  float m = -INFINITY, l = 0.f;
  const float c = a.scale * AT_LOG2E;
  const int64_t my_tok = tok0 + (lane & 31);

  for (int t = 0; t < nt; ++t) {
    wait_vm<0>();
    __syncthreads();   // tile t visible to all waves; stage (t+1)%2 free
    if (t + 1 < nt) {
      issue_tile(kr, kvo, (uint32_t)(t_begin + t + 1) * kstep, ring_k((t + 1) & 1));
      issue_tile(vr, vvo, (uint32_t)(t_begin + t + 1) * vstep, ring_v((t + 1) & 1));
    }
    const TPS_LDS char* ks = ring_k(t & 1);
    const TPS_LDS char* vs = ring_v(t & 1);

    // S^T for the tile's two 32-key blocks
    f32x16 st[2] = {f32x16{0.f}, f32x16{0.f}};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        st[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_rows<LAY_ROW>(ks, 32 * kb, kk), qf[kk], st[kb], 0, 0, 0);
    }

    // mask keys past the query (causal) or past the sequence; the scale (and
    // log2 e) enters once, in the exponent's fused multiply-add (c > 0)
    const int64_t key0 = (int64_t)(t_begin + t) * AT_KT;
    const bool need_mask = (key0 + AT_KT > a.S) || (a.causal && key0 + AT_KT - 1 > tok0);
    if (need_mask) {
      const int kmax = (int)min<int64_t>(a.causal ? my_tok - key0 : INT_MAX, a.S - 1 - key0);   // last visible key
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * kb + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3) > kmax) st[kb][r] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[kb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m, mx * c);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m - m_use);
    float rs = 0.f;
    uint32_t pk[2][8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(st[kb][r], c, -m_use));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(st[kb][r + 1], c, -m_use));
        rs += p0 + p1;
        pk[kb][r >> 1] = pack2(p0, p1);
      }
    rs += __shfl_xor(rs, 32);
    l = l * alpha + rs;
    m = m_new;
    if (__ballot(alpha != 1.0f)) {   // some row's max moved
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[i][r] *= alpha;
    }

    // P^T fragments: k-step s covers keys 16 s .. 16 s + 15 of block s / 2
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const bf16x8 pf = pk_frag(pk[s >> 1], s & 1);
#pragma unroll
      for (int db = 0; db < 4; ++db)
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_cols<LAY_COL>(vs, 32 * db, s), pf, o[db], 0, 0, 0);
    }
  }

  if (nchunks > 1) {   // partial: unnormalized O^T rows, running max (log2 domain) and sum
    float* slot = attn_slot(a, geo, qb, chunk);
    const int row = 32 * wave + (lane & 31);
    store_rows_f32(o, 1.f, slot + row * 128);
    if (lane < 32) {
      slot[128 * 128 + row] = m;
      slot[128 * 128 + 128 + row] = l;
    }
    return;
  }

  // O = O^T / l: lane holds row my_tok, d = 32 db + 8 (r / 4) + 4 (lane / 32) + r % 4;
  // one swap per register pair gives each lane 8 consecutive d for 16-byte stores.
  const float inv = 1.0f / l;
  if (my_tok < a.S) {
    if (lane < 32) {
      float* lse = a.lse + ((int64_t)b * a.n_q + head) * a.S + my_tok;
      *lse = (m + __log2f(l)) * 0.69314718055994531f;
    }
  }
  uint16_t* orow = static_cast<uint16_t*>(a.o) + (row0 + min<int64_t>(my_tok, a.S - 1)) * a.ldo + (int64_t)head * AT_D;
  store_rows_bf16(o, inv, orow, my_tok < a.S);
}

// Merge of the chunks of every split query block: for each of the block's 128
// rows, M = max m_c, L = sum l_c 2^(m_c - M), O = sum O_c 2^(m_c - M) / L in
// ascending chunk order; lse = (M + log2 L) ln 2.  A workgroup takes 8 rows of
// one block (32 threads per row, 4 columns each); the chunks' values are loaded
// 8 at a time before they are combined (past the last chunk the load repeats
// it and is not used).  Up to 8 chunks (one group) everything is loaded in one
// round, M taken from those registers; past that a first pass finds M.
__global__ __launch_bounds__(256) void attn_combine_kernel(const AttnArgs a) {
  const AttnGeo geo = attn_geo(a);
  const int64_t qb = blockIdx.x >> 4;
  const int nchunks = (attn_tiles(a, geo, qb) + a.chunk_tiles - 1) / a.chunk_tiles;
  if (nchunks <= 1) return;
  const int g = (int)blockIdx.y / geo.nquad, quad = (int)blockIdx.y % geo.nquad;
  const int64_t b = blockIdx.z;
  const int d4 = 4 * (threadIdx.x & 31);
  const int row = 8 * (blockIdx.x & 15) + (threadIdx.x >> 5);
  const int w = row >> 5;
  const int head = g * geo.group + quad * geo.hpw + (w % geo.hpw);
  const int64_t tok = qb * geo.tq + 32 * (w / geo.hpw) + (row & 31);
  if (tok >= a.S) return;
  const float* s0 = attn_slot(a, geo, qb, 0);
  float M = -INFINITY;
  if (nchunks > 8) {
    for (int c0 = 0; c0 < nchunks; c0 += 8) {
      float mc[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) mc[j] = s0[min(c0 + j, nchunks - 1) * AT_SLOT + 128 * 128 + row];
#pragma unroll
      for (int j = 0; j < 8; ++j) M = fmaxf(M, mc[j]);   // repeats of the last chunk change nothing
    }
  }
  float L = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < nchunks; c0 += 8) {
    float mc[8], lc[8];
    f32x4 oc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float* sl = s0 + min(c0 + j, nchunks - 1) * AT_SLOT;
      mc[j] = sl[128 * 128 + row];
      lc[j] = sl[128 * 128 + 128 + row];
      oc[j] = *reinterpret_cast<const f32x4*>(sl + row * 128 + d4);
    }
    if (nchunks <= 8) {
#pragma unroll
      for (int j = 0; j < 8; ++j) M = fmaxf(M, mc[j]);
    }
    const float Mu = M == -INFINITY ? 0.f : M;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (c0 + j < nchunks) {
        const float wgt = __builtin_amdgcn_exp2f(mc[j] - Mu);
        L += lc[j] * wgt;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] += oc[j][e] * wgt;
      }
    }
  }
  const float inv = 1.0f / L;
  uint16_t* orow = static_cast<uint16_t*>(a.o) + (b * a.S + tok) * a.ldo + (int64_t)head * AT_D + d4;
  *reinterpret_cast<u32x2*>(orow) = u32x2{pack2(acc[0] * inv, acc[1] * inv), pack2(acc[2] * inv, acc[3] * inv)};
  if (d4 == 0) a.lse[((int64_t)b * a.n_q + head) * a.S + tok] = (M + __log2f(L)) * 0.69314718055994531f;
}

}  // namespace

// Chunking (a function of the shape only, so the workspace size is known
// without a device).  Causal: the blocks' key ranges differ in length, so
// they are cut into chunks of about 1.2x the mean work per workgroup slot
// (512 slots: two workgroups on each CU of an MI355X), which keeps the number
// of workgroups near one round of slots and lets the short chunks fill the
// gaps.  Without the mask every block has the same work, and the range is cut
// only when there are fewer than 512 workgroups.
constexpr int64_t AT_TARGET_WGS = 512;

void attn_chunking(int64_t B, int64_t S, int n_q, int n_kv, int causal, int& chunk_tiles, int& max_chunks) {
  const int group = n_q / n_kv;
  const int hpw = group < 4 ? group : 4;
  const int tq = 32 * (4 / hpw);
  const int64_t nqb = (S + tq - 1) / tq;
  const int64_t nt_max = (S + AT_KT - 1) / AT_KT;
  int64_t c;
  if (causal) {
    int64_t tiles = 0;   // key tiles over all query blocks of one (sequence, head group)
    for (int64_t qb = 0; qb < nqb; ++qb) tiles += (std::min<int64_t>(S, (qb + 1) * tq) + AT_KT - 1) / AT_KT;
    const int64_t groups = (int64_t)n_kv * (group / hpw) * B;
    c = (12 * tiles * groups + 10 * AT_TARGET_WGS - 1) / (10 * AT_TARGET_WGS);
    c = std::max<int64_t>(c, 8);
  } else {
    const int64_t blocks = nqb * n_kv * (group / hpw) * B;
    const int64_t want = std::max<int64_t>(1, (AT_TARGET_WGS + blocks - 1) / blocks);
    c = (nt_max + want - 1) / want;
  }
  c = std::max<int64_t>(1, std::min<int64_t>(c, nt_max));
  chunk_tiles = (int)c;
  max_chunks = (int)((nt_max + c - 1) / c);
}

size_t attn_fwd_workspace_bytes(int64_t B, int64_t S, int n_q, int n_kv, int causal) {
  int ct, mc;
  attn_chunking(B, S, n_q, n_kv, causal, ct, mc);
  if (mc <= 1) return 0;
  const int group = n_q / n_kv;
  const int hpw = group < 4 ? group : 4;
  const int tq = 32 * (4 / hpw);
  const int64_t nqb = (S + tq - 1) / tq;
  return (size_t)(B * n_kv * (group / hpw) * nqb * mc * AT_SLOT * 4);
}

hipError_t launch_attn_fwd(const AttnArgs& a, hipStream_t s) {
  const int group = a.n_q / a.n_kv;
  const int hpw = group < 4 ? group : 4;
  const int tq = 32 * (4 / hpw);
  const int64_t nqb = (a.S + tq - 1) / tq;
  const unsigned gy = (unsigned)(a.n_kv * (group / hpw));
  hipLaunchKernelGGL(attn_fwd_kernel, dim3((unsigned)(nqb * a.max_chunks), gy, (unsigned)a.B), dim3(256), 0, s, a);
  if (a.max_chunks > 1)
    hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)(nqb * 16), gy, (unsigned)a.B), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace tps
