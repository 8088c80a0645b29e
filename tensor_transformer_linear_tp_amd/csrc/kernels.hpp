// Internal launch descriptors shared by the HIP kernels and the C-ABI layer.
// Not part of the public ABI (include/tpshard.h is).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tps {

// Operand layouts of C[M,N] = sum_k A(m,k) B(k,n), both stored row-major:
//   L_NN: A [M][K] (K contiguous), B [K][N] (N contiguous)   -- forward Y = X W
//   L_NT: A [M][K],                B [N][K] (K contiguous)   -- dgrad dX = dY W^T, LM head
//   L_TN: A [K][M] (M contiguous), B [K][N]                  -- wgrad dW = X^T dY
enum Layout : int { L_NN = 0, L_NT = 1, L_TN = 2 };

// Epilogues applied to the fp32 accumulator tile.
//   E_STORE : C = acc (+ bias)
//   E_GELU  : P = acc + bias; Pre = P; C = GeLU(P)
//   E_SWIGLU: G = acc_gate + bias, U = acc_up + bias2; Pre = [G | U]; C = silu(G) * U
//   E_CE_GRAD: C = gscale[m] * (exp(acc - lse[m]) - [n == target[m] - v0])  (CE backward)
enum EpiMode : int { E_STORE = 0, E_GELU = 1, E_SWIGLU = 2, E_CE_GRAD = 3 };

// One K-segment: C += A_seg * B_seg over K elements.  A problem may chain
// two segments that accumulate into the same tile (the SwiGLU dgrad sums the
// gate and up contributions).
struct Seg {
  const void* a;
  const void* b;
  int64_t lda, ldb, K;
};

struct Problem {
  int64_t M, N;          // output rows / columns (SwiGLU: columns of Y = gate width)
  Seg seg[2];
  int nseg;
  int layout;            // Layout (shared by both segments)
  int epi;               // EpiMode
  const void* b_up;      // E_SWIGLU: up-projection weight [K][N] (layout L_NN, one segment)
  int64_t ldb_up;
  const void* bias;      // [N] or nullptr
  const void* bias2;     // [N] or nullptr (SwiGLU up bias)
  void* c;               // output [M][ldc]
  int64_t ldc;
  void* pre;             // E_GELU / E_SWIGLU pre-activation output
  int64_t ldpre;
  const float* lse;      // E_CE_GRAD: per-row log-sum-exp [M]
  const float* gscale;   // E_CE_GRAD: per-row upstream gradient [M] or nullptr (1)
  const int32_t* target; // E_CE_GRAD: per-row target id [M]
  int64_t v0;            // E_CE_GRAD: first column's id
  // filled by the launcher
  int tiles_m, tiles_n, tile_begin;
  int edge_only;         // tiles enumerate only the ragged edge (right strip, then bottom strip)
  int full_m, full_n;    // whole tiles along M and N (edge_only)
  // Split contraction (one-segment plain-store problems of the two-layout
  // launch): ksplit > 1 cuts K into ksplit equal parts, each a tile set of
  // its own whose fp32 result goes to c32 + part * M * N ([M][N], rows of N
  // floats); splitk_reduce then sums the parts in ascending order into c.
  int ksplit;
  float* c32;
};

// Up to two independent GEMM problems share one launch (their tiles are
// concatenated), so a short GEMM can fill the CUs another one leaves idle.
struct GemmLaunch {
  Problem p[2];
  float* split_ws;       // caller scratch for split-contraction partials (two-layout launch), or nullptr
  size_t split_bytes;    // its size
  int nprob;
  int tiles;             // bf16 whole-tile kernels: tiles of the launch
  int g0;                // two-layout launch: workgroups of problem 0
  int half_base;         // half-tile launch: first (256-row) tile it splits
  int half_tail;         // 1: a half-tile tail launch (tiles are halves from half_base on)
  int strided;           // 1: workgroup g runs tiles g, g + G, ... (else a contiguous range)
};

struct CEArgs {
  int64_t M, Vr, K;
  const void* H;
  int64_t ldh;
  const void* W;
  int64_t ldw;
  const int32_t* target;
  int64_t v0;
  float* out_max;
  float* out_sumexp;
  float* out_tgt;
  float* ws;             // [ceil(Vr/256)][M] (max,sum) pairs, then [M] target logits
};

// Log-sum-exp recombination of R vocab shards' (max, sum exp, target logit)
// triples: shard r's arrays start at maxes / sumexps / tgts + r * stride.
struct CECombineArgs {
  int R;
  int64_t M, stride;
  const float* maxes;
  const float* sumexps;
  const float* tgts;
  float* lse;            // each output [M], nullable
  float* tgt;
  float* loss;
};

// Elementwise backward of the column epilogue, fused with fp32 column
// partial sums for the bias gradients.
struct ActBwdArgs {
  int64_t M, N;
  int act;               // E_STORE (= no activation), E_GELU, E_SWIGLU
  const void* dY;
  int64_t lddy;
  const void* pre;
  int64_t ldpre;
  void* dp;              // gate part (or the only part) [M][lddp]; nullptr: not written
  void* dp_up;           // SwiGLU up part [M][lddp]
  int64_t lddp;
  float* colpart;        // [ceil(M/64)][2][ldcp] fp32 or nullptr
  int64_t ldcp;
};

struct SumArgs {
  int t;
  int64_t M, N;
  const void* parts;
  int64_t ld, part_stride;
  const void* bias;
  void* out;
  int64_t ldo;
};

// Sequence-parallel block boundary: reduce-scatter of the t row partials over
// rows [r0, r0 + Mr), + bias + residual, then LayerNorm.
struct SpLnArgs {
  int t;
  int64_t Mr, N;
  const void* parts;
  int64_t ld, part_stride, r0;
  const void* bias;
  const void* resid;
  int64_t ldr;
  const void* gamma;
  const void* beta;
  float eps;
  void* out;
  int64_t ldo;
  void* hout;
  int64_t ldh;
};

// Vocab-parallel embedding: forward src = the rank's table block E [Vr, K]
// (lds), dst = out [M, K] (ldd); backward src = dout [M, K], dst = dE [Vr, K].
struct EmbArgs {
  int64_t M, Vr, K;
  const int32_t* ids;
  int64_t v0;
  const void* src;
  int64_t lds;
  void* dst;
  int64_t ldd;
};

// Attention core: B sequences of S tokens stacked by rows; head h of Q/O in
// columns [128 h, 128 h + 128), KV head g of K/V likewise; lse fp32 [B][n_q][S].
struct AttnArgs {
  int64_t B, S;
  int n_q, n_kv;
  int causal;
  float scale;
  const void* q;
  int64_t ldq;
  const void* k;
  int64_t ldk;
  const void* v;
  int64_t ldv;
  void* o;
  int64_t ldo;
  float* lse;
  int chunk_tiles;   // key tiles (64 keys) per workgroup along a query block's key range
  int max_chunks;    // chunks of the longest query block; > 1 needs ws
  float* ws;         // per-chunk partial results (attn_fwd_workspace_bytes)
};

// Attention backward: the forward's arguments (o = the forward output, lse)
// plus dO and the three gradients; ld, dq_ws and kv_ws point into the
// workspace (attn_bwd_layout).
struct AttnBwdArgs {
  AttnArgs f;
  const void* dout;
  int64_t ldg;
  void* dq;
  int64_t lddq;
  void* dk;
  int64_t lddk;
  void* dv;
  int64_t lddv;
  float* ld;        // [B][n_q][S] pairs (lse * log2 e, sum_d dO * O)
  float* dq_ws;     // per-chunk partial dQ (when the forward chunking splits)
  float* kv_ws;     // per (query head, query chunk) partial dK, dV
  int kv_chunk_tiles;
  int kv_max_chunks;
};

struct AttnBwdLayout {
  int chunk_tiles, max_chunks, kv_chunk_tiles, kv_max_chunks;
  size_t ld_bytes, dq_bytes, kv_bytes;
};

constexpr int kSpLnMaxN = 16384;   // row width the LayerNorm kernel holds in registers

constexpr int kColpartRows = 64;   // rows per column-partial block

hipError_t launch_gemm_bf16(GemmLaunch& L, hipStream_t s);
// The one-launch schedule of a (TN weight gradient, NT input gradient) pair
// on `cus` CUs: its tile pairing (0: 256x256 + 256x256, 1: 192x256 +
// 256x192, 2: 192x192 + 128x192, 3: 128x128 + 128x192, 4: 128x128 +
// 256x256, 5: 128x192 + 256x192, 6: 128x192 + 128x192) with the workgroups
// of problem 0 and each problem's tile count, or -1 when the two run as
// separate launches.
// Host-only.
// With L.split_bytes > 0 the plan may also cut either problem's contraction
// into ks0 / ks1 parts (1, 2 or 4; fp32 partials in L.split_ws, summed by a
// second launch); `split_need` returns the bytes that plan uses.
int dual_plan(const GemmLaunch& L, int cus, int& g0, int64_t& t0, int64_t& t1);
int dual_plan(const GemmLaunch& L, int cus, int& g0, int64_t& t0, int64_t& t1, int& ks0, int& ks1,
              size_t& split_need);
hipError_t launch_gemm_f32(GemmLaunch& L, hipStream_t s);
hipError_t launch_ce_partials(const CEArgs& a, hipStream_t s);
// Size of the library's own CE scratch array (one per device), and its
// device address on the current device (looked up once per device).
constexpr size_t kCeScratchBytes = size_t(16) << 20;
hipError_t ce_scratch(float** out);
size_t ce_workspace_bytes(int64_t M, int64_t Vr);
hipError_t launch_act_bwd(int is_bf16, const ActBwdArgs& a, hipStream_t s);
hipError_t launch_ce_combine(const CECombineArgs& a, hipStream_t s);
hipError_t launch_colsum_finalize(int is_bf16, const float* colpart, int64_t nrb, int64_t ldcp,
                                  int64_t N, int part, void* out, hipStream_t s);
hipError_t launch_sum_partials(int is_bf16, const SumArgs& a, hipStream_t s);
hipError_t launch_sp_rs_ln(int is_bf16, const SpLnArgs& a, hipStream_t s);
hipError_t launch_emb_fwd(int is_bf16, const EmbArgs& a, hipStream_t s);
void attn_chunking(int64_t B, int64_t S, int n_q, int n_kv, int causal, int& chunk_tiles, int& max_chunks);
size_t attn_fwd_workspace_bytes(int64_t B, int64_t S, int n_q, int n_kv, int causal);
hipError_t launch_attn_fwd(const AttnArgs& a, hipStream_t s);
void attn_bwd_layout(int64_t B, int64_t S, int n_q, int n_kv, int causal, AttnBwdLayout& L);
hipError_t launch_attn_bwd(const AttnBwdArgs& p, hipStream_t s);
// start [Vr + 1] and order [M] int32 come from the caller's workspace.
hipError_t launch_emb_bwd(int is_bf16, const EmbArgs& a, int32_t* start, int32_t* order, hipStream_t s);

}  // namespace tps
