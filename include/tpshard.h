/*
 * tpshard.h -- C ABI of libtpshard: one tensor-parallel rank's share of a
 * transformer block on one MI355X (gfx950) GPU.
 *
 * Sources of the operations (page titles and sections):
 *   [TP/SP]  "v4: Tensor Parallel and Sequence Parallel"
 *   [TPcomm] "TP communication: how many all-reduces per layer, how much data"
 *
 * Common conventions
 * ------------------
 * Layout.    Every matrix is row-major with a leading dimension `ld` counted
 *            in elements (ld >= row width).  Weights use the math layout of
 *            Y = X W: a column shard A_i is [K, N_i], a row shard B_i is
 *            [K_i, N]; the LM-head shard W_r is [V_r, K] (vocab rows).
 * Pointers.  All tensor pointers are DEVICE pointers owned by the caller.
 *            The library never allocates or frees device memory.  Its only
 *            state is the per-GPU scratch array of
 *            tp_vocab_ce_partials_noalloc (see there); every other call is
 *            reentrant.
 * Streams.   `stream` is a hipStream_t (NULL = the null stream).  Every call
 *            validates its arguments synchronously, then only enqueues work
 *            on `stream` and returns; the caller synchronizes.
 * Errors.    Validation runs fully before anything is enqueued: on any error
 *            code except TP_E_HIP nothing is launched and no output byte is
 *            written.  A failed launch returns TP_E_HIP (outputs undefined).
 *            A device fault surfaces at the caller's next synchronization.
 * Shapes.    M, N, K >= 1 (int64, each < 2^31); tails of any size are masked
 *            inside the kernels.  A bf16 matrix must span less than 2 GiB:
 *            ((rows - 1) * ld + width rounded up to 8) * 2 bytes < 2^31
 *            (the kernels address operands with 32-bit offsets); otherwise
 *            TP_E_SHAPE.
 * Alignment. Every base pointer must be 16-byte aligned and every `ld` a
 *            multiple of 8 elements for bf16 (4 for fp32), so 16-byte vector
 *            accesses are legal.  The kernels may READ each input row up to
 *            its width rounded up to that multiple (never past ld); values
 *            there are ignored.  Outputs are written only inside their width.
 * Dtypes.    TP_BF16: bf16 storage, fp32 accumulation, fp32 epilogue math,
 *            outputs rounded to bf16 (round to nearest even).
 *            TP_FP32: fp32 storage and accumulation.
 *            Outputs take the input dtype except the CE outputs (fp32).
 * Aliasing.  Outputs must not overlap inputs or each other, except where a
 *            call states otherwise.
 * Determinism. No floating-point atomics: every sum runs in a fixed order,
 *            so two identical calls give bitwise identical outputs (the only
 *            atomics are integer counters, exact in any order).
 */
#ifndef TPSHARD_H
#define TPSHARD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TP_ABI_VERSION 1

#ifndef TP_API
#define TP_API __attribute__((visibility("default")))
#endif

typedef enum {
  TP_OK = 0,
  TP_E_NULL = 1,      /* a required pointer is NULL */
  TP_E_SHAPE = 2,     /* a size < 1 or >= 2^31, ld < width, t < 1 */
  TP_E_ALIGN = 3,     /* base pointer not 16-byte aligned or ld not a multiple of 8 (bf16) / 4 (fp32) */
  TP_E_DTYPE = 4,     /* unknown dtype, or dtype not supported by this call */
  TP_E_ACT = 5,       /* unknown activation, or activation arguments inconsistent */
  TP_E_WORKSPACE = 6, /* workspace NULL or smaller than the matching *_workspace_bytes() */
  TP_E_HIP = 7        /* a HIP launch failed */
} tp_status;

typedef enum { TP_FP32 = 0, TP_BF16 = 1 } tp_dtype;

typedef enum {
  TP_ACT_NONE = 0,
  TP_ACT_GELU = 1,   /* exact GeLU: x * Phi(x) = x/2 * (1 + erf(x / sqrt 2)) */
  TP_ACT_SWIGLU = 2  /* silu(gate) * up, silu(x) = x * sigmoid(x) */
} tp_act;

/* Returns TP_ABI_VERSION. */
TP_API int tp_abi_version(void);

/* Static, never-NULL description of a status code (unknown codes included). */
TP_API const char* tp_status_str(int status);

/*
 * Column-parallel shard forward.  [TP/SP] "TP math: block matrix
 * multiplication" (X[A_1, A_2] = [X A_1, X A_2]), "Full flow: column
 * parallel, t = 3" (f is the identity forward: the full X goes in; the column
 * bias is split with the columns) and "MLP: column first, then row" (GeLU or
 * SwiGLU gate x up applied locally on the shard).
 *
 *   P  = X A + bias                      X [M,K], A [K,N], bias [N] (nullable)
 *   NONE   : Y = P                        (Pre unused, may be NULL)
 *   GELU   : Y = GeLU(P),  Pre = P        Pre [M,N]
 *   SWIGLU : U = X A2 + bias2,  Y = silu(P) * U,
 *            Pre = [P | U]                Pre [M,2N]: P in columns [0,N), U in [N,2N)
 * Y is [M,N].  A2 is required for SWIGLU (else ignored); bias2 is nullable.
 * Pre holds the pre-activation (bias included) rounded to the dtype; the
 * column backward consumes it.
 */
TP_API tp_status tp_column_fwd(int dtype, int act, int64_t M, int64_t N, int64_t K,
                        const void* X, int64_t ldx, const void* A, int64_t lda,
                        const void* A2, int64_t lda2, const void* bias, const void* bias2,
                        void* Y, int64_t ldy, void* Pre, int64_t ldpre, void* stream);

/*
 * Row-parallel shard forward.  [TP/SP] "TP math": [X_1, X_2][A_1; A_2] =
 * X_1 A_1 + X_2 A_2.  The shard emits the full-shape partial Zp = X_i B_i,
 * X_i [M,K], B_i [K,N], Zp [M,N], in the input dtype.  No bias and no
 * activation: the bias is added once after the sum (tp_sum_partials) and an
 * activation cannot act on a partial ("MLP: column first, then row").
 */
TP_API tp_status tp_row_fwd(int dtype, int64_t M, int64_t N, int64_t K,
                     const void* Xi, int64_t ldx, const void* Bi, int64_t ldb,
                     void* Zp, int64_t ldz, void* stream);

/*
 * Sum of t shard partials held on ONE device -- the value that g's forward
 * all-reduce (or f's backward all-reduce) leaves on every rank; this is not a
 * collective.  [TP/SP] "Full flow" (f and g), "Self-test" (the row bias is
 * added once, after the sum); [TPcomm] Fig. 2.
 *
 *   out = sum_{i<t} parts_i (+ bias once)     parts_i = parts + i*part_stride (elements)
 * Each parts_i is [M,N] with leading dimension ld; out is [M,N] with ldo;
 * bias [N] nullable.  Accumulation is fp32 in ascending i with one final
 * rounding.  `out` may be exactly parts_0 (same pointer, ldo == ld); no other
 * overlap is allowed.  part_stride must be a multiple of 8 (bf16) / 4 (fp32).
 */
TP_API tp_status tp_sum_partials(int dtype, int t, int64_t M, int64_t N,
                          const void* parts, int64_t ld, int64_t part_stride,
                          const void* bias, void* out, int64_t ldo, void* stream);

/*
 * Row-parallel shard backward.  [TP/SP] "Where column and row communicate":
 * g's backward is the identity, so the shard holds the full dZ and its input
 * gradient dX_i = dZ B_i^T is local; the weight gradient is dB_i = X_i^T dZ.
 *
 *   dXi   = dZ  B_i^T     dZ [M,N], B_i [K,N] -> dXi [M,K]     (nullable: skipped)
 *   dBi   = X_i^T dZ      X_i [M,K]           -> dBi [K,N]     (nullable: skipped)
 *   dbias = sum_m dZ      fp32-accumulated, dtype out, [N]     (nullable: skipped)
 * dbias is the gradient of the replicated row bias; it needs a workspace of
 * tp_row_bwd_workspace_bytes() bytes (workspace may be NULL when dbias is NULL).
 *
 * Split contractions (bf16, dXi and dBi both requested): workspace bytes past
 * tp_row_bwd_workspace_bytes(dtype, M, N) -- whether or not dbias is asked
 * for -- are scratch that lets the one-launch schedule cut a long contraction
 * into 2 or 4 parts (fp32 partial products [parts][rows][cols], then a second
 * kernel sums them in ascending part order and rounds once to bf16).  It is
 * taken only when it fits; tp_row_bwd_workspace_bytes_split() is the size
 * that the fastest schedule for these sizes uses.  The workspace must be
 * 16-byte aligned for the split to be taken.  Results may differ from the
 * unsplit schedule's in the fp32 summation order only.
 */
TP_API tp_status tp_row_bwd(int dtype, int64_t M, int64_t N, int64_t K,
                     const void* dZ, int64_t lddz, const void* Xi, int64_t ldx,
                     const void* Bi, int64_t ldb,
                     void* dXi, int64_t lddx, void* dBi, int64_t lddb, void* dbias,
                     void* workspace, size_t ws_bytes, void* stream);
TP_API size_t tp_row_bwd_workspace_bytes(int dtype, int64_t M, int64_t N);
/* Workspace for tp_row_bwd with room for its split-contraction schedule on a
 * GPU with `cus` compute units (host only; 0 for invalid sizes). */
TP_API size_t tp_row_bwd_workspace_bytes_split(int dtype, int64_t M, int64_t N, int64_t K, int cus);

/*
 * Planning query for tp_row_bwd (bf16, dXi and dBi both requested): which
 * tile pairing its one-launch schedule of the two GEMMs takes for these sizes
 * (same M, N, K as tp_row_bwd, 16-byte aligned operands) on a GPU with `cus`
 * compute units.  For schedulers and tests that want the launch shape; host
 * only: no GPU call, no allocation.  Returns 0 (256x256 weight-gradient tiles
 * beside 256x256 input-gradient tiles), 1 (192x256 beside 256x192), 2
 * (192x192 beside 128x192), 3 (128x128 beside 128x192), 4 (128x128 beside
 * 256x256), 5 (128x192 beside 256x192), 6 (128x192 beside 128x192), -1 (the
 * two GEMMs run as separate launches), or -2 for sizes tp_row_bwd rejects or
 * cus < 1.
 */
TP_API int tp_row_bwd_plan(int64_t M, int64_t N, int64_t K, int cus);
/* As tp_row_bwd_plan with `split_bytes` of split scratch available (the
 * workspace past tp_row_bwd_workspace_bytes): also returns how many parts
 * each contraction is cut into (*ks_dB for dBi over M, *ks_dX for dXi over
 * N; 1 = not cut, also for a return of -1 or -2; either pointer may be
 * NULL). */
TP_API int tp_row_bwd_plan_split(int64_t M, int64_t N, int64_t K, int cus, size_t split_bytes, int* ks_dB,
                                 int* ks_dX);

/*
 * Column-parallel shard backward.  [TP/SP] "Where column and row
 * communicate" and "Full flow: column parallel, t = 3": the input gradient is
 * a partial (dX = sum_i dY_i A_i^T, summed by f's backward -- use
 * tp_sum_partials), the weight gradient dA_i = X^T dY_i is complete locally.
 *
 *   dP      = dY                               (NONE)
 *           = dY * GeLU'(Pre)                  (GELU, Pre [M,N])
 *           = [dY*U*silu'(G) | dY*silu(G)]     (SWIGLU, Pre = [G|U] [M,2N])
 *   dXpart  = dP_g A^T (+ dP_u A2^T)           [M,K]  (nullable: skipped)
 *   dA      = X^T dP_g,  dA2 = X^T dP_u        [K,N]  (nullable: skipped; SWIGLU: both or neither)
 *   dbias   = sum_m dP_g, dbias2 = sum_m dP_u  [N]    (nullable)
 * dY [M,N], X [M,K], A/A2 [K,N].  dP is materialized in the workspace, in the
 * dtype, for GELU/SWIGLU; bias gradients use fp32 partial sums there too.
 * ws_bytes must be >= tp_column_bwd_workspace_bytes(dtype, act, M, N, bias
 * gradients requested).  Without an activation (bf16, dXpart and dA both
 * requested) the two GEMMs run as tp_row_bwd's do, and workspace bytes past
 * that size are split-contraction scratch as described there
 * (tp_column_bwd_workspace_bytes_split: the size the fastest schedule uses).
 */
TP_API tp_status tp_column_bwd(int dtype, int act, int64_t M, int64_t N, int64_t K,
                        const void* dY, int64_t lddy, const void* X, int64_t ldx,
                        const void* A, int64_t lda, const void* A2, int64_t lda2,
                        const void* Pre, int64_t ldpre,
                        void* dXpart, int64_t lddx, void* dA, int64_t ldda,
                        void* dA2, int64_t ldda2, void* dbias, void* dbias2,
                        void* workspace, size_t ws_bytes, void* stream);
TP_API size_t tp_column_bwd_workspace_bytes(int dtype, int act, int64_t M, int64_t N, int with_bias_grad);
TP_API size_t tp_column_bwd_workspace_bytes_split(int dtype, int act, int64_t M, int64_t N, int64_t K,
                                                  int with_bias_grad, int cus);

/*
 * Vocab-parallel LM-head shard with cross-entropy partials.  [TP/SP]
 * "Embedding and LM head: split by vocab": the LM head is column parallel
 * over the vocabulary and the loss never gathers the logits -- each token
 * all-reduces only the max, the sum of e^z and the target logit.
 *
 * Shard [v0, v0+Vr):  z = H W^T (H [M,K], W [Vr,K]); z is never written.
 *   out_max[m]    = max_j z[m,j]
 *   out_sumexp[m] = sum_j exp(z[m,j] - out_max[m])
 *   out_tgt[m]    = z[m, target[m]-v0] if v0 <= target[m] < v0+Vr, else 0
 * target: int32 [M] (device).  Outputs fp32 [M] (device).  Logits, exp and
 * sums are fp32.  workspace >= tp_vocab_ce_workspace_bytes(M, Vr).
 * Only TP_BF16 is supported (TP_FP32 returns TP_E_DTYPE).
 * Combining shards: M* = max_r m_r, S* = sum_r s_r e^(m_r-M*),
 * lse = M* + ln S*, loss = lse - sum_r tgt_r.
 */
TP_API tp_status tp_vocab_ce_partials(int dtype, int64_t M, int64_t Vr, int64_t K,
                               const void* H, int64_t ldh, const void* W, int64_t ldw,
                               const int32_t* target, int64_t v0,
                               float* out_max, float* out_sumexp, float* out_tgt,
                               void* workspace, size_t ws_bytes, void* stream);
TP_API size_t tp_vocab_ce_workspace_bytes(int64_t M, int64_t Vr);

/*
 * tp_vocab_ce_partials without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, kernels and results as
 * tp_vocab_ce_partials minus the workspace: the per-tile partials live in a
 * scratch array of TP_CE_NOALLOC_SCRATCH_BYTES inside the library, one per
 * GPU, held until the process ends (its address is looked up on the first
 * call on each device).  The call allocates nothing.
 * Limit: tp_vocab_ce_workspace_bytes(M, Vr) = (2*ceil(Vr/256) + 1) * M * 4
 * bytes must not exceed TP_CE_NOALLOC_SCRATCH_BYTES (16 MiB: e.g. M = 8192
 * tokens with Vr up to 65280), else TP_E_WORKSPACE and nothing is launched.
 * Every call on one GPU uses that GPU's one array: calls that overlap in time
 * on the same GPU (other streams, other threads) race and give undefined
 * results; calls on one stream run in order and are safe.  No part of the
 * array needs to start at zero (every byte read is written first).
 */
#define TP_CE_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
TP_API tp_status tp_vocab_ce_partials_noalloc(int dtype, int64_t M, int64_t Vr, int64_t K,
                                              const void* H, int64_t ldh, const void* W, int64_t ldw,
                                              const int32_t* target, int64_t v0,
                                              float* out_max, float* out_sumexp, float* out_tgt,
                                              void* stream);

/*
 * Recombination of the vocab shards' cross-entropy partials: the value the
 * all-reduce of the three per-token numbers leaves, computed on one device
 * (not a collective).  [TP/SP] "Embedding and LM head: split by vocab": each
 * token exchanges only its shard max, sum of e^z and target logit, and the
 * loss follows from them:
 *
 *   M*[m]   = max_r max_r[m]
 *   S*[m]   = sum_r sumexp_r[m] * exp(max_r[m] - M*[m])     (ascending r)
 *   lse[m]  = M*[m] + ln S*[m]
 *   tgt[m]  = sum_r tgt_r[m]            (exactly one shard owns each target)
 *   loss[m] = lse[m] - tgt[m]
 *
 * R >= 1 shards; shard r's triple is maxes + r*stride, sumexps + r*stride,
 * tgts + r*stride (fp32 [M] each, the outputs of tp_vocab_ce_partials for
 * that shard; stride >= M, a multiple of 4, R*stride < 2^31).  Outputs lse,
 * tgt, loss: fp32 [M] each, device, nullable (not all three NULL).  The
 * arithmetic is fp64 with one rounding to fp32 per output; lse feeds
 * tp_vocab_ce_bwd.  A token whose shard maxes are all -inf gets lse = -inf.
 */
TP_API tp_status tp_vocab_ce_combine(int R, int64_t M, const float* maxes, const float* sumexps,
                                     const float* tgts, int64_t stride, float* lse, float* tgt, float* loss,
                                     void* stream);

/*
 * Backward of the vocab-parallel cross entropy for shard [v0, v0+Vr).
 * [TP/SP] "Embedding and LM head: split by vocab": with the per-token
 * log-sum-exp recombined over all shards, each rank differentiates its own
 * logits locally; its weight gradient completes locally and its input
 * gradient is a partial summed over the shards (like the column-parallel dX).
 *
 *   z  = H W^T, recomputed tile by tile (the forward stored no logits)
 *   dz = gscale[m] * (exp(z[m,j] - lse[m]) - [j == target[m]-v0])
 *   dH = dz W    [M, K]: this shard's partial (nullable: not computed)
 *   dW = dz^T H  [Vr, K]: the shard's weight gradient (nullable)
 * lse: fp32 [M], the recombined lse (M* + ln S* over all shards).
 * gscale: fp32 [M], upstream gradient of each token's loss; NULL means 1.
 * target: int32 [M]; a target outside [v0, v0+Vr) (negative included) adds
 * no onehot term on this shard.  dz is stored as bf16 in the workspace
 * (>= tp_vocab_ce_bwd_workspace_bytes(M, Vr)) between its two GEMMs; exp
 * and the subtraction are fp32.  Outputs take the input dtype.  Only TP_BF16
 * is supported (TP_FP32 returns TP_E_DTYPE).
 */
TP_API tp_status tp_vocab_ce_bwd(int dtype, int64_t M, int64_t Vr, int64_t K,
                                 const void* H, int64_t ldh, const void* W, int64_t ldw,
                                 const int32_t* target, int64_t v0, const float* lse, const float* gscale,
                                 void* dH, int64_t lddh, void* dW, int64_t lddw,
                                 void* workspace, size_t ws_bytes, void* stream);
TP_API size_t tp_vocab_ce_bwd_workspace_bytes(int64_t M, int64_t Vr);

/*
 * Sequence-parallel block boundary of one rank, on one device (not a
 * collective).  [TP/SP] section "SP: shard the activations that TP leaves
 * whole": the all-reduce after the row-parallel layer becomes a
 * reduce-scatter, so each rank keeps the sum for its own block of tokens, and
 * the residual add and LayerNorm that follow are per-token work done on that
 * block only; [TPcomm] Fig. 2 (reduce-scatter half of the all-reduce).
 * Rank rows [r0, r0 + Mr) of the t partials parts_i [M, N] (ld; parts_i =
 * parts + i*part_stride elements):
 *
 *   h[m]   = sum_{i<t} parts_i[r0 + m] (ascending i) + bias + resid[m]
 *   out[m] = (h[m] - mean) / sqrt(var + eps) * gamma + beta
 *
 * mean and var (biased, 1/N) are over the N columns of h[m]; m in [0, Mr).
 * bias, gamma, beta: [N], nullable (absent = 0, 1, 0).  resid: the rank's
 * [Mr, N] block (ldr), nullable.  hout: [Mr, N] (ldh), nullable -- the
 * residual stream h rounded to the dtype; hout may be exactly resid (same
 * pointer, ldh == ldr) to update the residual stream in place.  out: [Mr, N]
 * (ldo).  h, mean, var and the normalisation are fp32 from unrounded h.
 * Limits: 1 <= N <= 16384 and 0 <= r0, r0 + Mr <= M; eps >= 0 and finite;
 * otherwise TP_E_SHAPE.  part_stride: a multiple of 8 (bf16) / 4 (fp32).
 */
TP_API tp_status tp_sp_reduce_scatter_ln(int dtype, int t, int64_t M, int64_t N,
                                         const void* parts, int64_t ld, int64_t part_stride,
                                         int64_t r0, int64_t Mr, const void* bias,
                                         const void* resid, int64_t ldr,
                                         const void* gamma, const void* beta, float eps,
                                         void* out, int64_t ldo, void* hout, int64_t ldh,
                                         void* stream);

/*
 * Vocab-parallel embedding lookup of one rank.  [TP/SP] "Embedding and LM
 * head: split by vocab": the embedding table is split by rows (token ids)
 * into t blocks; the rank holding rows [v0, v0 + Vr) outputs, for each
 * token, its row when the rank owns the id and a zero row otherwise, so the
 * all-reduce (tp_sum_partials on one device) gives every token its own row.
 *
 *   out[m] = E[ids[m] - v0]   if v0 <= ids[m] < v0 + Vr,   else 0
 *
 * ids: int32 [M] (any value; ids of other ranks, negative ids and ids past
 * the table give zero rows).  E: the rank's block [Vr, K] (lde).  out:
 * [M, K] (ldo).  Rows are copied bit for bit (no arithmetic).
 */
TP_API tp_status tp_vocab_embed_fwd(int dtype, int64_t M, int64_t Vr, int64_t K,
                                    const int32_t* ids, int64_t v0,
                                    const void* E, int64_t lde, void* out, int64_t ldo,
                                    void* stream);

/*
 * Backward of tp_vocab_embed_fwd: the gradient of the rank's table block.
 * Same section: the lookup copies row ids[m] - v0 to token m, so
 *
 *   dE[v] = sum of dout[m] over the tokens m with ids[m] = v0 + v
 *
 * added in ascending m in fp32 and rounded once; rows no token uses are
 * written as zeros (dE [Vr, K] is overwritten completely).  dout: [M, K]
 * (lddo).  The tokens are grouped by row through a stable counting sort in
 * the workspace (>= tp_vocab_embed_bwd_workspace_bytes(M, Vr) bytes), so the
 * result does not depend on scheduling; no floating-point atomics.
 */
TP_API tp_status tp_vocab_embed_bwd(int dtype, int64_t M, int64_t Vr, int64_t K,
                                    const int32_t* ids, int64_t v0,
                                    const void* dout, int64_t lddo, void* dE, int64_t ldde,
                                    void* workspace, size_t ws_bytes, void* stream);
TP_API size_t tp_vocab_embed_bwd_workspace_bytes(int64_t M, int64_t Vr);

/*
 * Attention core of one rank's heads, between the column-parallel QKV
 * projection and the row-parallel W_O.  [TP/SP] "Attention: split by head":
 * each head is computed on its own, so the rank attends with its n_q query
 * heads locally, without communication; with GQA (32 query / 8 KV heads at
 * t = 8: 4 query heads and 1 KV head per rank) query head h reads KV head
 * h / (n_q / n_kv).  Per head, over the keys of its sequence:
 *
 *   O_h = softmax(Q_h K_g^T * scale  [+ causal mask: key > query -> -inf]) V_g
 *   lse[b][h][i] = log sum_j exp(s_ij)       (natural log, fp32, masked keys excluded)
 *
 * B sequences of S tokens are stacked by rows (sequence b = rows
 * [b S, b S + S)).  Q [B S, n_q * 128] (ldq), K and V [B S, n_kv * 128]
 * (ldk, ldv); head h in columns [128 h, 128 h + 128).  The packed QKV output
 * of tp_column_fwd is passed as Q = qkv, K = qkv + 128 n_q, V = qkv +
 * 128 (n_q + n_kv), all with ld = 128 (n_q + 2 n_kv).  O [B S, n_q * 128]
 * (ldo), the W_O input; lse fp32 [B][n_q][S] (kept for the backward).
 * head_dim must be 128; n_q / n_kv must divide 4 or be a multiple of 4;
 * scale > 0 (1/sqrt(128) for the usual attention); causal is 0 or 1.
 * Scores, softmax and accumulation are fp32; the probabilities enter the
 * second product as bf16.  Only TP_BF16.  Long key ranges are cut into
 * chunks run by separate workgroups and merged in a fixed order; their
 * partial results need a workspace of tp_attention_fwd_workspace_bytes()
 * bytes (0 = none needed; workspace may then be NULL).
 */
TP_API tp_status tp_attention_fwd(int dtype, int64_t B, int64_t S, int n_q, int n_kv, int head_dim,
                                  int causal, float scale,
                                  const void* Q, int64_t ldq, const void* K, int64_t ldk,
                                  const void* V, int64_t ldv, void* O, int64_t ldo, float* lse,
                                  void* workspace, size_t ws_bytes, void* stream);
/* Workspace of tp_attention_fwd for this shape (head_dim 128); 0 for an invalid shape. */
TP_API size_t tp_attention_fwd_workspace_bytes(int64_t B, int64_t S, int n_q, int n_kv, int causal);

/*
 * Backward of tp_attention_fwd (the pages print no backward; the textbook
 * gradients of softmax attention).  With P = softmax(s) recomputed from the
 * forward's lse, per head:
 *
 *   dV_g += P^T dO_h        dP = dO_h V_g^T        dS = P * (dP - D),
 *   D_i  = sum_j P_ij dP_ij = sum_d dO_h[i] O_h[i]   (fp32, from O and dO)
 *   dQ_h  = dS K_g * scale  dK_g += dS^T Q_h * scale
 *
 * A KV head's dK, dV sum over the query heads that read it.  Shapes and
 * layouts as tp_attention_fwd; O and lse are that call's outputs, dO is
 * [B S, n_q * 128] (lddo); dQ [B S, n_q * 128], dK and dV [B S, n_kv * 128]
 * are written completely.  Products in bf16 with fp32 accumulation; partial
 * results (key chunks for dQ, query heads and query chunks for dK and dV)
 * live in the workspace (>= tp_attention_bwd_workspace_bytes()) and are
 * summed in a fixed order: no atomics.  Only TP_BF16.
 */
TP_API tp_status tp_attention_bwd(int dtype, int64_t B, int64_t S, int n_q, int n_kv, int head_dim,
                                  int causal, float scale,
                                  const void* Q, int64_t ldq, const void* K, int64_t ldk,
                                  const void* V, int64_t ldv, const void* O, int64_t ldo,
                                  const float* lse, const void* dO, int64_t lddo,
                                  void* dQ, int64_t lddq, void* dK, int64_t lddk, void* dV, int64_t lddv,
                                  void* workspace, size_t ws_bytes, void* stream);
TP_API size_t tp_attention_bwd_workspace_bytes(int64_t B, int64_t S, int n_q, int n_kv, int causal);

#ifdef __cplusplus
}
#endif
#endif /* TPSHARD_H */
