// C ABI of libtpshard (declared in include/tpshard.h): argument validation,
// workspace carving and kernel dispatch.  Every entry point validates all of
// its arguments before it enqueues anything.
#include "tpshard.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "kernels.hpp"

namespace {

using tps::GemmLaunch;
using tps::Problem;

constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;
constexpr size_t kWsAlign = 256;

bool valid_dtype(int d) { return d == TP_FP32 || d == TP_BF16; }
bool valid_act(int a) { return a == TP_ACT_NONE || a == TP_ACT_GELU || a == TP_ACT_SWIGLU; }
int64_t vec_elems(int dtype) { return dtype == TP_BF16 ? 8 : 4; }
size_t esize(int dtype) { return dtype == TP_BF16 ? 2 : 4; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
bool bad_dim(int64_t v) { return v < 1 || v > kMaxDim; }
int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }
size_t align_ws(size_t v) { return (v + kWsAlign - 1) / kWsAlign * kWsAlign; }

// bf16 matrices are addressed through buffer descriptors with 32-bit
// offsets (a lane's offset plus a stage offset): the bytes from a matrix's
// base to the end of its last row (width rounded up to 8 elements) must stay
// below 2 GiB.
bool bf16_extent_ok(int64_t rows, int64_t ld, int64_t width) {
  constexpr int64_t kMaxElems = int64_t(0x7fffffff) / 2;
  if (rows > 1 && ld > kMaxElems / (rows - 1)) return false;
  return (rows - 1) * ld + round_up(width, 8) <= kMaxElems;
}

// Matrix operand: [rows][ld] with `width` used columns.  Rows are validated
// separately (bad_dim); here: ld range, extent, ld multiple, base alignment.
tp_status check_mat(const void* p, int64_t rows, int64_t ld, int64_t width, int dtype) {
  if (ld < width || ld > (int64_t(1) << 40)) return TP_E_SHAPE;
  if (dtype == TP_BF16 && !bf16_extent_ok(rows, ld, width)) return TP_E_SHAPE;
  if (ld % vec_elems(dtype) != 0 || !aligned16(p)) return TP_E_ALIGN;
  return TP_OK;
}

tp_status check_vec(const void* p) { return (p && !aligned16(p)) ? TP_E_ALIGN : TP_OK; }

#define TPS_TRY(expr)                  \
  do {                                 \
    const tp_status st_ = (expr);      \
    if (st_ != TP_OK) return st_;      \
  } while (0)

// Tile-count limits of the launch grids (bf16: counted in 256 x 128 tiles, the
// SwiGLU tile; the launcher takes narrower tiles, down to 128 x 192, only when
// their count also fits in an int; fp32: 64 x 32 tiles with the row tiles on
// grid.y).
tp_status check_grid(int dtype, int64_t M, int64_t N) {
  if (dtype == TP_BF16) {
    if (((M + 255) / 256) * ((N + 127) / 128) > kMaxDim) return TP_E_SHAPE;
  } else {
    if ((M + 63) / 64 > 65535 || (N + 31) / 32 > kMaxDim) return TP_E_SHAPE;
  }
  return TP_OK;
}

hipError_t run_gemm(int dtype, GemmLaunch& L, hipStream_t s) {
  return dtype == TP_BF16 ? tps::launch_gemm_bf16(L, s) : tps::launch_gemm_f32(L, s);
}

Problem make_problem(int64_t M, int64_t N, int layout, int epi) {
  Problem P = {};
  P.M = M;
  P.N = N;
  P.layout = layout;
  P.epi = epi;
  P.nseg = 1;
  return P;
}

// tp_row_bwd's two GEMMs as one launch: dB_i = X_i^T dZ (TN over M), then
// dX_i = dZ B_i^T (NT over N).
GemmLaunch row_bwd_pair(int64_t M, int64_t N, int64_t K, const void* dZ, int64_t lddz, const void* Xi,
                        int64_t ldx, const void* Bi, int64_t ldb, void* dXi, int64_t lddx, void* dBi,
                        int64_t lddb) {
  GemmLaunch L = {};
  L.nprob = 2;
  L.p[0] = make_problem(K, N, tps::L_TN, tps::E_STORE);
  L.p[0].seg[0] = tps::Seg{Xi, dZ, ldx, lddz, M};
  L.p[0].c = dBi;
  L.p[0].ldc = lddb;
  L.p[1] = make_problem(M, K, tps::L_NT, tps::E_STORE);
  L.p[1].seg[0] = tps::Seg{dZ, Bi, lddz, ldb, N};
  L.p[1].c = dXi;
  L.p[1].ldc = lddx;
  return L;
}

int64_t colpart_rows(int64_t M) { return (M + tps::kColpartRows - 1) / tps::kColpartRows; }

size_t colpart_bytes(int64_t M, int64_t N) {
  return align_ws((size_t)colpart_rows(M) * 2 * (size_t)round_up(N, 4) * sizeof(float));
}

size_t dp_bytes(int dtype, int64_t M, int64_t N) {
  return align_ws((size_t)M * (size_t)round_up(N, 8) * esize(dtype));
}

// The workspace past `used` bytes, as scratch for split-contraction partials.
void give_split_ws(GemmLaunch& L, void* workspace, size_t ws_bytes, size_t used) {
  if (workspace && ws_bytes > used) {
    L.split_ws = reinterpret_cast<float*>(static_cast<char*>(workspace) + used);
    L.split_bytes = ws_bytes - used;
  }
}

// Bytes of split-contraction scratch the one-launch schedule of L takes on
// `cus` CUs when scratch is unlimited (0: it does not split).
size_t split_scratch(GemmLaunch L, int cus) {
  L.split_ws = reinterpret_cast<float*>(uintptr_t(256));
  L.split_bytes = SIZE_MAX;
  int g0 = 0, ks0 = 1, ks1 = 1;
  int64_t t0 = 0, t1 = 0;
  size_t need = 0;
  return tps::dual_plan(L, cus, g0, t0, t1, ks0, ks1, need) >= 0 ? need : 0;
}

// Stand-in operands for host-only planning queries: aligned addresses,
// leading dimensions rounded up to 8 elements.
GemmLaunch row_bwd_standin(int64_t M, int64_t N, int64_t K) {
  char* const p = reinterpret_cast<char*>(uintptr_t(256));
  return row_bwd_pair(M, N, K, p, round_up(N, 8), p, round_up(K, 8), p, round_up(N, 8), p, round_up(K, 8), p,
                      round_up(N, 8));
}

}  // namespace

extern "C" {

int tp_abi_version(void) { return TP_ABI_VERSION; }

const char* tp_status_str(int status) {
  switch (status) {
    case TP_OK: return "TP_OK: success";
    case TP_E_NULL: return "TP_E_NULL: a required pointer is NULL";
    case TP_E_SHAPE: return "TP_E_SHAPE: a size is out of range or a leading dimension is smaller than the row width";
    case TP_E_ALIGN: return "TP_E_ALIGN: a pointer is not 16-byte aligned or a leading dimension is not a multiple of 8 (bf16) / 4 (fp32) elements";
    case TP_E_DTYPE: return "TP_E_DTYPE: unknown dtype or dtype not supported by this call";
    case TP_E_ACT: return "TP_E_ACT: unknown activation or inconsistent activation arguments";
    case TP_E_WORKSPACE: return "TP_E_WORKSPACE: workspace missing or too small";
    case TP_E_HIP: return "TP_E_HIP: a HIP kernel launch failed";
    default: return "unknown tp_status code";
  }
}

tp_status tp_column_fwd(int dtype, int act, int64_t M, int64_t N, int64_t K, const void* X, int64_t ldx,
                        const void* A, int64_t lda, const void* A2, int64_t lda2, const void* bias,
                        const void* bias2, void* Y, int64_t ldy, void* Pre, int64_t ldpre, void* stream) {
  if (!valid_dtype(dtype)) return TP_E_DTYPE;
  if (!valid_act(act)) return TP_E_ACT;
  if (!X || !A || !Y) return TP_E_NULL;
  if (act != TP_ACT_NONE && !Pre) return TP_E_NULL;
  if (act == TP_ACT_SWIGLU && !A2) return TP_E_NULL;
  if (bad_dim(M) || bad_dim(N) || bad_dim(K)) return TP_E_SHAPE;
  TPS_TRY(check_grid(dtype, M, N));
  TPS_TRY(check_mat(X, M, ldx, K, dtype));
  TPS_TRY(check_mat(A, K, lda, N, dtype));
  if (act == TP_ACT_SWIGLU) TPS_TRY(check_mat(A2, K, lda2, N, dtype));
  TPS_TRY(check_mat(Y, M, ldy, N, dtype));
  if (act != TP_ACT_NONE) TPS_TRY(check_mat(Pre, M, ldpre, act == TP_ACT_SWIGLU ? 2 * N : N, dtype));
  TPS_TRY(check_vec(bias));
  if (act == TP_ACT_SWIGLU) TPS_TRY(check_vec(bias2));

  GemmLaunch L = {};
  L.nprob = 1;
  Problem& P = L.p[0];
  P = make_problem(M, N, tps::L_NN, act == TP_ACT_NONE ? tps::E_STORE : act == TP_ACT_GELU ? tps::E_GELU : tps::E_SWIGLU);
  P.seg[0] = tps::Seg{X, A, ldx, lda, K};
  if (act == TP_ACT_SWIGLU) {
    P.b_up = A2;
    P.ldb_up = lda2;
    P.bias2 = bias2;
  }
  P.bias = bias;
  P.c = Y;
  P.ldc = ldy;
  P.pre = Pre;
  P.ldpre = ldpre;
  return run_gemm(dtype, L, static_cast<hipStream_t>(stream)) == hipSuccess ? TP_OK : TP_E_HIP;
}

tp_status tp_row_fwd(int dtype, int64_t M, int64_t N, int64_t K, const void* Xi, int64_t ldx, const void* Bi,
                     int64_t ldb, void* Zp, int64_t ldz, void* stream) {
  if (!valid_dtype(dtype)) return TP_E_DTYPE;
  if (!Xi || !Bi || !Zp) return TP_E_NULL;
  if (bad_dim(M) || bad_dim(N) || bad_dim(K)) return TP_E_SHAPE;
  TPS_TRY(check_grid(dtype, M, N));
  TPS_TRY(check_mat(Xi, M, ldx, K, dtype));
  TPS_TRY(check_mat(Bi, K, ldb, N, dtype));
  TPS_TRY(check_mat(Zp, M, ldz, N, dtype));
  GemmLaunch L = {};
  L.nprob = 1;
  L.p[0] = make_problem(M, N, tps::L_NN, tps::E_STORE);
  L.p[0].seg[0] = tps::Seg{Xi, Bi, ldx, ldb, K};
  L.p[0].c = Zp;
  L.p[0].ldc = ldz;
  return run_gemm(dtype, L, static_cast<hipStream_t>(stream)) == hipSuccess ? TP_OK : TP_E_HIP;
}

tp_status tp_sum_partials(int dtype, int t, int64_t M, int64_t N, const void* parts, int64_t ld,
                          int64_t part_stride, const void* bias, void* out, int64_t ldo, void* stream) {
  if (!valid_dtype(dtype)) return TP_E_DTYPE;
  if (!parts || !out) return TP_E_NULL;
  if (t < 1 || bad_dim(M) || bad_dim(N) || part_stride < 0) return TP_E_SHAPE;
  TPS_TRY(check_mat(parts, M, ld, N, dtype));
  TPS_TRY(check_mat(out, M, ldo, N, dtype));
  if (part_stride % vec_elems(dtype) != 0) return TP_E_ALIGN;
  TPS_TRY(check_vec(bias));
  tps::SumArgs a = {t, M, N, parts, ld, part_stride, bias, out, ldo};
  return tps::launch_sum_partials(dtype == TP_BF16, a, static_cast<hipStream_t>(stream)) == hipSuccess ? TP_OK
                                                                                                       : TP_E_HIP;
}

tp_status tp_sp_reduce_scatter_ln(int dtype, int t, int64_t M, int64_t N, const void* parts, int64_t ld,
                                  int64_t part_stride, int64_t r0, int64_t Mr, const void* bias, const void* resid,
                                  int64_t ldr, const void* gamma, const void* beta, float eps, void* out, int64_t ldo,
                                  void* hout, int64_t ldh, void* stream) {
  if (!valid_dtype(dtype)) return TP_E_DTYPE;
  if (!parts || !out) return TP_E_NULL;
  if (t < 1 || bad_dim(M) || bad_dim(N) || N > tps::kSpLnMaxN || part_stride < 0) return TP_E_SHAPE;
  if (bad_dim(Mr) || r0 < 0 || r0 > M - Mr) return TP_E_SHAPE;
  if (!(eps >= 0.f) || !(eps <= 3.4e38f)) return TP_E_SHAPE;   // rejects NaN and inf
  TPS_TRY(check_mat(parts, M, ld, N, dtype));
  if (part_stride % vec_elems(dtype) != 0) return TP_E_ALIGN;
  TPS_TRY(check_mat(out, Mr, ldo, N, dtype));
  if (resid) TPS_TRY(check_mat(resid, Mr, ldr, N, dtype));
  if (hout) TPS_TRY(check_mat(hout, Mr, ldh, N, dtype));
  if (hout && hout == resid && ldh != ldr) return TP_E_SHAPE;
  TPS_TRY(check_vec(bias));
  TPS_TRY(check_vec(gamma));
  TPS_TRY(check_vec(beta));
  tps::SpLnArgs a = {t, Mr, N, parts, ld, part_stride, r0, bias, resid, ldr, gamma, beta, eps, out, ldo, hout, ldh};
  return tps::launch_sp_rs_ln(dtype == TP_BF16, a, static_cast<hipStream_t>(stream)) == hipSuccess ? TP_OK
                                                                                                   : TP_E_HIP;
}

size_t tp_row_bwd_workspace_bytes(int dtype, int64_t M, int64_t N) {
  (void)dtype;
  if (bad_dim(M) || bad_dim(N)) return 0;
  return colpart_bytes(M, N);
}

tp_status tp_row_bwd(int dtype, int64_t M, int64_t N, int64_t K, const void* dZ, int64_t lddz, const void* Xi,
                     int64_t ldx, const void* Bi, int64_t ldb, void* dXi, int64_t lddx, void* dBi, int64_t lddb,
                     void* dbias, void* workspace, size_t ws_bytes, void* stream) {
  if (!valid_dtype(dtype)) return TP_E_DTYPE;
  if (!dZ || !Xi || !Bi) return TP_E_NULL;
  if (bad_dim(M) || bad_dim(N) || bad_dim(K)) return TP_E_SHAPE;
  TPS_TRY(check_grid(dtype, M, K));
  TPS_TRY(check_grid(dtype, K, N));
  TPS_TRY(check_mat(dZ, M, lddz, N, dtype));
  TPS_TRY(check_mat(Xi, M, ldx, K, dtype));
  TPS_TRY(check_mat(Bi, K, ldb, N, dtype));
  if (dXi) TPS_TRY(check_mat(dXi, M, lddx, K, dtype));
  if (dBi) TPS_TRY(check_mat(dBi, K, lddb, N, dtype));
  TPS_TRY(check_vec(dbias));
  if (dbias) {
    if (!workspace || ws_bytes < tp_row_bwd_workspace_bytes(dtype, M, N)) return TP_E_WORKSPACE;
    if (!aligned16(workspace)) return TP_E_ALIGN;
  }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (dXi && dBi && dtype == TP_BF16) {   // both GEMMs in one launch (the library may share the CUs)
    GemmLaunch L = row_bwd_pair(M, N, K, dZ, lddz, Xi, ldx, Bi, ldb, dXi, lddx, dBi, lddb);
    give_split_ws(L, workspace, ws_bytes, colpart_bytes(M, N));   // past the bias-gradient partials
    if (run_gemm(dtype, L, s) != hipSuccess) return TP_E_HIP;
  } else if (dXi) {   // dX_i = dZ B_i^T: NT over K' = N
    GemmLaunch L = {};
    L.nprob = 1;
    L.p[0] = make_problem(M, K, tps::L_NT, tps::E_STORE);
    L.p[0].seg[0] = tps::Seg{dZ, Bi, lddz, ldb, N};
    L.p[0].c = dXi;
    L.p[0].ldc = lddx;
    if (run_gemm(dtype, L, s) != hipSuccess) return TP_E_HIP;
  }
  if (dBi && !(dXi && dtype == TP_BF16)) {   // dB_i = X_i^T dZ: TN over K' = M
    GemmLaunch L = {};
    L.nprob = 1;
    L.p[0] = make_problem(K, N, tps::L_TN, tps::E_STORE);
    L.p[0].seg[0] = tps::Seg{Xi, dZ, ldx, lddz, M};
    L.p[0].c = dBi;
    L.p[0].ldc = lddb;
    if (run_gemm(dtype, L, s) != hipSuccess) return TP_E_HIP;
  }
  if (dbias) {
    float* colpart = static_cast<float*>(workspace);
    const int64_t ldcp = round_up(N, 4);
    tps::ActBwdArgs a = {};
    a.M = M;
    a.N = N;
    a.act = tps::E_STORE;
    a.dY = dZ;
    a.lddy = lddz;
    a.colpart = colpart;
    a.ldcp = ldcp;
    if (tps::launch_act_bwd(dtype == TP_BF16, a, s) != hipSuccess) return TP_E_HIP;
    if (tps::launch_colsum_finalize(dtype == TP_BF16, colpart, colpart_rows(M), ldcp, N, 0, dbias, s) != hipSuccess)
      return TP_E_HIP;
  }
  return TP_OK;
}

int tp_row_bwd_plan(int64_t M, int64_t N, int64_t K, int cus) {
  if (bad_dim(M) || bad_dim(N) || bad_dim(K) || cus < 1) return -2;
  if (check_grid(TP_BF16, M, K) != TP_OK || check_grid(TP_BF16, K, N) != TP_OK) return -2;
  const GemmLaunch L = row_bwd_standin(M, N, K);
  int g0 = 0;
  int64_t t0 = 0, t1 = 0;
  return tps::dual_plan(L, cus, g0, t0, t1);
}

int tp_row_bwd_plan_split(int64_t M, int64_t N, int64_t K, int cus, size_t split_bytes, int* ks_dB, int* ks_dX) {
  if (ks_dB) *ks_dB = 1;
  if (ks_dX) *ks_dX = 1;
  if (bad_dim(M) || bad_dim(N) || bad_dim(K) || cus < 1) return -2;
  if (check_grid(TP_BF16, M, K) != TP_OK || check_grid(TP_BF16, K, N) != TP_OK) return -2;
  GemmLaunch L = row_bwd_standin(M, N, K);
  L.split_ws = split_bytes ? reinterpret_cast<float*>(uintptr_t(256)) : nullptr;
  L.split_bytes = split_bytes;
  int g0 = 0, k0 = 1, k1 = 1;
  int64_t t0 = 0, t1 = 0;
  size_t need = 0;
  const int plan = tps::dual_plan(L, cus, g0, t0, t1, k0, k1, need);
  if (ks_dB) *ks_dB = k0;
  if (ks_dX) *ks_dX = k1;
  return plan;
}

size_t tp_row_bwd_workspace_bytes_split(int dtype, int64_t M, int64_t N, int64_t K, int cus) {
  if (!valid_dtype(dtype) || bad_dim(M) || bad_dim(N) || bad_dim(K) || cus < 1) return 0;
  const size_t base = colpart_bytes(M, N);
  if (dtype != TP_BF16 || check_grid(TP_BF16, M, K) != TP_OK || check_grid(TP_BF16, K, N) != TP_OK) return base;
  return base + split_scratch(row_bwd_standin(M, N, K), cus);
}

size_t tp_column_bwd_workspace_bytes(int dtype, int act, int64_t M, int64_t N, int with_bias_grad) {
  if (!valid_dtype(dtype) || !valid_act(act) || bad_dim(M) || bad_dim(N)) return 0;
  size_t bytes = 0;
  if (act != TP_ACT_NONE) bytes += dp_bytes(dtype, M, N) * (act == TP_ACT_SWIGLU ? 2 : 1);
  if (with_bias_grad) bytes += colpart_bytes(M, N);
  return bytes;
}

size_t tp_column_bwd_workspace_bytes_split(int dtype, int act, int64_t M, int64_t N, int64_t K, int with_bias_grad,
                                           int cus) {
  const size_t base = tp_column_bwd_workspace_bytes(dtype, act, M, N, with_bias_grad);
  if (base == 0 && (!valid_dtype(dtype) || !valid_act(act) || bad_dim(M) || bad_dim(N))) return 0;
  if (bad_dim(K) || cus < 1) return 0;
  // only the activation-free bf16 backward runs its two GEMMs as one launch
  if (dtype != TP_BF16 || act != TP_ACT_NONE || check_grid(TP_BF16, M, K) != TP_OK ||
      check_grid(TP_BF16, K, N) != TP_OK)
    return base;
  // the same pair of products as the row backward's (dA = X^T dP beside dX = dP A^T)
  return base + split_scratch(row_bwd_standin(M, N, K), cus);
}

tp_status tp_column_bwd(int dtype, int act, int64_t M, int64_t N, int64_t K, const void* dY, int64_t lddy,
                        const void* X, int64_t ldx, const void* A, int64_t lda, const void* A2, int64_t lda2,
                        const void* Pre, int64_t ldpre, void* dXpart, int64_t lddx, void* dA, int64_t ldda,
                        void* dA2, int64_t ldda2, void* dbias, void* dbias2, void* workspace, size_t ws_bytes,
                        void* stream) {
  if (!valid_dtype(dtype)) return TP_E_DTYPE;
  if (!valid_act(act)) return TP_E_ACT;
  const bool swiglu = act == TP_ACT_SWIGLU;
  if (!dY || !X || !A) return TP_E_NULL;
  if (act != TP_ACT_NONE && !Pre) return TP_E_NULL;
  if (swiglu && !A2) return TP_E_NULL;
  if (swiglu && ((dA == nullptr) != (dA2 == nullptr))) return TP_E_NULL;
  if (bad_dim(M) || bad_dim(N) || bad_dim(K)) return TP_E_SHAPE;
  TPS_TRY(check_grid(dtype, M, K));
  TPS_TRY(check_grid(dtype, K, N));
  TPS_TRY(check_mat(dY, M, lddy, N, dtype));
  TPS_TRY(check_mat(X, M, ldx, K, dtype));
  TPS_TRY(check_mat(A, K, lda, N, dtype));
  if (swiglu) TPS_TRY(check_mat(A2, K, lda2, N, dtype));
  if (act != TP_ACT_NONE) TPS_TRY(check_mat(Pre, M, ldpre, swiglu ? 2 * N : N, dtype));
  if (dXpart) TPS_TRY(check_mat(dXpart, M, lddx, K, dtype));
  if (dA) TPS_TRY(check_mat(dA, K, ldda, N, dtype));
  if (swiglu && dA2) TPS_TRY(check_mat(dA2, K, ldda2, N, dtype));
  TPS_TRY(check_vec(dbias));
  if (swiglu) TPS_TRY(check_vec(dbias2));
  const bool want_bias = dbias || (swiglu && dbias2);
  if (dtype == TP_BF16 && act != TP_ACT_NONE && !bf16_extent_ok(M, round_up(N, 8), N)) return TP_E_SHAPE;
  const size_t need = tp_column_bwd_workspace_bytes(dtype, act, M, N, want_bias);
  if (need > 0) {
    if (!workspace || ws_bytes < need) return TP_E_WORKSPACE;
    if (!aligned16(workspace)) return TP_E_ALIGN;
  }
  if (!dXpart && !dA && !want_bias) return TP_OK;

  const hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const int64_t lddp = round_up(N, 8);
  const void* dPg = dY;     // act NONE: dP = dY
  const void* dPu = nullptr;
  int64_t ldp = lddy;
  size_t off = 0;
  tps::ActBwdArgs a = {};
  a.M = M;
  a.N = N;
  a.act = act == TP_ACT_NONE ? tps::E_STORE : act == TP_ACT_GELU ? tps::E_GELU : tps::E_SWIGLU;
  a.dY = dY;
  a.lddy = lddy;
  a.pre = Pre;
  a.ldpre = ldpre;
  if (act != TP_ACT_NONE) {
    a.dp = ws + off;
    off += dp_bytes(dtype, M, N);
    if (swiglu) {
      a.dp_up = ws + off;
      off += dp_bytes(dtype, M, N);
    }
    a.lddp = lddp;
    dPg = a.dp;
    dPu = a.dp_up;
    ldp = lddp;
  }
  float* colpart = nullptr;
  const int64_t ldcp = round_up(N, 4);
  if (want_bias) {
    colpart = reinterpret_cast<float*>(ws + off);
    a.colpart = colpart;
    a.ldcp = ldcp;
  }
  if (act != TP_ACT_NONE || want_bias) {
    if (tps::launch_act_bwd(dtype == TP_BF16, a, s) != hipSuccess) return TP_E_HIP;
  }
  if (want_bias) {
    if (dbias && tps::launch_colsum_finalize(dtype == TP_BF16, colpart, colpart_rows(M), ldcp, N, 0, dbias, s) !=
                     hipSuccess)
      return TP_E_HIP;
    if (swiglu && dbias2 &&
        tps::launch_colsum_finalize(dtype == TP_BF16, colpart, colpart_rows(M), ldcp, N, 1, dbias2, s) != hipSuccess)
      return TP_E_HIP;
  }
  if (dXpart && dA && !swiglu && dtype == TP_BF16) {
    // dA = X^T dP (TN) and dX_part = dP A^T (NT) in one launch: the library
    // may run them side by side (few long weight-gradient tiles beside many
    // short input-gradient ones), as for the row-parallel backward.
    GemmLaunch L = {};
    L.nprob = 2;
    L.p[0] = make_problem(K, N, tps::L_TN, tps::E_STORE);
    L.p[0].seg[0] = tps::Seg{X, dPg, ldx, ldp, M};
    L.p[0].c = dA;
    L.p[0].ldc = ldda;
    L.p[1] = make_problem(M, K, tps::L_NT, tps::E_STORE);
    L.p[1].seg[0] = tps::Seg{dPg, A, ldp, lda, N};
    L.p[1].c = dXpart;
    L.p[1].ldc = lddx;
    give_split_ws(L, workspace, ws_bytes, need);   // past the bias-gradient partials
    if (run_gemm(dtype, L, s) != hipSuccess) return TP_E_HIP;
    return TP_OK;
  }
  if (dXpart) {   // dX_part = dP_g A^T (+ dP_u A2^T): NT over K' = N per segment
    GemmLaunch L = {};
    L.nprob = 1;
    L.p[0] = make_problem(M, K, tps::L_NT, tps::E_STORE);
    L.p[0].seg[0] = tps::Seg{dPg, A, ldp, lda, N};
    if (swiglu) {
      L.p[0].seg[1] = tps::Seg{dPu, A2, ldp, lda2, N};
      L.p[0].nseg = 2;
    }
    L.p[0].c = dXpart;
    L.p[0].ldc = lddx;
    if (run_gemm(dtype, L, s) != hipSuccess) return TP_E_HIP;
  }
  if (dA) {   // dA = X^T dP_g, dA2 = X^T dP_u: TN over K' = M, one launch
    GemmLaunch L = {};
    L.nprob = swiglu ? 2 : 1;
    L.p[0] = make_problem(K, N, tps::L_TN, tps::E_STORE);
    L.p[0].seg[0] = tps::Seg{X, dPg, ldx, ldp, M};
    L.p[0].c = dA;
    L.p[0].ldc = ldda;
    if (swiglu) {
      L.p[1] = make_problem(K, N, tps::L_TN, tps::E_STORE);
      L.p[1].seg[0] = tps::Seg{X, dPu, ldx, ldp, M};
      L.p[1].c = dA2;
      L.p[1].ldc = ldda2;
    }
    if (run_gemm(dtype, L, s) != hipSuccess) return TP_E_HIP;
  }
  return TP_OK;
}

size_t tp_vocab_ce_workspace_bytes(int64_t M, int64_t Vr) {
  if (bad_dim(M) || bad_dim(Vr)) return 0;
  return tps::ce_workspace_bytes(M, Vr);
}

tp_status tp_vocab_ce_partials(int dtype, int64_t M, int64_t Vr, int64_t K, const void* H, int64_t ldh,
                               const void* W, int64_t ldw, const int32_t* target, int64_t v0, float* out_max,
                               float* out_sumexp, float* out_tgt, void* workspace, size_t ws_bytes, void* stream) {
  if (dtype != TP_BF16) return TP_E_DTYPE;
  if (!H || !W || !target || !out_max || !out_sumexp || !out_tgt) return TP_E_NULL;
  if (bad_dim(M) || bad_dim(Vr) || bad_dim(K)) return TP_E_SHAPE;
  TPS_TRY(check_grid(dtype, M, Vr));
  TPS_TRY(check_mat(H, M, ldh, K, dtype));
  TPS_TRY(check_mat(W, Vr, ldw, K, dtype));
  if (!aligned16(target) || !aligned16(out_max) || !aligned16(out_sumexp) || !aligned16(out_tgt)) return TP_E_ALIGN;
  if (!workspace || ws_bytes < tp_vocab_ce_workspace_bytes(M, Vr)) return TP_E_WORKSPACE;
  if (!aligned16(workspace)) return TP_E_ALIGN;
  tps::CEArgs a = {M, Vr, K, H, ldh, W, ldw, target, v0, out_max, out_sumexp, out_tgt, static_cast<float*>(workspace)};
  return tps::launch_ce_partials(a, static_cast<hipStream_t>(stream)) == hipSuccess ? TP_OK : TP_E_HIP;
}

tp_status tp_vocab_ce_combine(int R, int64_t M, const float* maxes, const float* sumexps, const float* tgts,
                              int64_t stride, float* lse, float* tgt, float* loss, void* stream) {
  if (!maxes || !sumexps || !tgts) return TP_E_NULL;
  if (!lse && !tgt && !loss) return TP_E_NULL;
  if (R < 1 || bad_dim(M) || stride < M || (R > 1 && stride > kMaxDim / R)) return TP_E_SHAPE;
  if (stride % 4 != 0 || !aligned16(maxes) || !aligned16(sumexps) || !aligned16(tgts)) return TP_E_ALIGN;
  TPS_TRY(check_vec(lse));
  TPS_TRY(check_vec(tgt));
  TPS_TRY(check_vec(loss));
  const tps::CECombineArgs a = {R, M, stride, maxes, sumexps, tgts, lse, tgt, loss};
  return tps::launch_ce_combine(a, static_cast<hipStream_t>(stream)) == hipSuccess ? TP_OK : TP_E_HIP;
}

tp_status tp_vocab_ce_partials_noalloc(int dtype, int64_t M, int64_t Vr, int64_t K, const void* H, int64_t ldh,
                                       const void* W, int64_t ldw, const int32_t* target, int64_t v0, float* out_max,
                                       float* out_sumexp, float* out_tgt, void* stream) {
  static_assert(TP_CE_NOALLOC_SCRATCH_BYTES == tps::kCeScratchBytes, "header and library agree on the scratch size");
  if (dtype != TP_BF16) return TP_E_DTYPE;
  if (!H || !W || !target || !out_max || !out_sumexp || !out_tgt) return TP_E_NULL;
  if (bad_dim(M) || bad_dim(Vr) || bad_dim(K)) return TP_E_SHAPE;
  TPS_TRY(check_grid(dtype, M, Vr));
  TPS_TRY(check_mat(H, M, ldh, K, dtype));
  TPS_TRY(check_mat(W, Vr, ldw, K, dtype));
  if (!aligned16(target) || !aligned16(out_max) || !aligned16(out_sumexp) || !aligned16(out_tgt)) return TP_E_ALIGN;
  if (tps::ce_workspace_bytes(M, Vr) > tps::kCeScratchBytes) return TP_E_WORKSPACE;
  float* ws = nullptr;
  if (tps::ce_scratch(&ws) != hipSuccess) return TP_E_HIP;
  tps::CEArgs a = {M, Vr, K, H, ldh, W, ldw, target, v0, out_max, out_sumexp, out_tgt, ws};
  return tps::launch_ce_partials(a, static_cast<hipStream_t>(stream)) == hipSuccess ? TP_OK : TP_E_HIP;
}

size_t tp_vocab_ce_bwd_workspace_bytes(int64_t M, int64_t Vr) {
  if (bad_dim(M) || bad_dim(Vr)) return 0;
  return align_ws((size_t)M * (size_t)round_up(Vr, 8) * 2);
}

tp_status tp_vocab_ce_bwd(int dtype, int64_t M, int64_t Vr, int64_t K, const void* H, int64_t ldh, const void* W,
                          int64_t ldw, const int32_t* target, int64_t v0, const float* lse, const float* gscale,
                          void* dH, int64_t lddh, void* dW, int64_t lddw, void* workspace, size_t ws_bytes,
                          void* stream) {
  if (dtype != TP_BF16) return TP_E_DTYPE;
  if (!H || !W || !target || !lse) return TP_E_NULL;
  if (bad_dim(M) || bad_dim(Vr) || bad_dim(K)) return TP_E_SHAPE;
  TPS_TRY(check_grid(dtype, M, Vr));
  TPS_TRY(check_grid(dtype, M, K));
  TPS_TRY(check_grid(dtype, Vr, K));
  TPS_TRY(check_mat(H, M, ldh, K, dtype));
  TPS_TRY(check_mat(W, Vr, ldw, K, dtype));
  if (dH) TPS_TRY(check_mat(dH, M, lddh, K, dtype));
  if (dW) TPS_TRY(check_mat(dW, Vr, lddw, K, dtype));
  const int64_t lddz = round_up(Vr, 8);
  if (!bf16_extent_ok(M, lddz, Vr)) return TP_E_SHAPE;
  if (!aligned16(target) || !aligned16(lse) || (gscale && !aligned16(gscale))) return TP_E_ALIGN;
  if (!dH && !dW) return TP_OK;
  if (!workspace || ws_bytes < tp_vocab_ce_bwd_workspace_bytes(M, Vr)) return TP_E_WORKSPACE;
  if (!aligned16(workspace)) return TP_E_ALIGN;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  void* dz = workspace;
  {   // dz = gscale * (softmax(z) - onehot), z = H W^T: NT with the CE-gradient epilogue
    GemmLaunch L = {};
    L.nprob = 1;
    L.p[0] = make_problem(M, Vr, tps::L_NT, tps::E_CE_GRAD);
    L.p[0].seg[0] = tps::Seg{H, W, ldh, ldw, K};
    L.p[0].c = dz;
    L.p[0].ldc = lddz;
    L.p[0].lse = lse;
    L.p[0].gscale = gscale;
    L.p[0].target = target;
    L.p[0].v0 = v0;
    if (tps::launch_gemm_bf16(L, s) != hipSuccess) return TP_E_HIP;
  }
  if (dH) {   // dH = dz W: NN over K' = Vr
    GemmLaunch L = {};
    L.nprob = 1;
    L.p[0] = make_problem(M, K, tps::L_NN, tps::E_STORE);
    L.p[0].seg[0] = tps::Seg{dz, W, lddz, ldw, Vr};
    L.p[0].c = dH;
    L.p[0].ldc = lddh;
    if (tps::launch_gemm_bf16(L, s) != hipSuccess) return TP_E_HIP;
  }
  if (dW) {   // dW = dz^T H: TN over K' = M
    GemmLaunch L = {};
    L.nprob = 1;
    L.p[0] = make_problem(Vr, K, tps::L_TN, tps::E_STORE);
    L.p[0].seg[0] = tps::Seg{dz, H, lddz, ldh, M};
    L.p[0].c = dW;
    L.p[0].ldc = lddw;
    if (tps::launch_gemm_bf16(L, s) != hipSuccess) return TP_E_HIP;
  }
  return TP_OK;
}

// ---------------------------------------------------------------------------
// Vocab-parallel embedding.
// ---------------------------------------------------------------------------

tp_status tp_vocab_embed_fwd(int dtype, int64_t M, int64_t Vr, int64_t K, const int32_t* ids, int64_t v0,
                             const void* E, int64_t lde, void* out, int64_t ldo, void* stream) {
  if (!valid_dtype(dtype)) return TP_E_DTYPE;
  if (!ids || !E || !out) return TP_E_NULL;
  if (bad_dim(M) || bad_dim(Vr) || bad_dim(K)) return TP_E_SHAPE;
  TPS_TRY(check_mat(E, Vr, lde, K, dtype));
  TPS_TRY(check_mat(out, M, ldo, K, dtype));
  if (!aligned16(ids)) return TP_E_ALIGN;
  const tps::EmbArgs a = {M, Vr, K, ids, v0, E, lde, out, ldo};
  return tps::launch_emb_fwd(dtype == TP_BF16, a, static_cast<hipStream_t>(stream)) == hipSuccess ? TP_OK
                                                                                                : TP_E_HIP;
}

size_t tp_vocab_embed_bwd_workspace_bytes(int64_t M, int64_t Vr) {
  if (bad_dim(M) || bad_dim(Vr)) return 0;
  // row starts [Vr + 1] and token order [M]: int32 each
  return align_ws((size_t)(Vr + 1) * 4) + align_ws((size_t)M * 4);
}

tp_status tp_vocab_embed_bwd(int dtype, int64_t M, int64_t Vr, int64_t K, const int32_t* ids, int64_t v0,
                             const void* dout, int64_t lddo, void* dE, int64_t ldde, void* workspace,
                             size_t ws_bytes, void* stream) {
  if (!valid_dtype(dtype)) return TP_E_DTYPE;
  if (!ids || !dout || !dE) return TP_E_NULL;
  if (bad_dim(M) || bad_dim(Vr) || bad_dim(K)) return TP_E_SHAPE;
  TPS_TRY(check_mat(dout, M, lddo, K, dtype));
  TPS_TRY(check_mat(dE, Vr, ldde, K, dtype));
  if (!aligned16(ids)) return TP_E_ALIGN;
  if (!workspace || ws_bytes < tp_vocab_embed_bwd_workspace_bytes(M, Vr)) return TP_E_WORKSPACE;
  if (!aligned16(workspace)) return TP_E_ALIGN;
  char* w = static_cast<char*>(workspace);
  int32_t* start = reinterpret_cast<int32_t*>(w);
  int32_t* order = reinterpret_cast<int32_t*>(w + align_ws((size_t)(Vr + 1) * 4));
  const tps::EmbArgs a = {M, Vr, K, ids, v0, dout, lddo, dE, ldde};
  const hipError_t e = tps::launch_emb_bwd(dtype == TP_BF16, a, start, order, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TP_OK : TP_E_HIP;
}

// ---------------------------------------------------------------------------
// Attention core.
// ---------------------------------------------------------------------------

namespace {
// Head layout shared by the attention entry points; fills the common fields.
tp_status attn_check(int dtype, int64_t B, int64_t S, int n_q, int n_kv, int head_dim, int causal, float scale,
                     const void* Q, int64_t ldq, const void* K, int64_t ldk, const void* V, int64_t ldv,
                     tps::AttnArgs& a) {
  if (dtype != TP_BF16) return TP_E_DTYPE;
  if (!Q || !K || !V) return TP_E_NULL;
  if (head_dim != 128 || bad_dim(B) || B > 65535 || bad_dim(S) || bad_dim(B * S) || B * S > kMaxDim) return TP_E_SHAPE;
  if (n_q < 1 || n_kv < 1 || n_q > 65535 || n_q % n_kv != 0) return TP_E_SHAPE;
  const int group = n_q / n_kv;
  if (!(group % 4 == 0 || 4 % group == 0)) return TP_E_SHAPE;
  if (causal != 0 && causal != 1) return TP_E_SHAPE;
  if (!(scale > 0.f) || !(scale <= 3.4e38f)) return TP_E_SHAPE;
  TPS_TRY(check_mat(Q, B * S, ldq, (int64_t)n_q * head_dim, dtype));
  TPS_TRY(check_mat(K, B * S, ldk, (int64_t)n_kv * head_dim, dtype));
  TPS_TRY(check_mat(V, B * S, ldv, (int64_t)n_kv * head_dim, dtype));
  a = tps::AttnArgs{};
  a.B = B;
  a.S = S;
  a.n_q = n_q;
  a.n_kv = n_kv;
  a.causal = causal;
  a.scale = scale;
  a.q = Q;
  a.ldq = ldq;
  a.k = K;
  a.ldk = ldk;
  a.v = V;
  a.ldv = ldv;
  return TP_OK;
}
}  // namespace

size_t tp_attention_fwd_workspace_bytes(int64_t B, int64_t S, int n_q, int n_kv, int causal) {
  if (bad_dim(B) || bad_dim(S) || n_q < 1 || n_kv < 1 || n_q % n_kv != 0) return 0;
  const int group = n_q / n_kv;
  if (!(group % 4 == 0 || 4 % group == 0)) return 0;
  return align_ws(tps::attn_fwd_workspace_bytes(B, S, n_q, n_kv, causal != 0));
}

tp_status tp_attention_fwd(int dtype, int64_t B, int64_t S, int n_q, int n_kv, int head_dim, int causal, float scale,
                           const void* Q, int64_t ldq, const void* K, int64_t ldk, const void* V, int64_t ldv,
                           void* O, int64_t ldo, float* lse, void* workspace, size_t ws_bytes, void* stream) {
  tps::AttnArgs a;
  TPS_TRY(attn_check(dtype, B, S, n_q, n_kv, head_dim, causal, scale, Q, ldq, K, ldk, V, ldv, a));
  if (!O || !lse) return TP_E_NULL;
  TPS_TRY(check_mat(O, B * S, ldo, (int64_t)n_q * head_dim, dtype));
  if (!aligned16(lse)) return TP_E_ALIGN;
  const size_t need = tp_attention_fwd_workspace_bytes(B, S, n_q, n_kv, causal);
  if (need > 0 && (!workspace || ws_bytes < need)) return TP_E_WORKSPACE;
  if (need > 0 && !aligned16(workspace)) return TP_E_ALIGN;
  a.o = O;
  a.ldo = ldo;
  a.lse = lse;
  tps::attn_chunking(B, S, n_q, n_kv, causal, a.chunk_tiles, a.max_chunks);
  a.ws = static_cast<float*>(workspace);
  return tps::launch_attn_fwd(a, static_cast<hipStream_t>(stream)) == hipSuccess ? TP_OK : TP_E_HIP;
}

size_t tp_attention_bwd_workspace_bytes(int64_t B, int64_t S, int n_q, int n_kv, int causal) {
  if (bad_dim(B) || bad_dim(S) || n_q < 1 || n_kv < 1 || n_q % n_kv != 0) return 0;
  const int group = n_q / n_kv;
  if (!(group % 4 == 0 || 4 % group == 0)) return 0;
  tps::AttnBwdLayout L;
  tps::attn_bwd_layout(B, S, n_q, n_kv, causal != 0, L);
  return L.ld_bytes + L.dq_bytes + L.kv_bytes;
}

tp_status tp_attention_bwd(int dtype, int64_t B, int64_t S, int n_q, int n_kv, int head_dim, int causal, float scale,
                           const void* Q, int64_t ldq, const void* K, int64_t ldk, const void* V, int64_t ldv,
                           const void* O, int64_t ldo, const float* lse, const void* dO, int64_t lddo, void* dQ,
                           int64_t lddq, void* dK, int64_t lddk, void* dV, int64_t lddv, void* workspace,
                           size_t ws_bytes, void* stream) {
  tps::AttnBwdArgs p = {};
  TPS_TRY(attn_check(dtype, B, S, n_q, n_kv, head_dim, causal, scale, Q, ldq, K, ldk, V, ldv, p.f));
  if (!O || !lse || !dO || !dQ || !dK || !dV) return TP_E_NULL;
  const int64_t rows = B * S, wq = (int64_t)n_q * head_dim, wkv = (int64_t)n_kv * head_dim;
  TPS_TRY(check_mat(O, rows, ldo, wq, dtype));
  TPS_TRY(check_mat(dO, rows, lddo, wq, dtype));
  TPS_TRY(check_mat(dQ, rows, lddq, wq, dtype));
  TPS_TRY(check_mat(dK, rows, lddk, wkv, dtype));
  TPS_TRY(check_mat(dV, rows, lddv, wkv, dtype));
  if (!aligned16(lse)) return TP_E_ALIGN;
  const size_t need = tp_attention_bwd_workspace_bytes(B, S, n_q, n_kv, causal);
  if (!workspace || ws_bytes < need) return TP_E_WORKSPACE;
  if (!aligned16(workspace)) return TP_E_ALIGN;
  tps::AttnBwdLayout L;
  tps::attn_bwd_layout(B, S, n_q, n_kv, causal, L);
  char* w = static_cast<char*>(workspace);
  p.f.o = const_cast<void*>(O);
  p.f.ldo = ldo;
  p.f.lse = const_cast<float*>(lse);
  p.f.chunk_tiles = L.chunk_tiles;
  p.f.max_chunks = L.max_chunks;
  p.dout = dO;
  p.ldg = lddo;
  p.dq = dQ;
  p.lddq = lddq;
  p.dk = dK;
  p.lddk = lddk;
  p.dv = dV;
  p.lddv = lddv;
  p.ld = reinterpret_cast<float*>(w);
  p.dq_ws = reinterpret_cast<float*>(w + L.ld_bytes);
  p.kv_ws = reinterpret_cast<float*>(w + L.ld_bytes + L.dq_bytes);
  p.kv_chunk_tiles = L.kv_chunk_tiles;
  p.kv_max_chunks = L.kv_max_chunks;
  return tps::launch_attn_bwd(p, static_cast<hipStream_t>(stream)) == hipSuccess ? TP_OK : TP_E_HIP;
}

}  // extern "C"
