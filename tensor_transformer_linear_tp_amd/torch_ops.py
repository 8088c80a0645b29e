"""torch-tensor front end of the libtpshard binding.

Argument marshalling only: shapes and leading dimensions are read from the
tensors, outputs and workspaces are allocated with ``torch.empty`` on the
inputs' device (padded so every leading dimension meets the library's
alignment rule), and the call goes to the C ABI on torch's current stream.
No arithmetic of the method happens here.
"""
from __future__ import annotations

import torch

from . import (TP_ACT_GELU, TP_ACT_NONE, TP_ACT_SWIGLU, TP_BF16, TP_FP32, tp_column_bwd,
               tp_column_bwd_workspace_bytes, tp_column_bwd_workspace_bytes_split, tp_column_fwd, tp_row_bwd,
               tp_row_bwd_workspace_bytes, tp_row_bwd_workspace_bytes_split, tp_row_fwd,
               tp_sp_reduce_scatter_ln, tp_sum_partials, tp_vocab_ce_bwd, tp_vocab_embed_bwd,
               tp_vocab_embed_bwd_workspace_bytes, tp_vocab_embed_fwd, tp_attention_fwd,
               tp_attention_fwd_workspace_bytes, tp_attention_bwd, tp_attention_bwd_workspace_bytes, tp_vocab_ce_bwd_workspace_bytes, tp_vocab_ce_combine, tp_vocab_ce_partials,
               tp_vocab_ce_workspace_bytes)

ACTS = {"none": TP_ACT_NONE, "gelu": TP_ACT_GELU, "swiglu": TP_ACT_SWIGLU}


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return TP_BF16
    if t.dtype == torch.float32:
        return TP_FP32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _vec(dtype: torch.dtype) -> int:
    return 8 if dtype == torch.bfloat16 else 4


def empty_padded(rows: int, cols: int, dtype, device) -> torch.Tensor:
    """[rows, cols] view of a buffer whose row stride is a multiple of the vector width."""
    v = _vec(dtype)
    ld = (cols + v - 1) // v * v
    return torch.empty(rows, ld, dtype=dtype, device=device)[:, :cols]


def aligned(t: torch.Tensor) -> torch.Tensor:
    """Return ``t`` if it already satisfies the ABI layout rule, else a padded copy."""
    if t is None:
        return None
    if t.dim() == 1:
        return t if (t.is_contiguous() and t.data_ptr() % 16 == 0) else t.clone()
    v = _vec(t.dtype)
    if t.stride(1) == 1 and t.stride(0) % v == 0 and t.data_ptr() % 16 == 0 and t.stride(0) >= t.shape[1]:
        return t
    out = empty_padded(t.shape[0], t.shape[1], t.dtype, t.device)
    out.copy_(t)
    return out


def ld(t: torch.Tensor) -> int:
    return t.stride(0)


def column_fwd(X, A, act="none", A2=None, bias=None, bias2=None):
    """Y = act(X A + b) (SwiGLU: silu(X A + b) * (X A2 + b2)); returns (Y, Pre)."""
    X, A, A2, bias, bias2 = (aligned(t) for t in (X, A, A2, bias, bias2))
    M, K = X.shape
    N = A.shape[1]
    Y = empty_padded(M, N, X.dtype, X.device)
    Pre = None
    if act == "gelu":
        Pre = empty_padded(M, N, X.dtype, X.device)
    elif act == "swiglu":
        Pre = empty_padded(M, 2 * N, X.dtype, X.device)
    tp_column_fwd(dtype_code(X), ACTS[act], M, N, K, X, ld(X), A, ld(A), A2, ld(A2) if A2 is not None else 0,
                  bias, bias2, Y, ld(Y), Pre, ld(Pre) if Pre is not None else 0)
    return Y, Pre


def row_fwd(Xi, Bi):
    """Full-shape partial Z_i = X_i B_i."""
    Xi, Bi = aligned(Xi), aligned(Bi)
    M, K = Xi.shape
    N = Bi.shape[1]
    Z = empty_padded(M, N, Xi.dtype, Xi.device)
    tp_row_fwd(dtype_code(Xi), M, N, K, Xi, ld(Xi), Bi, ld(Bi), Z, ld(Z))
    return Z


def stack_partials(parts):
    """Copy a list of [M, N] partials into one padded [t, M, ld] buffer."""
    t = len(parts)
    M, N = parts[0].shape
    v = _vec(parts[0].dtype)
    ldp = (N + v - 1) // v * v
    buf = torch.empty(t, M, ldp, dtype=parts[0].dtype, device=parts[0].device)
    for i, p in enumerate(parts):
        buf[i, :, :N].copy_(p)
    return buf, N


def sum_partials(buf, N, bias=None, out=None):
    """out = sum_i buf[i, :, :N] (+ bias once); ``buf`` is a [t, M, ld] tensor."""
    t, M, ldp = buf.shape
    bias = aligned(bias)
    if out is None:
        out = empty_padded(M, N, buf.dtype, buf.device)
    tp_sum_partials(dtype_code(buf), t, M, N, buf, ldp, M * ldp, bias, out, ld(out))
    return out


def sp_reduce_scatter_ln(buf, N, r0, Mr, bias=None, resid=None, gamma=None, beta=None, eps=1e-5, want_h=True,
                         h_inplace=False):
    """Rank rows [r0, r0+Mr) of sum_i buf[i] + bias + resid, then LayerNorm; returns (y, h).

    ``buf`` is a [t, M, ld] tensor of partials; ``resid`` is the rank's [Mr, N] block.  With
    ``h_inplace`` the residual stream h overwrites ``resid`` (which must then satisfy the layout rule).
    """
    t, M, ldp = buf.shape
    bias, gamma, beta = aligned(bias), aligned(gamma), aligned(beta)
    if not h_inplace:
        resid = aligned(resid)
    y = empty_padded(Mr, N, buf.dtype, buf.device)
    if h_inplace:
        h = resid
    else:
        h = empty_padded(Mr, N, buf.dtype, buf.device) if want_h else None
    tp_sp_reduce_scatter_ln(dtype_code(buf), t, M, N, buf, ldp, M * ldp, r0, Mr, bias, resid,
                            ld(resid) if resid is not None else 0, gamma, beta, eps, y, ld(y), h,
                            ld(h) if h is not None else 0)
    return y, h


def _cus(device):
    return torch.cuda.get_device_properties(device).multi_processor_count


def row_bwd(dZ, Xi, Bi, want_dx=True, want_dw=True, want_db=False, split=False):
    """(dX_i, dB_i, dbias) of the row shard; unrequested outputs are None.  split: give the call
    the workspace its split-contraction schedule takes (tp_row_bwd_workspace_bytes_split)."""
    dZ, Xi, Bi = aligned(dZ), aligned(Xi), aligned(Bi)
    M, N = dZ.shape
    K = Xi.shape[1]
    dt = dtype_code(dZ)
    dX = empty_padded(M, K, dZ.dtype, dZ.device) if want_dx else None
    dB = empty_padded(K, N, dZ.dtype, dZ.device) if want_dw else None
    db = torch.empty(N, dtype=dZ.dtype, device=dZ.device) if want_db else None
    if split:
        ws_n = tp_row_bwd_workspace_bytes_split(dt, M, N, K, _cus(dZ.device))
    else:
        ws_n = tp_row_bwd_workspace_bytes(dt, M, N) if want_db else 0
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=dZ.device) if (want_db or split) else None
    tp_row_bwd(dt, M, N, K, dZ, ld(dZ), Xi, ld(Xi), Bi, ld(Bi), dX, ld(dX) if dX is not None else 0,
               dB, ld(dB) if dB is not None else 0, db, ws, ws_n)
    return dX, dB, db


def column_bwd(dY, X, A, Pre=None, act="none", A2=None, want_dx=True, want_dw=True, want_db=False, split=False):
    """(dX_part, dA, dA2, dbias, dbias2) of the column shard; unrequested outputs are None.  split: the
    workspace of the split-contraction schedule (tp_column_bwd_workspace_bytes_split)."""
    dY, X, A, A2, Pre = (aligned(t) for t in (dY, X, A, A2, Pre))
    M, N = dY.shape
    K = X.shape[1]
    dt = dtype_code(dY)
    sw = act == "swiglu"
    dX = empty_padded(M, K, dY.dtype, dY.device) if want_dx else None
    dA = empty_padded(K, N, dY.dtype, dY.device) if want_dw else None
    dA2 = empty_padded(K, N, dY.dtype, dY.device) if (want_dw and sw) else None
    db = torch.empty(N, dtype=dY.dtype, device=dY.device) if want_db else None
    db2 = torch.empty(N, dtype=dY.dtype, device=dY.device) if (want_db and sw) else None
    if split:
        ws_n = tp_column_bwd_workspace_bytes_split(dt, ACTS[act], M, N, K, want_db, _cus(dY.device))
    else:
        ws_n = tp_column_bwd_workspace_bytes(dt, ACTS[act], M, N, want_db)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=dY.device)
    tp_column_bwd(dt, ACTS[act], M, N, K, dY, ld(dY), X, ld(X), A, ld(A), A2, ld(A2) if A2 is not None else 0,
                  Pre, ld(Pre) if Pre is not None else 0, dX, ld(dX) if dX is not None else 0,
                  dA, ld(dA) if dA is not None else 0, dA2, ld(dA2) if dA2 is not None else 0,
                  db, db2, ws, ws_n)
    return dX, dA, dA2, db, db2


def vocab_ce_partials(H, W, target, v0):
    """Per-token (max, sum exp(z - max), target logit) over the vocab shard starting at v0."""
    H, W = aligned(H), aligned(W)
    M, K = H.shape
    Vr = W.shape[0]
    target = target.to(torch.int32).contiguous()
    m = torch.empty(M, dtype=torch.float32, device=H.device)
    s = torch.empty(M, dtype=torch.float32, device=H.device)
    tg = torch.empty(M, dtype=torch.float32, device=H.device)
    ws_n = tp_vocab_ce_workspace_bytes(M, Vr)
    ws = torch.empty(ws_n, dtype=torch.uint8, device=H.device)
    tp_vocab_ce_partials(TP_BF16, M, Vr, K, H, ld(H), W, ld(W), target, v0, m, s, tg, ws, ws_n)
    return m, s, tg


def _rows_f32(x):
    """[R, M] fp32 device tensor whose row stride is a multiple of 4 (stacks a list of [M] tensors)."""
    if isinstance(x, (list, tuple)):
        x = torch.stack([v.to(torch.float32) for v in x])
    x = x.to(torch.float32)
    if x.dim() == 1:
        x = x[None, :]
    if x.stride(1) != 1 or x.stride(0) % 4 or x.data_ptr() % 16 or x.stride(0) < x.shape[1]:
        buf = torch.empty(x.shape[0], (x.shape[1] + 3) // 4 * 4, dtype=torch.float32, device=x.device)
        buf[:, :x.shape[1]].copy_(x)
        x = buf[:, :x.shape[1]]
    return x


def vocab_ce_combine(maxes, sumexps, tgts):
    """Recombine R shards' CE partials ([R, M] each, or lists of [M]); returns (lse, tgt, loss) fp32 [M]."""
    ms, ss, ts = _rows_f32(maxes), _rows_f32(sumexps), _rows_f32(tgts)
    if not (ms.shape == ss.shape == ts.shape):
        raise ValueError("the three partial arrays must have the same shape")
    if not (ms.stride(0) == ss.stride(0) == ts.stride(0)):
        ms, ss, ts = (_rows_f32(v.clone()) for v in (ms, ss, ts))
    R, M = ms.shape
    out = [torch.empty(M, dtype=torch.float32, device=ms.device) for _ in range(3)]
    tp_vocab_ce_combine(R, M, ms, ss, ts, ms.stride(0), *out)
    return tuple(out)


def vocab_ce_bwd(H, W, target, v0, lse, gscale=None, want_dh=True, want_dw=True):
    """(dH partial, dW) of the CE loss for the vocab shard starting at v0, given the recombined lse."""
    H, W = aligned(H), aligned(W)
    M, K = H.shape
    Vr = W.shape[0]
    target = target.to(torch.int32).contiguous()
    lse = lse.to(torch.float32).contiguous()
    if gscale is not None:
        gscale = gscale.to(torch.float32).contiguous()
    dH = empty_padded(M, K, H.dtype, H.device) if want_dh else None
    dW = empty_padded(Vr, K, H.dtype, H.device) if want_dw else None
    ws_n = tp_vocab_ce_bwd_workspace_bytes(M, Vr)
    ws = torch.empty(ws_n, dtype=torch.uint8, device=H.device)
    tp_vocab_ce_bwd(TP_BF16, M, Vr, K, H, ld(H), W, ld(W), target, v0, lse, gscale, dH,
                    ld(dH) if dH is not None else 0, dW, ld(dW) if dW is not None else 0, ws, ws_n)
    return dH, dW


__all__ = ["column_fwd", "row_fwd", "stack_partials", "sum_partials", "row_bwd", "column_bwd", "vocab_ce_combine",
           "vocab_ce_partials", "vocab_ce_bwd", "empty_padded", "aligned", "dtype_code", "TP_FP32", "TP_BF16"]


def _ids(ids: torch.Tensor) -> torch.Tensor:
    if ids.dtype != torch.int32:
        raise TypeError("token ids must be int32")
    return ids if (ids.is_contiguous() and ids.data_ptr() % 16 == 0) else ids.clone()


def vocab_embed_fwd(ids, E, v0):
    """Rows of the rank's table block E [Vr, K] for owned ids, zero rows otherwise; returns [M, K]."""
    ids, E = _ids(ids), aligned(E)
    M, (Vr, K) = ids.shape[0], E.shape
    out = empty_padded(M, K, E.dtype, E.device)
    tp_vocab_embed_fwd(dtype_code(E), M, Vr, K, ids, v0, E, ld(E), out, ld(out))
    return out


def vocab_embed_bwd(ids, dout, v0, Vr):
    """Gradient of the rank's table block [Vr, K] from dout [M, K]."""
    ids, dout = _ids(ids), aligned(dout)
    M, K = dout.shape
    dE = empty_padded(Vr, K, dout.dtype, dout.device)
    n = tp_vocab_embed_bwd_workspace_bytes(M, Vr)
    ws = torch.empty(n, dtype=torch.uint8, device=dout.device)
    tp_vocab_embed_bwd(dtype_code(dout), M, Vr, K, ids, v0, dout, ld(dout), dE, ld(dE), ws, n)
    return dE


def attention_fwd(q, k, v, n_q, n_kv, causal=True, scale=None, B=1):
    """Attention core on views q [B S, 128 n_q], k / v [B S, 128 n_kv] (views of a packed QKV are
    passed as they are); returns (O [B S, 128 n_q], lse [B, n_q, S] fp32)."""
    rows = q.shape[0]
    S = rows // B
    scale = 1.0 / 128 ** 0.5 if scale is None else scale
    o = empty_padded(rows, 128 * n_q, q.dtype, q.device)
    lse = torch.empty(B, n_q, S, dtype=torch.float32, device=q.device)
    n = tp_attention_fwd_workspace_bytes(B, S, n_q, n_kv, causal)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)
    tp_attention_fwd(dtype_code(q), B, S, n_q, n_kv, 128, causal, scale, q, ld(q), k, ld(k), v, ld(v), o, ld(o), lse,
                     ws, n)
    return o, lse


def attention_bwd(q, k, v, o, lse, do, n_q, n_kv, causal=True, scale=None, B=1):
    """Gradients (dQ, dK, dV) of attention_fwd from its outputs o, lse and the output gradient do."""
    rows = q.shape[0]
    S = rows // B
    scale = 1.0 / 128 ** 0.5 if scale is None else scale
    do = aligned(do)
    dq = empty_padded(rows, 128 * n_q, q.dtype, q.device)
    dk = empty_padded(rows, 128 * n_kv, q.dtype, q.device)
    dv = empty_padded(rows, 128 * n_kv, q.dtype, q.device)
    n = tp_attention_bwd_workspace_bytes(B, S, n_q, n_kv, causal)
    ws = torch.empty(n, dtype=torch.uint8, device=q.device)
    tp_attention_bwd(dtype_code(q), B, S, n_q, n_kv, 128, causal, scale, q, ld(q), k, ld(k), v, ld(v), o, ld(o), lse,
                     do, ld(do), dq, ld(dq), dk, ld(dk), dv, ld(dv), ws, n)
    return dq, dk, dv
