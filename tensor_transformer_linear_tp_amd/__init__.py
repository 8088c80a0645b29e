"""Python binding of libtpshard: one tensor-parallel rank's share of a
transformer block on an MI355X (gfx950) GPU.

This module only marshals arguments to the C ABI declared in
``include/tpshard.h`` (same function names, same argument order); every step
of the computation runs in the library's HIP kernels.  Pointer arguments
accept an int (device address), None (NULL) or any object with
``data_ptr()`` (e.g. a torch tensor).  ``stream`` accepts an int hipStream_t,
an object with ``cuda_stream`` (a torch stream), or None for torch's current
stream (the null stream when torch is not imported).

A non-OK status raises :class:`TPError`.  The library must have been built
(``python -m tensor_transformer_linear_tp_amd.build``); importing the binding
without it fails loudly -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import sys

__all__ = [
    "TP_FP32", "TP_BF16", "TP_ACT_NONE", "TP_ACT_GELU", "TP_ACT_SWIGLU", "TPError", "LIB_PATH",
    "tp_abi_version", "tp_status_str", "tp_column_fwd", "tp_row_fwd", "tp_sum_partials", "tp_row_bwd",
    "tp_row_bwd_workspace_bytes", "tp_row_bwd_workspace_bytes_split", "tp_row_bwd_plan", "tp_row_bwd_plan_split",
    "tp_column_bwd", "tp_column_bwd_workspace_bytes", "tp_column_bwd_workspace_bytes_split", "tp_vocab_ce_partials",
    "tp_vocab_ce_workspace_bytes", "tp_vocab_ce_partials_noalloc", "tp_vocab_ce_combine", "tp_vocab_ce_bwd", "tp_vocab_ce_bwd_workspace_bytes", "tp_sp_reduce_scatter_ln",
    "tp_vocab_embed_fwd", "tp_vocab_embed_bwd", "tp_vocab_embed_bwd_workspace_bytes", "tp_attention_fwd",
    "tp_attention_fwd_workspace_bytes", "tp_attention_bwd", "tp_attention_bwd_workspace_bytes", "EXPORTED_SYMBOLS",
]

TP_FP32, TP_BF16 = 0, 1
TP_ACT_NONE, TP_ACT_GELU, TP_ACT_SWIGLU = 0, 1, 2

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtpshard.so")

_i64, _i32, _vp, _sz = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t

# name -> (restype, argtypes); mirrors include/tpshard.h
_SIGS = {
    "tp_abi_version": (_i32, []),
    "tp_status_str": (ctypes.c_char_p, [_i32]),
    "tp_column_fwd": (_i32, [_i32, _i32, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _vp,
                             _vp, _i64, _vp, _i64, _vp]),
    "tp_row_fwd": (_i32, [_i32, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp]),
    "tp_sum_partials": (_i32, [_i32, _i32, _i64, _i64, _vp, _i64, _i64, _vp, _vp, _i64, _vp]),
    "tp_row_bwd": (_i32, [_i32, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp,
                          _vp, _sz, _vp]),
    "tp_row_bwd_workspace_bytes": (_sz, [_i32, _i64, _i64]),
    "tp_row_bwd_workspace_bytes_split": (_sz, [_i32, _i64, _i64, _i64, _i32]),
    "tp_row_bwd_plan": (_i32, [_i64, _i64, _i64, _i32]),
    "tp_row_bwd_plan_split": (_i32, [_i64, _i64, _i64, _i32, _sz, ctypes.POINTER(_i32), ctypes.POINTER(_i32)]),
    "tp_column_bwd": (_i32, [_i32, _i32, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64,
                             _vp, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _sz, _vp]),
    "tp_column_bwd_workspace_bytes": (_sz, [_i32, _i32, _i64, _i64, _i32]),
    "tp_column_bwd_workspace_bytes_split": (_sz, [_i32, _i32, _i64, _i64, _i64, _i32, _i32]),
    "tp_vocab_ce_partials": (_i32, [_i32, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _vp,
                                    _sz, _vp]),
    "tp_vocab_ce_workspace_bytes": (_sz, [_i64, _i64]),
    "tp_vocab_ce_partials_noalloc": (_i32, [_i32, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _vp,
                                            _vp, _vp]),
    "tp_vocab_ce_combine": (_i32, [_i32, _i64, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _vp]),
    "tp_vocab_ce_bwd": (_i32, [_i32, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _i64, _vp,
                               _i64, _vp, _sz, _vp]),
    "tp_vocab_ce_bwd_workspace_bytes": (_sz, [_i64, _i64]),
    "tp_sp_reduce_scatter_ln": (_i32, [_i32, _i32, _i64, _i64, _vp, _i64, _i64, _i64, _i64, _vp, _vp, _i64, _vp, _vp,
                                       ctypes.c_float, _vp, _i64, _vp, _i64, _vp]),
    "tp_vocab_embed_fwd": (_i32, [_i32, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp]),
    "tp_vocab_embed_bwd": (_i32, [_i32, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _sz, _vp]),
    "tp_vocab_embed_bwd_workspace_bytes": (_sz, [_i64, _i64]),
    "tp_attention_fwd": (_i32, [_i32, _i64, _i64, _i32, _i32, _i32, _i32, ctypes.c_float, _vp, _i64, _vp, _i64, _vp,
                                _i64, _vp, _i64, _vp, _vp, _sz, _vp]),
    "tp_attention_fwd_workspace_bytes": (_sz, [_i64, _i64, _i32, _i32, _i32]),
    "tp_attention_bwd": (_i32, [_i32, _i64, _i64, _i32, _i32, _i32, _i32, ctypes.c_float, _vp, _i64, _vp, _i64, _vp,
                                _i64, _vp, _i64, _vp, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _sz, _vp]),
    "tp_attention_bwd_workspace_bytes": (_sz, [_i64, _i64, _i32, _i32, _i32]),
}
EXPORTED_SYMBOLS = tuple(_SIGS)

_STATUS_NAMES = {0: "TP_OK", 1: "TP_E_NULL", 2: "TP_E_SHAPE", 3: "TP_E_ALIGN", 4: "TP_E_DTYPE", 5: "TP_E_ACT",
                 6: "TP_E_WORKSPACE", 7: "TP_E_HIP"}


class TPError(RuntimeError):
    """A libtpshard call returned a non-OK status."""

    def __init__(self, func: str, status: int, message: str):
        super().__init__(f"{func}: {message}")
        self.func = func
        self.status = status
        self.name = _STATUS_NAMES.get(status, str(status))


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libtpshard is not built ({LIB_PATH} missing); run "
                              "`python -m tensor_transformer_linear_tp_amd.build` or __graft_entry__.build()")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(s):
    if s is None:
        torch = sys.modules.get("torch")
        if torch is not None and torch.cuda.is_available() and torch.cuda.is_initialized():
            return torch.cuda.current_stream().cuda_stream
        return None
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(func: str, status: int):
    if status != 0:
        raise TPError(func, status, _load().tp_status_str(status).decode())


def tp_abi_version() -> int:
    return _load().tp_abi_version()


def tp_status_str(status: int) -> str:
    return _load().tp_status_str(status).decode()


def tp_column_fwd(dtype, act, M, N, K, X, ldx, A, lda, A2, lda2, bias, bias2, Y, ldy, Pre, ldpre, stream=None):
    _check("tp_column_fwd", _load().tp_column_fwd(
        dtype, act, M, N, K, _ptr(X), ldx, _ptr(A), lda, _ptr(A2), lda2, _ptr(bias), _ptr(bias2),
        _ptr(Y), ldy, _ptr(Pre), ldpre, _stream(stream)))


def tp_row_fwd(dtype, M, N, K, Xi, ldx, Bi, ldb, Zp, ldz, stream=None):
    _check("tp_row_fwd", _load().tp_row_fwd(dtype, M, N, K, _ptr(Xi), ldx, _ptr(Bi), ldb, _ptr(Zp), ldz,
                                             _stream(stream)))


def tp_sum_partials(dtype, t, M, N, parts, ld, part_stride, bias, out, ldo, stream=None):
    _check("tp_sum_partials", _load().tp_sum_partials(dtype, t, M, N, _ptr(parts), ld, part_stride, _ptr(bias),
                                                       _ptr(out), ldo, _stream(stream)))


def tp_row_bwd(dtype, M, N, K, dZ, lddz, Xi, ldx, Bi, ldb, dXi, lddx, dBi, lddb, dbias, workspace, ws_bytes,
               stream=None):
    _check("tp_row_bwd", _load().tp_row_bwd(
        dtype, M, N, K, _ptr(dZ), lddz, _ptr(Xi), ldx, _ptr(Bi), ldb, _ptr(dXi), lddx, _ptr(dBi), lddb,
        _ptr(dbias), _ptr(workspace), ws_bytes, _stream(stream)))


def tp_row_bwd_workspace_bytes(dtype, M, N) -> int:
    return _load().tp_row_bwd_workspace_bytes(dtype, M, N)


def tp_row_bwd_workspace_bytes_split(dtype, M, N, K, cus) -> int:
    """Workspace with room for tp_row_bwd's split-contraction schedule on `cus` CUs (host only)."""
    return _load().tp_row_bwd_workspace_bytes_split(dtype, M, N, K, cus)


def tp_row_bwd_plan(M, N, K, cus) -> int:
    """Tile pairing of tp_row_bwd's one-launch schedule (host-only query): 0 = 256x256 + 256x256,
    1 = 192x256 + 256x192, 2 = 192x192 + 128x192, 3 = 128x128 + 128x192, 4 = 128x128 + 256x256,
    5 = 128x192 + 256x192, 6 = 128x192 + 128x192, -1 = separate launches, -2 = invalid sizes."""
    return _load().tp_row_bwd_plan(M, N, K, cus)


def tp_row_bwd_plan_split(M, N, K, cus, split_bytes):
    """(pairing, parts of dB's contraction, parts of dX's) with `split_bytes` of split scratch (host only)."""
    k0, k1 = ctypes.c_int(0), ctypes.c_int(0)
    plan = _load().tp_row_bwd_plan_split(M, N, K, cus, split_bytes, ctypes.byref(k0), ctypes.byref(k1))
    return plan, k0.value, k1.value


def tp_column_bwd(dtype, act, M, N, K, dY, lddy, X, ldx, A, lda, A2, lda2, Pre, ldpre, dXpart, lddx, dA, ldda,
                  dA2, ldda2, dbias, dbias2, workspace, ws_bytes, stream=None):
    _check("tp_column_bwd", _load().tp_column_bwd(
        dtype, act, M, N, K, _ptr(dY), lddy, _ptr(X), ldx, _ptr(A), lda, _ptr(A2), lda2, _ptr(Pre), ldpre,
        _ptr(dXpart), lddx, _ptr(dA), ldda, _ptr(dA2), ldda2, _ptr(dbias), _ptr(dbias2), _ptr(workspace),
        ws_bytes, _stream(stream)))


def tp_column_bwd_workspace_bytes(dtype, act, M, N, with_bias_grad) -> int:
    return _load().tp_column_bwd_workspace_bytes(dtype, act, M, N, int(bool(with_bias_grad)))


def tp_column_bwd_workspace_bytes_split(dtype, act, M, N, K, with_bias_grad, cus) -> int:
    """Workspace with room for tp_column_bwd's split-contraction schedule on `cus` CUs (host only)."""
    return _load().tp_column_bwd_workspace_bytes_split(dtype, act, M, N, K, int(bool(with_bias_grad)), cus)


def tp_vocab_ce_partials(dtype, M, Vr, K, H, ldh, W, ldw, target, v0, out_max, out_sumexp, out_tgt, workspace,
                         ws_bytes, stream=None):
    _check("tp_vocab_ce_partials", _load().tp_vocab_ce_partials(
        dtype, M, Vr, K, _ptr(H), ldh, _ptr(W), ldw, _ptr(target), v0, _ptr(out_max), _ptr(out_sumexp),
        _ptr(out_tgt), _ptr(workspace), ws_bytes, _stream(stream)))


def tp_vocab_ce_workspace_bytes(M, Vr) -> int:
    return _load().tp_vocab_ce_workspace_bytes(M, Vr)


def tp_vocab_ce_partials_noalloc(dtype, M, Vr, K, H, ldh, W, ldw, target, v0, out_max, out_sumexp, out_tgt,
                                 stream=None):
    _check("tp_vocab_ce_partials_noalloc", _load().tp_vocab_ce_partials_noalloc(
        dtype, M, Vr, K, _ptr(H), ldh, _ptr(W), ldw, _ptr(target), v0, _ptr(out_max), _ptr(out_sumexp),
        _ptr(out_tgt), _stream(stream)))


def tp_vocab_ce_combine(R, M, maxes, sumexps, tgts, stride, lse, tgt, loss, stream=None):
    _check("tp_vocab_ce_combine", _load().tp_vocab_ce_combine(
        R, M, _ptr(maxes), _ptr(sumexps), _ptr(tgts), stride, _ptr(lse), _ptr(tgt), _ptr(loss), _stream(stream)))


def tp_vocab_ce_bwd(dtype, M, Vr, K, H, ldh, W, ldw, target, v0, lse, gscale, dH, lddh, dW, lddw, workspace,
                    ws_bytes, stream=None):
    _check("tp_vocab_ce_bwd", _load().tp_vocab_ce_bwd(
        dtype, M, Vr, K, _ptr(H), ldh, _ptr(W), ldw, _ptr(target), v0, _ptr(lse), _ptr(gscale), _ptr(dH), lddh,
        _ptr(dW), lddw, _ptr(workspace), ws_bytes, _stream(stream)))


def tp_vocab_ce_bwd_workspace_bytes(M, Vr) -> int:
    return _load().tp_vocab_ce_bwd_workspace_bytes(M, Vr)


def tp_sp_reduce_scatter_ln(dtype, t, M, N, parts, ld, part_stride, r0, Mr, bias, resid, ldr, gamma, beta, eps, out,
                            ldo, hout, ldh, stream=None):
    _check("tp_sp_reduce_scatter_ln", _load().tp_sp_reduce_scatter_ln(
        dtype, t, M, N, _ptr(parts), ld, part_stride, r0, Mr, _ptr(bias), _ptr(resid), ldr, _ptr(gamma), _ptr(beta),
        float(eps), _ptr(out), ldo, _ptr(hout), ldh, _stream(stream)))


def tp_vocab_embed_fwd(dtype, M, Vr, K, ids, v0, E, lde, out, ldo, stream=None):
    _check("tp_vocab_embed_fwd", _load().tp_vocab_embed_fwd(dtype, M, Vr, K, _ptr(ids), v0, _ptr(E), lde, _ptr(out),
                                                             ldo, _stream(stream)))


def tp_vocab_embed_bwd(dtype, M, Vr, K, ids, v0, dout, lddo, dE, ldde, workspace, ws_bytes, stream=None):
    _check("tp_vocab_embed_bwd", _load().tp_vocab_embed_bwd(dtype, M, Vr, K, _ptr(ids), v0, _ptr(dout), lddo,
                                                             _ptr(dE), ldde, _ptr(workspace), ws_bytes,
                                                             _stream(stream)))


def tp_vocab_embed_bwd_workspace_bytes(M, Vr) -> int:
    return _load().tp_vocab_embed_bwd_workspace_bytes(M, Vr)


def tp_attention_fwd(dtype, B, S, n_q, n_kv, head_dim, causal, scale, Q, ldq, K, ldk, V, ldv, O, ldo, lse,
                     workspace, ws_bytes, stream=None):
    _check("tp_attention_fwd", _load().tp_attention_fwd(
        dtype, B, S, n_q, n_kv, head_dim, int(causal), float(scale), _ptr(Q), ldq, _ptr(K), ldk, _ptr(V), ldv, _ptr(O),
        ldo, _ptr(lse), _ptr(workspace), ws_bytes, _stream(stream)))


def tp_attention_fwd_workspace_bytes(B, S, n_q, n_kv, causal) -> int:
    return _load().tp_attention_fwd_workspace_bytes(B, S, n_q, n_kv, int(causal))


def tp_attention_bwd(dtype, B, S, n_q, n_kv, head_dim, causal, scale, Q, ldq, K, ldk, V, ldv, O, ldo, lse, dO, lddo,
                     dQ, lddq, dK, lddk, dV, lddv, workspace, ws_bytes, stream=None):
    _check("tp_attention_bwd", _load().tp_attention_bwd(
        dtype, B, S, n_q, n_kv, head_dim, int(causal), float(scale), _ptr(Q), ldq, _ptr(K), ldk, _ptr(V), ldv, _ptr(O),
        ldo, _ptr(lse), _ptr(dO), lddo, _ptr(dQ), lddq, _ptr(dK), lddk, _ptr(dV), lddv, _ptr(workspace), ws_bytes,
        _stream(stream)))


def tp_attention_bwd_workspace_bytes(B, S, n_q, n_kv, causal) -> int:
    return _load().tp_attention_bwd_workspace_bytes(B, S, n_q, n_kv, int(causal))
