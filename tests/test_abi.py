"""The C ABI on the CPU: the library loads, exports exactly what the header
declares, and rejects every invalid argument with its status code before any
HIP call (no compute call is made here)."""
import os
import re
import subprocess

import pytest

import tensor_transformer_linear_tp_amd as tp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tpshard.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(tp.LIB_PATH):
        from tensor_transformer_linear_tp_amd import build
        build.build()
    return tp._load()


def _header_functions():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^TP_API\s+[\w\s\*]+?\b(tp_\w+)\s*\(", src, flags=re.M)))


def test_exports_match_header(lib):
    declared = _header_functions()
    assert declared == sorted(tp.EXPORTED_SYMBOLS)
    out = subprocess.run(["nm", "-D", "--defined-only", tp.LIB_PATH], capture_output=True, text=True, check=True)
    exported = sorted(l.split()[-1] for l in out.stdout.splitlines() if " T tp_" in l)
    assert exported == declared
    for name in declared:
        assert hasattr(lib, name)


def test_calibration_library_exports_its_header():
    # libtpcalib (the MFMA-only calibration kernel) is a measurement helper with
    # its own header; it loads and exports exactly what include/tpcalib.h declares.
    import ctypes
    from tensor_transformer_linear_tp_amd import build
    if not os.path.exists(build.CALIB_PATH):
        build.build()
    src = open(os.path.join(ROOT, "include", "tpcalib.h")).read()
    declared = sorted(set(re.findall(r"^TPC_API\s+[\w\s\*]+?\b(tpc_\w+)\s*\(", src, flags=re.M)))
    out = subprocess.run(["nm", "-D", "--defined-only", build.CALIB_PATH], capture_output=True, text=True, check=True)
    exported = sorted(l.split()[-1] for l in out.stdout.splitlines() if " T " in l)
    assert declared == exported == ["tpc_clock_probe", "tpc_lds_read_rate", "tpc_mfma_loop"]
    lib = ctypes.CDLL(build.CALIB_PATH)
    lib.tpc_mfma_loop.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_void_p]
    assert lib.tpc_mfma_loop(None, None, 256, 10, 32, None) == -1      # validation only, nothing launched
    assert lib.tpc_mfma_loop(P, P, 256, 0, 32, None) == -1
    assert lib.tpc_mfma_loop(P, P, 256, 10, 8, None) == -1
    lib.tpc_clock_probe.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    assert lib.tpc_clock_probe(None, 256, 1000, None) == -1
    assert lib.tpc_clock_probe(P, 0, 1000, None) == -1 and lib.tpc_clock_probe(P, 256, 0, None) == -1
    lib.tpc_lds_read_rate.argtypes = [ctypes.c_void_p, ctypes.c_void_p] + [ctypes.c_int] * 4 + [ctypes.c_void_p]
    assert lib.tpc_lds_read_rate(None, P, 256, 8, 10, 0, None) == -1
    assert lib.tpc_lds_read_rate(P, None, 256, 8, 10, 0, None) == -1
    assert lib.tpc_lds_read_rate(P, P, 256, 17, 10, 0, None) == -1     # at most 16 waves
    assert lib.tpc_lds_read_rate(P, P, 256, 8, 10, 3, None) == -1      # kinds 0..2
    assert lib.tpc_lds_read_rate(P, P, 0, 8, 10, 0, None) == -1 and lib.tpc_lds_read_rate(P, P, 256, 8, 0, 0, None) == -1


def test_version_and_status_strings(lib):
    assert tp.tp_abi_version() == 1
    seen = set()
    for code in range(8):
        s = tp.tp_status_str(code)
        assert s and s not in seen
        seen.add(s)
    assert "unknown" in tp.tp_status_str(99)


P = 0x100000  # a 16-byte aligned stand-in address; validation fails before it is ever used


def _rc(fn, *args):
    return getattr(tp._load(), fn)(*args)


def test_column_fwd_validation(lib):
    ok = dict(dtype=tp.TP_BF16, act=tp.TP_ACT_GELU, M=64, N=64, K=64, X=P, ldx=64, A=P, lda=64, A2=None, lda2=0,
              bias=None, bias2=None, Y=P, ldy=64, Pre=P, ldpre=64, stream=None)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return _rc("tp_column_fwd", *a.values())

    assert call(dtype=7) == 4
    assert call(act=9) == 5
    assert call(X=None) == 1
    assert call(Pre=None) == 1                              # GeLU needs Pre
    assert call(act=tp.TP_ACT_SWIGLU, ldpre=128) == 1       # SwiGLU needs A2
    assert call(M=0) == 2 and call(N=-1) == 2 and call(K=1 << 31) == 2
    assert call(ldx=32) == 2                                # ld < width
    assert call(ldx=68) == 3                                # ld not a multiple of 8 (bf16)
    assert call(X=P + 8) == 3                               # misaligned base
    assert call(bias=P + 2) == 3
    assert call(act=tp.TP_ACT_SWIGLU, A2=P, lda2=64, ldpre=64) == 2   # SwiGLU Pre needs 2N columns
    assert call(dtype=tp.TP_FP32, ldx=66) == 3              # fp32: multiple of 4


def test_row_and_sum_validation(lib):
    assert _rc("tp_row_fwd", 5, 8, 8, 8, P, 8, P, 8, P, 8, None) == 4
    assert _rc("tp_row_fwd", tp.TP_BF16, 8, 8, 8, None, 8, P, 8, P, 8, None) == 1
    assert _rc("tp_row_fwd", tp.TP_BF16, 8, 8, 8, P, 8, P, 8, P, 4, None) == 2
    assert _rc("tp_sum_partials", tp.TP_BF16, 0, 8, 8, P, 8, 64, None, P, 8, None) == 2
    assert _rc("tp_sum_partials", tp.TP_BF16, 2, 8, 8, P, 8, -64, None, P, 8, None) == 2
    assert _rc("tp_sum_partials", tp.TP_BF16, 2, 8, 8, P, 8, 60, None, P, 8, None) == 3
    assert _rc("tp_sum_partials", tp.TP_BF16, 2, 8, 8, None, 8, 64, None, P, 8, None) == 1


def test_backward_validation_and_workspace(lib):
    need = tp.tp_row_bwd_workspace_bytes(tp.TP_BF16, 100, 300)
    assert need >= 2 * 4 * 300 * 2  # two 64-row partial blocks of fp32 column sums
    # dbias without workspace
    assert _rc("tp_row_bwd", tp.TP_BF16, 100, 300, 64, P, 304, P, 64, P, 304, P, 64, None, 0, P, None, 0, None) == 6
    assert _rc("tp_row_bwd", tp.TP_BF16, 100, 300, 64, P, 304, P, 64, P, 304, P, 64, None, 0, P, P, need - 1,
               None) == 6
    # column bwd: SwiGLU needs both or neither weight gradients
    args = [tp.TP_BF16, tp.TP_ACT_SWIGLU, 64, 64, 64, P, 64, P, 64, P, 64, P, 64, P, 128, P, 64, P, 64, None, 0,
            None, None, P, 1 << 30, None]
    assert _rc("tp_column_bwd", *args) == 1
    args[19], args[20] = P, 64
    ws = tp.tp_column_bwd_workspace_bytes(tp.TP_BF16, tp.TP_ACT_SWIGLU, 64, 64, 0)
    assert ws == 2 * 64 * 64 * 2
    args[23], args[24] = P, ws - 1
    assert _rc("tp_column_bwd", *args) == 6
    assert tp.tp_column_bwd_workspace_bytes(tp.TP_BF16, tp.TP_ACT_NONE, 64, 64, 0) == 0


def test_ce_validation(lib):
    ws = tp.tp_vocab_ce_workspace_bytes(8192, 18992)
    assert ws == (2 * 75 * 8192 + 8192) * 4
    base = [tp.TP_BF16, 8192, 18992, 4096, P, 4096, P, 4096, P, 0, P, P, P, P, ws, None]
    a = list(base); a[0] = tp.TP_FP32
    assert _rc("tp_vocab_ce_partials", *a) == 4
    a = list(base); a[8] = None
    assert _rc("tp_vocab_ce_partials", *a) == 1
    a = list(base); a[14] = ws - 4
    assert _rc("tp_vocab_ce_partials", *a) == 6
    a = list(base); a[10] = P + 4
    assert _rc("tp_vocab_ce_partials", *a) == 3


def test_ce_noalloc_validation(lib):
    # Same checks as tp_vocab_ce_partials, and shapes whose per-tile partials
    # exceed the library's scratch array are rejected before any HIP call.
    assert tp.tp_vocab_ce_workspace_bytes(8192, 18992) <= 16 << 20
    base = [tp.TP_BF16, 8192, 18992, 4096, P, 4096, P, 4096, P, 0, P, P, P, None]
    a = list(base); a[0] = tp.TP_FP32
    assert _rc("tp_vocab_ce_partials_noalloc", *a) == 4
    a = list(base); a[8] = None
    assert _rc("tp_vocab_ce_partials_noalloc", *a) == 1
    a = list(base); a[12] = P + 4
    assert _rc("tp_vocab_ce_partials_noalloc", *a) == 3
    # (2 * ceil(Vr / 256) + 1) * M * 4 bytes: Vr = 65280 is the largest that fits at M = 8192
    assert tp.tp_vocab_ce_workspace_bytes(8192, 65280) <= 16 << 20 < tp.tp_vocab_ce_workspace_bytes(8192, 65281)
    a = list(base); a[2] = 65281
    assert _rc("tp_vocab_ce_partials_noalloc", *a) == 6
    a = list(base); a[2] = 256; a[3] = 8; a[5] = 8; a[7] = 8   # one vocab tile: (2 + 1) * M * 4 bytes
    a[1] = 1 << 21                                             # 24 MiB at 2^21 tokens
    assert _rc("tp_vocab_ce_partials_noalloc", *a) == 6


def test_row_bwd_plan(lib):
    # The one-launch row backward's tile pairing, host-only (library order: dZ [M, N], X_i [M, K]).
    assert tp.tp_row_bwd_plan(8192, 4096, 1536, 256) == 1    # the MLP shard step: 192x256 + 256x192
    assert tp.tp_row_bwd_plan(768, 768, 8192, 256) == 0      # 256x256 + 256x256
    assert tp.tp_row_bwd_plan(512, 512, 8192, 256) == 1
    assert tp.tp_row_bwd_plan(512, 768, 256, 256) == 2       # 192x192 + 128x192
    assert tp.tp_row_bwd_plan(768, 512, 512, 256) == 3       # 128x128 + 128x192
    assert tp.tp_row_bwd_plan(1536, 512, 4096, 256) == 4     # 128x128 + 256x256
    assert tp.tp_row_bwd_plan(8192, 4096, 512, 256) == 5     # the attention output projection, without scratch: 128x192 + 256x192
    assert tp.tp_row_bwd_plan(8192, 768, 4096, 256) == 5     # the QKV projection's backward, without scratch
    assert tp.tp_row_bwd_plan(512, 512, 256, 256) == 6       # 128x192 + 128x192
    assert tp.tp_row_bwd_plan(4096, 8192, 8192, 256) == -1   # separate launches
    assert tp.tp_row_bwd_plan(8192, 4096, 1536, 100) == -1   # CUs not a multiple of 8: no shared launch
    assert tp.tp_row_bwd_plan(0, 1, 1, 256) == -2 and tp.tp_row_bwd_plan(1, 1, 1, 0) == -2


def test_row_bwd_split_plan(lib):
    # Split contractions need scratch past the bias-gradient partials; without it the plan is tp_row_bwd_plan's.
    BF = tp.TP_BF16
    for shape in [(8192, 4096, 1536), (8192, 4096, 512), (8192, 768, 4096), (512, 512, 128)]:
        assert tp.tp_row_bwd_plan_split(*shape, 256, 0) == (tp.tp_row_bwd_plan(*shape, 256), 1, 1)
    # the attention output projection's backward: dW [512, 4096] over 8192 tokens in 4 parts, dX [8192, 512]
    # over 4096 in 2, both in 256x256 tiles: 4 * 512 * 4096 + 2 * 8192 * 512 floats of scratch
    need = (4 * 512 * 4096 + 2 * 8192 * 512) * 4
    base = tp.tp_row_bwd_workspace_bytes(BF, 8192, 4096)
    assert tp.tp_row_bwd_workspace_bytes_split(BF, 8192, 4096, 512, 256) == base + need
    assert tp.tp_row_bwd_plan_split(8192, 4096, 512, 256, need) == (0, 4, 2)
    assert tp.tp_row_bwd_plan_split(8192, 4096, 512, 256, need - 1)[1:] != (4, 2)   # does not fit: another plan
    # the MLP shard step does not split
    assert tp.tp_row_bwd_workspace_bytes_split(BF, 8192, 4096, 1536, 256) == base
    assert tp.tp_row_bwd_plan_split(8192, 4096, 1536, 256, 1 << 40) == (1, 1, 1)
    # the QKV projection's backward: 256x256 tiles, dW [4096, 768] over 8192 tokens in 2 parts
    assert tp.tp_row_bwd_plan_split(8192, 768, 4096, 256, 1 << 40) == (0, 2, 1)
    qkv = tp.tp_column_bwd_workspace_bytes(BF, tp.TP_ACT_NONE, 8192, 768, 0)
    assert tp.tp_column_bwd_workspace_bytes_split(BF, tp.TP_ACT_NONE, 8192, 768, 4096, 0, 256) == qkv + 2 * 4096 * 768 * 4
    col = tp.tp_column_bwd_workspace_bytes(BF, tp.TP_ACT_NONE, 8192, 4096, 1)
    assert tp.tp_column_bwd_workspace_bytes_split(BF, tp.TP_ACT_NONE, 8192, 4096, 512, 1, 256) == col + need
    # only the activation-free bf16 backward runs the pair as one launch
    assert (tp.tp_column_bwd_workspace_bytes_split(BF, tp.TP_ACT_GELU, 8192, 4096, 512, 0, 256) ==
            tp.tp_column_bwd_workspace_bytes(BF, tp.TP_ACT_GELU, 8192, 4096, 0))
    assert (tp.tp_row_bwd_workspace_bytes_split(tp.TP_FP32, 8192, 4096, 512, 256) ==
            tp.tp_row_bwd_workspace_bytes(tp.TP_FP32, 8192, 4096))
    assert tp.tp_row_bwd_workspace_bytes_split(BF, 0, 4096, 512, 256) == 0
    assert tp.tp_row_bwd_plan_split(8192, 4096, 512, 0, need) == (-2, 1, 1)


def test_row_bwd_split_workspace_matches_plan(lib):
    # Over a grid of shapes: the workspace that tp_row_bwd_workspace_bytes_split reports holds exactly
    # the planes of the plan taken with unlimited scratch (ks * rows * cols fp32 per split product,
    # 256-byte rounded), that plan is the one taken with just that much, and a plan never splits a
    # contraction into parts that are not whole 32-deep stages.
    BF = tp.TP_BF16
    dims = [128, 384, 768, 1536, 4096, 8192]
    seen = set()
    for M in dims:
        for N in dims:
            for K in dims:
                base = tp.tp_row_bwd_workspace_bytes(BF, M, N)
                extra = tp.tp_row_bwd_workspace_bytes_split(BF, M, N, K, 256) - base
                plan, k0, k1 = tp.tp_row_bwd_plan_split(M, N, K, 256, 1 << 50)
                planes = lambda ks, r, c: 0 if ks == 1 else (ks * r * c * 4 + 255) // 256 * 256
                assert extra == planes(k0, K, N) + planes(k1, M, K), (M, N, K, plan, k0, k1)
                assert tp.tp_row_bwd_plan_split(M, N, K, 256, extra) == (plan, k0, k1)
                assert M % (32 * k0) == 0 and N % (32 * k1) == 0
                if plan == -1:
                    assert (k0, k1) == (1, 1)
                seen.add((k0 > 1, k1 > 1))
    assert seen == {(False, False), (True, False), (False, True), (True, True)}


def test_ce_combine_validation(lib):
    def call(R=8, M=64, ms=P, ss=P, ts=P, stride=64, lse=P, tgt=P, loss=P):
        return _rc("tp_vocab_ce_combine", R, M, ms, ss, ts, stride, lse, tgt, loss, None)

    assert call(ms=None) == 1 and call(ss=None) == 1 and call(ts=None) == 1
    assert call(lse=None, tgt=None, loss=None) == 1          # nothing to write
    assert call(R=0) == 2 and call(M=0) == 2
    assert call(stride=32) == 2                              # stride < M
    assert call(R=1 << 20, stride=1 << 12, M=64) == 2        # R * stride past 2^31
    assert call(stride=66) == 3                              # not a multiple of 4 floats
    assert call(ms=P + 4) == 3 and call(loss=P + 8) == 3


def test_ce_bwd_validation(lib):
    ws = tp.tp_vocab_ce_bwd_workspace_bytes(8192, 18992)
    assert ws == 8192 * 18992 * 2                        # bf16 dz, rows padded to 8 (already)
    assert tp.tp_vocab_ce_bwd_workspace_bytes(3, 5) == 256    # 3 x 8 x 2 bytes, rounded to 256
    base = [tp.TP_BF16, 8192, 18992, 4096, P, 4096, P, 4096, P, 0, P, None, P, 4096, P, 4096, P, ws, None]
    a = list(base); a[0] = tp.TP_FP32
    assert _rc("tp_vocab_ce_bwd", *a) == 4
    a = list(base); a[10] = None                              # lse is required
    assert _rc("tp_vocab_ce_bwd", *a) == 1
    a = list(base); a[17] = ws - 2
    assert _rc("tp_vocab_ce_bwd", *a) == 6
    a = list(base); a[11] = P + 4                             # gscale misaligned
    assert _rc("tp_vocab_ce_bwd", *a) == 3
    a = list(base); a[13] = 4000                              # ld(dH) < K
    assert _rc("tp_vocab_ce_bwd", *a) == 2
    a = list(base); a[12], a[14], a[16] = None, None, None    # nothing requested: no work, no workspace
    assert _rc("tp_vocab_ce_bwd", *a) == 0


def test_sp_reduce_scatter_ln_validation(lib):
    # t=8 partials [8192, 4096], rank 3 of 8 keeps rows [3072, 4096)
    base = [tp.TP_BF16, 8, 8192, 4096, P, 4096, 8192 * 4096, 3072, 1024, P, P, 4096, P, P, 1e-5, P, 4096, P, 4096,
            None]
    a = list(base); a[0] = 7
    assert _rc("tp_sp_reduce_scatter_ln", *a) == 4
    a = list(base); a[15] = None                              # out is required
    assert _rc("tp_sp_reduce_scatter_ln", *a) == 1
    a = list(base); a[3] = 16385                              # wider than the register-held row
    a[5] = a[16] = a[11] = a[18] = 16392
    assert _rc("tp_sp_reduce_scatter_ln", *a) == 2
    a = list(base); a[7] = 7169                               # r0 + Mr > M
    assert _rc("tp_sp_reduce_scatter_ln", *a) == 2
    a = list(base); a[7] = -1
    assert _rc("tp_sp_reduce_scatter_ln", *a) == 2
    a = list(base); a[8] = 0                                  # empty block
    assert _rc("tp_sp_reduce_scatter_ln", *a) == 2
    for eps in (-1e-5, float("nan"), float("inf")):
        a = list(base); a[14] = eps
        assert _rc("tp_sp_reduce_scatter_ln", *a) == 2
    a = list(base); a[6] = 8192 * 4096 + 4                    # part_stride not a multiple of 8
    assert _rc("tp_sp_reduce_scatter_ln", *a) == 3
    a = list(base); a[12] = P + 2                             # gamma misaligned
    assert _rc("tp_sp_reduce_scatter_ln", *a) == 3
    a = list(base); a[11] = 4000                              # ld(resid) < N
    assert _rc("tp_sp_reduce_scatter_ln", *a) == 2
    a = list(base); a[18] = 4104                              # hout == resid with another ld
    assert _rc("tp_sp_reduce_scatter_ln", *a) == 2
    a = list(base); a[2] = 1 << 19                            # partials span >= 2 GiB
    a[8] = 1 << 16
    assert _rc("tp_sp_reduce_scatter_ln", *a) == 2


def test_vocab_embed_validation(lib):
    ws = tp.tp_vocab_embed_bwd_workspace_bytes(8192, 18992)
    assert ws == 76032 + 32768                               # row starts (Vr + 1), token order (M), int32
    assert tp.tp_vocab_embed_bwd_workspace_bytes(0, 5) == 0
    fwd = [tp.TP_BF16, 8192, 18992, 4096, P, 0, P, 4096, P, 4096, None]
    a = list(fwd); a[0] = 9
    assert _rc("tp_vocab_embed_fwd", *a) == 4
    a = list(fwd); a[4] = None                                # ids required
    assert _rc("tp_vocab_embed_fwd", *a) == 1
    a = list(fwd); a[4] = P + 4                               # ids not 16-byte aligned
    assert _rc("tp_vocab_embed_fwd", *a) == 3
    a = list(fwd); a[7] = 4000                                # lde < K
    assert _rc("tp_vocab_embed_fwd", *a) == 2
    a = list(fwd); a[9] = 4100                                # ldo not a multiple of 8
    assert _rc("tp_vocab_embed_fwd", *a) == 3
    a = list(fwd); a[1] = 0
    assert _rc("tp_vocab_embed_fwd", *a) == 2
    bwd = [tp.TP_FP32, 8192, 18992, 4096, P, 0, P, 4096, P, 4096, P, ws, None]
    a = list(bwd); a[11] = ws - 4
    assert _rc("tp_vocab_embed_bwd", *a) == 6
    a = list(bwd); a[10] = None
    assert _rc("tp_vocab_embed_bwd", *a) == 6
    a = list(bwd); a[10] = P + 8
    assert _rc("tp_vocab_embed_bwd", *a) == 3
    a = list(bwd); a[8] = None                                # dE required
    assert _rc("tp_vocab_embed_bwd", *a) == 1
    a = list(bwd); a[2] = 1 << 31                             # Vr out of range
    assert _rc("tp_vocab_embed_bwd", *a) == 2


def test_attention_validation(lib):
    sc = 1.0 / 128 ** 0.5
    # packed QKV [8192, 768]: 4 query heads, 1 KV head
    ws = tp.tp_attention_fwd_workspace_bytes(1, 8192, 4, 1, 1)
    # 256 query blocks of 32 tokens x 4 heads; causal chunks of ceil(1.2 x 16512 key tiles / 512) = 39
    # tiles, so up to 4 chunks per block; 130 x 128 floats per chunk
    assert ws == 256 * 4 * (128 * 128 + 256) * 4
    assert tp.tp_attention_fwd_workspace_bytes(1, 512, 4, 1, 1) == 0           # one chunk: no workspace
    assert tp.tp_attention_fwd_workspace_bytes(1, 8192, 4, 3, 1) == 0          # invalid shape
    base = [tp.TP_BF16, 1, 8192, 4, 1, 128, 1, sc, P, 768, P + 1024, 768, P + 1280, 768, P, 512, P, P, ws, None]
    a = list(base); a[18] = ws - 1
    assert _rc("tp_attention_fwd", *a) == 6
    a = list(base); a[17] = None
    assert _rc("tp_attention_fwd", *a) == 6
    a = list(base); a[0] = tp.TP_FP32
    assert _rc("tp_attention_fwd", *a) == 4
    a = list(base); a[5] = 64                                 # head dim other than 128
    assert _rc("tp_attention_fwd", *a) == 2
    a = list(base); a[3], a[4] = 6, 2                         # group 3: neither divides nor is divided by 4
    assert _rc("tp_attention_fwd", *a) == 2
    a = list(base); a[3], a[4] = 4, 3                         # n_q not a multiple of n_kv
    assert _rc("tp_attention_fwd", *a) == 2
    a = list(base); a[6] = 2
    assert _rc("tp_attention_fwd", *a) == 2
    for bad in (0.0, -1.0, float("nan"), float("inf")):
        a = list(base); a[7] = bad
        assert _rc("tp_attention_fwd", *a) == 2
    a = list(base); a[16] = None                              # lse required
    assert _rc("tp_attention_fwd", *a) == 1
    a = list(base); a[16] = P + 4
    assert _rc("tp_attention_fwd", *a) == 3
    a = list(base); a[9] = 500                                # ldq < 4 x 128
    assert _rc("tp_attention_fwd", *a) == 2
    a = list(base); a[10] = P + 1026                          # K not 16-byte aligned
    assert _rc("tp_attention_fwd", *a) == 3
    a = list(base); a[1] = 1 << 16                            # more sequences than the grid takes
    assert _rc("tp_attention_fwd", *a) == 2


def test_attention_bwd_validation(lib):
    sc = 1.0 / 128 ** 0.5
    ws = tp.tp_attention_bwd_workspace_bytes(1, 8192, 4, 1, 1)
    ld = 4 * 8192 * 8                                          # (lse2, D) pairs
    dq = 256 * 4 * 128 * 128 * 4                               # dQ partials: 256 blocks x 4 key chunks
    kv = 64 * 4 * 2 * 128 * 256 * 4                            # dK/dV partials: 64 key blocks x 4 heads x 2 chunks
    assert ws == ld + dq + kv
    assert tp.tp_attention_bwd_workspace_bytes(1, 8192, 4, 3, 1) == 0
    base = [tp.TP_BF16, 1, 8192, 4, 1, 128, 1, sc, P, 768, P + 1024, 768, P + 1280, 768, P, 512, P, P, 512,
            P, 512, P, 128, P, 128, P, ws, None]
    a = list(base); a[0] = tp.TP_FP32
    assert _rc("tp_attention_bwd", *a) == 4
    for i in (14, 16, 17, 19, 21, 23):                         # O, lse, dO, dQ, dK, dV are required
        a = list(base); a[i] = None
        assert _rc("tp_attention_bwd", *a) == 1
    a = list(base); a[26] = ws - 1
    assert _rc("tp_attention_bwd", *a) == 6
    a = list(base); a[22] = 120                                # ld(dK) < 128
    assert _rc("tp_attention_bwd", *a) == 2
    a = list(base); a[16] = P + 8                              # lse not 16-byte aligned
    assert _rc("tp_attention_bwd", *a) == 3


def test_bf16_operands_below_2gib(lib):
    # X [2^17, 2^13] bf16 spans exactly 2 GiB: rejected before any HIP call.
    K = 1 << 13
    args = [tp.TP_BF16, tp.TP_ACT_NONE, 1 << 17, 256, K, P, K, P, 256, None, 0, None, None, P, 256, None, 0, None]
    assert _rc("tp_column_fwd", *args) == 2
    # the same through an ld that makes a small matrix span 2 GiB
    args = [tp.TP_BF16, tp.TP_ACT_NONE, 2, 256, 64, P, 1 << 30, P, 256, None, 0, None, None, P, 256, None, 0, None]
    assert _rc("tp_column_fwd", *args) == 2


def test_binding_raises_typed_errors(lib):
    with pytest.raises(tp.TPError) as ei:
        tp.tp_row_fwd(tp.TP_BF16, 0, 8, 8, P, 8, P, 8, P, 8, stream=0)
    assert ei.value.status == 2 and ei.value.name == "TP_E_SHAPE"
