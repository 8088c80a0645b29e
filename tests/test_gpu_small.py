"""GPU parity on the pages' worked examples and on small ragged shapes.

Every call goes through the C ABI (via the torch front end of the binding)
and is compared element by element with the float64 oracle on the same
seeded inputs."""
import json
import os

import numpy as np
import pytest

import oracle
import synthetic as syn

from .gpu_util import TOL, assert_close, dev, host64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
ops = pytest.importorskip("tensor_transformer_linear_tp_amd.torch_ops")
tp = pytest.importorskip("tensor_transformer_linear_tp_amd")

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
DTYPES = [syn.FP32, syn.BF16]


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _t(values, dtype):
    return dev(syn.from_values(values, dtype))


def _exact(gpu, ref):
    assert np.array_equal(host64(gpu), np.asarray(ref, dtype=np.float64)), (host64(gpu), ref)


@pytest.mark.parametrize("dtype", DTYPES)
def test_v1_block_2x2_on_gpu(dtype):
    g = _golden("v1_block_2x2.json")
    X = np.array(g["X"], np.float32)
    A = np.array(g["A"], np.float32)
    for i in range(2):
        Y, _ = ops.column_fwd(_t(X, dtype), _t(A[:, i:i + 1], dtype))
        torch.cuda.synchronize()
        _exact(Y, g["column_t2"]["shard_outputs"][i])
    parts = [ops.row_fwd(_t(X[:, i:i + 1], dtype), _t(A[i:i + 1, :], dtype)) for i in range(2)]
    torch.cuda.synchronize()
    for i in range(2):
        _exact(parts[i], g["row_t2"]["shard_partials"][i])
    buf, N = ops.stack_partials(parts)
    Z = ops.sum_partials(buf, N)
    torch.cuda.synchronize()
    _exact(Z, g["row_t2"]["sum"])


@pytest.mark.parametrize("dtype", DTYPES)
def test_v2_column_t3_on_gpu(dtype):
    g = _golden("v2_column_t3.json")
    X = np.array(g["X"], np.float32)
    W = np.array(g["W"], np.float32)
    dY = np.array(g["dY"], np.float32)
    parts = []
    for i in range(3):
        Xd = _t(X, dtype)
        Y, _ = ops.column_fwd(Xd, _t(W[:, i:i + 1], dtype))
        dXp, dA, dA2, db, db2 = ops.column_bwd(_t(dY[:, i:i + 1], dtype), Xd, _t(W[:, i:i + 1], dtype),
                                                want_db=True)
        torch.cuda.synchronize()
        _exact(Y, g["Y_shards"][i])
        _exact(dA, g["dW_shards"][i])
        _exact(dXp, g["dX_parts"][i])
        _exact(db, dY[0, i:i + 1])
        assert dA2 is None and db2 is None
        parts.append(dXp)
    buf, N = ops.stack_partials(parts)
    dX = ops.sum_partials(buf, N)
    torch.cuda.synchronize()
    _exact(dX, g["dX"])


def test_bf16_output_rounding_is_nearest_even():
    # Products exact in fp32; ties must go to the even bf16 neighbour.
    h = 2.0 ** -9
    X = np.array([[1.0, h]], np.float32)
    A = np.array([[1, 1, 1, 1, 1], [2, 6, -1, 3, -3]], np.float32)
    Y, _ = ops.column_fwd(_t(X, syn.BF16), _t(A, syn.BF16))
    torch.cuda.synchronize()
    _exact(Y, [[1.0, 1.015625, 1.0, 1.0078125, 0.9921875]])


SHAPES = [(1, 1, 1), (5, 3, 17), (129, 200, 72), (300, 520, 136), (520, 300, 1030)]


def _inputs(dtype, M, N, K, seed, act):
    s = 1_000_000 + seed
    d = {
        "X": syn.normal(s + 1, (M, K), 1.0, dtype),
        "A": syn.normal(s + 2, (K, N), 0.1, dtype),
        "A2": syn.normal(s + 3, (K, N), 0.1, dtype),
        "b": syn.normal(s + 4, (N,), 0.5, dtype),
        "b2": syn.normal(s + 5, (N,), 0.5, dtype),
        "dY": syn.normal(s + 6, (M, N), 1.0, dtype),
        "Pre": syn.normal(s + 7, (M, 2 * N if act == "swiglu" else N), 1.0, dtype),
        "B": syn.normal(s + 8, (N, K), 0.1, dtype),      # row weight [K_i = N, N_out = K]
        "dZ": syn.normal(s + 9, (M, K), 1.0, dtype),
    }
    return d


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("act", ["none", "gelu", "swiglu"])
@pytest.mark.parametrize("bias", [False, True])
def test_column_fwd_ragged(dtype, shape, act, bias):
    M, N, K = shape
    d = _inputs(dtype, M, N, K, 7 * M + 13 * N + 17 * K + 3 * ["none", "gelu", "swiglu"].index(act) + int(bias), act)
    Y, Pre = ops.column_fwd(dev(d["X"]), dev(d["A"]), act, A2=dev(d["A2"]) if act == "swiglu" else None,
                            bias=dev(d["b"]) if bias else None,
                            bias2=dev(d["b2"]) if (bias and act == "swiglu") else None)
    torch.cuda.synchronize()
    Yr, Prer = oracle.column_fwd(d["X"].f64, d["A"].f64, act, bias=d["b"].f64 if bias else None,
                                 A2=d["A2"].f64 if act == "swiglu" else None,
                                 bias2=d["b2"].f64 if (bias and act == "swiglu") else None)
    assert_close("Y", host64(Y), Yr, TOL[dtype])
    if act != "none":
        assert_close("Pre", host64(Pre), Prer, TOL[dtype])


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("shape", SHAPES)
def test_row_fwd_and_bwd_ragged(dtype, shape):
    M, N, K = shape   # row shard: X_i [M, N], B_i [N, K], Z [M, K]
    d = _inputs(dtype, M, N, K, 7 + M, "none")
    Xi, Bi = dev(d["dY"]), dev(d["B"])
    Z = ops.row_fwd(Xi, Bi)
    dX, dB, db = ops.row_bwd(dev(d["dZ"]), Xi, Bi, want_db=True)
    torch.cuda.synchronize()
    assert_close("Z", host64(Z), oracle.row_fwd(d["dY"].f64, d["B"].f64), TOL[dtype])
    rdX, rdB, rdb = oracle.row_bwd(d["dZ"].f64, d["dY"].f64, d["B"].f64)
    assert_close("dX", host64(dX), rdX, TOL[dtype])
    assert_close("dB", host64(dB), rdB, TOL[dtype])
    assert_close("db", host64(db), rdb, TOL[dtype])


# Whole tiles only (the persistent whole-tile kernels; for the row backward,
# its two GEMMs share one launch).  On 256 CUs the row backward takes 192 x
# 192 weight-gradient tiles beside 128 x 192 input-gradient tiles for the
# first shape and 128 x 128 beside 256 x 256 for the second and third
# (tp_row_bwd_plan); test_row_bwd_whole_matrix_pairings
# asserts each pairing.
TILE_SHAPES = [(512, 256, 768), (768, 512, 256), (2048, 1024, 768)]


@pytest.mark.parametrize("act", ["none", "gelu", "swiglu"])
@pytest.mark.parametrize("bias", [False, True])
def test_column_fwd_half_tile_tail_round(act, bias):
    # 17 x 17 = 289 whole tiles on 256 CUs: the last 33 run as 128-row halves
    # (with a bias: the fast kernels start those tiles' accumulators at it).
    M, K = 17 * 256, 64
    N = 17 * (128 if act == "swiglu" else 256)
    dtype = syn.BF16
    d = _inputs(dtype, M, N, K, 5 + int(bias), act)
    b2 = d["b2"] if (bias and act == "swiglu") else None
    Y, Pre = ops.column_fwd(dev(d["X"]), dev(d["A"]), act, A2=dev(d["A2"]) if act == "swiglu" else None,
                            bias=dev(d["b"]) if bias else None, bias2=dev(b2) if b2 is not None else None)
    torch.cuda.synchronize()
    Yr, Prer = oracle.column_fwd(d["X"].f64, d["A"].f64, act, bias=d["b"].f64 if bias else None,
                                 A2=d["A2"].f64 if act == "swiglu" else None,
                                 bias2=b2.f64 if b2 is not None else None)
    assert_close("Y", host64(Y), Yr, TOL[dtype])
    if act != "none":
        assert_close("Pre", host64(Pre), Prer, TOL[dtype])


# Biases on the fast kernels (K a multiple of 32, 16-byte aligned outputs):
# (512, 512, 256) whole tiles; (300, 200, 64) tiles overhanging rows and
# columns (N a multiple of 8: a lane's bias columns past N start at zero);
# (2048, 768, 256) with no activation takes 128 x 192 tiles.  "up": SwiGLU
# with only the up-projection bias.
@pytest.mark.parametrize("act", ["none", "gelu", "swiglu", "up"])
@pytest.mark.parametrize("shape", [(512, 512, 256), (300, 200, 64), (2048, 768, 256)])
def test_column_fwd_bias_fast_kernels(act, shape):
    M, N, K = shape
    dtype = syn.BF16
    kind = "swiglu" if act == "up" else act
    d = _inputs(dtype, M, N, K, 3 * M + N + ["none", "gelu", "swiglu", "up"].index(act), kind)
    b = None if act == "up" else d["b"]
    b2 = d["b2"] if kind == "swiglu" else None
    Y, Pre = ops.column_fwd(dev(d["X"]), dev(d["A"]), kind, A2=dev(d["A2"]) if kind == "swiglu" else None,
                            bias=dev(b) if b is not None else None, bias2=dev(b2) if b2 is not None else None)
    torch.cuda.synchronize()
    Yr, Prer = oracle.column_fwd(d["X"].f64, d["A"].f64, kind, bias=b.f64 if b is not None else None,
                                 A2=d["A2"].f64 if kind == "swiglu" else None,
                                 bias2=b2.f64 if b2 is not None else None)
    assert_close("Y", host64(Y), Yr, TOL[dtype])
    if kind != "none":
        assert_close("Pre", host64(Pre), Prer, TOL[dtype])


def test_row_bwd_dx_only_half_tile_tail_round():
    # dX = dZ B^T alone (an NT launch): 17 x 17 = 289 whole tiles on 256 CUs, so one launch runs
    # 256 whole tiles and then the last 33 as 66 half tiles of 128 rows.
    M, N, K = 17 * 256, 17 * 256, 64   # row input [M, N], weight [N, K], dZ [M, K]: dX [M, N] over K
    dtype = syn.BF16
    d = _inputs(dtype, M, N, K, 29, "none")
    dX, dB, _ = ops.row_bwd(dev(d["dZ"]), dev(d["dY"]), dev(d["B"]), want_dw=False)
    torch.cuda.synchronize()
    assert dB is None
    rdX, _, _ = oracle.row_bwd(d["dZ"].f64, d["dY"].f64, d["B"].f64)
    assert_close("dX", host64(dX), rdX, TOL[dtype])


@pytest.mark.parametrize("shape", TILE_SHAPES)
def test_row_bwd_whole_tiles(shape):
    M, N, K = shape
    dtype = syn.BF16
    d = _inputs(dtype, M, N, K, 11 + M, "none")
    Xi, Bi = dev(d["dY"]), dev(d["B"])
    dX, dB, _ = ops.row_bwd(dev(d["dZ"]), Xi, Bi)
    torch.cuda.synchronize()
    rdX, rdB, _ = oracle.row_bwd(d["dZ"].f64, d["dY"].f64, d["B"].f64)
    assert_close("dX", host64(dX), rdX, TOL[dtype])
    assert_close("dB", host64(dB), rdB, TOL[dtype])


# Whole-matrix checks of the one-launch row backward in each of its tile
# pairings (shapes in this file's order: X_i [M, N], B_i [N, K], dZ [M, K]),
# on 256 CUs: (768, 8192, 768) takes 256 x 256 tiles for both GEMMs,
# (512, 8192, 512) 192 x 256 weight-gradient tiles beside 256 x 192
# input-gradient tiles (the pairing of the MLP shard step's row backward),
# (512, 256, 768) 192 x 192 beside 128 x 192, (768, 512, 512) 128 x 128
# beside 128 x 192, (1536, 4096, 512) 128 x 128 beside 256 x 256,
# (1024, 4096, 512) 128 x 192 beside 256 x 192 (the pairing of the attention
# projections' backwards), (512, 256, 512) 128 x 192 beside 128 x 192.
@pytest.mark.parametrize("shape,pairing", [((768, 8192, 768), 0), ((512, 8192, 512), 1), ((512, 256, 768), 2),
                                           ((768, 512, 512), 3), ((1536, 4096, 512), 4), ((1024, 4096, 512), 5),
                                           ((512, 256, 512), 6)])
def test_row_bwd_whole_matrix_pairings(shape, pairing):
    M, N, K = shape
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    plan = tp.tp_row_bwd_plan(M, K, N, cus)   # the library's (M, N, K): dZ [M, K], X_i [M, N]
    if cus == 256:
        assert plan == pairing, (plan, pairing)
    dtype = syn.BF16
    d = _inputs(dtype, M, N, K, 41 + pairing, "none")
    Xi, Bi = dev(d["dY"]), dev(d["B"])
    dX, dB, _ = ops.row_bwd(dev(d["dZ"]), Xi, Bi)
    torch.cuda.synchronize()
    rdX, rdB, _ = oracle.row_bwd(d["dZ"].f64, d["dY"].f64, d["B"].f64)
    assert_close("dX", host64(dX), rdX, TOL[dtype])
    assert_close("dB", host64(dB), rdB, TOL[dtype])


# Split contractions: with the workspace of tp_row_bwd_workspace_bytes_split the one-launch
# schedule may cut either product's contraction into parts (fp32 partial planes, then a
# reduction launch).  Shapes in this file's order (X_i [M, N], B_i [N, K], dZ [M, K]); on 256
# CUs the planner cuts (ks_dB, ks_dX) as listed: the weight gradient only, the input gradient
# only, both, in 2 or 4 parts; (8192, 512, 4096) is the attention output projection's backward;
# (1000, 520, 136) has tiles overhanging both outputs.
SPLIT_CASES = [((512, 128, 128), (4, 1)), ((128, 128, 1024), (1, 4)), ((512, 128, 512), (4, 4)),
               ((512, 768, 256), (2, 1)), ((512, 1024, 768), (1, 2)), ((1024, 768, 1024), (2, 2)),
               ((8192, 512, 4096), (4, 2)), ((1000, 520, 136), None)]


@pytest.mark.parametrize("shape,parts", SPLIT_CASES)
def test_row_bwd_split_contraction(shape, parts):
    M, N, K = shape
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    ws = tp.tp_row_bwd_workspace_bytes_split(tp.TP_BF16, M, K, N, cus) - tp.tp_row_bwd_workspace_bytes(tp.TP_BF16, M, K)
    plan, k0, k1 = tp.tp_row_bwd_plan_split(M, K, N, cus, ws)
    if cus == 256 and parts is not None:
        assert (k0, k1) == parts, (plan, k0, k1)
    dtype = syn.BF16
    d = _inputs(dtype, M, N, K, 61 + M + K, "none")
    Xi, Bi = dev(d["dY"]), dev(d["B"])
    dX, dB, _ = ops.row_bwd(dev(d["dZ"]), Xi, Bi, split=True)
    torch.cuda.synchronize()
    rdX, rdB, _ = oracle.row_bwd(d["dZ"].f64, d["dY"].f64, d["B"].f64)
    assert_close("dX", host64(dX), rdX, TOL[dtype])
    assert_close("dB", host64(dB), rdB, TOL[dtype])
    # the same call twice gives the same bits (fixed summation order)
    dX2, dB2, _ = ops.row_bwd(dev(d["dZ"]), Xi, Bi, split=True)
    torch.cuda.synchronize()
    assert torch.equal(dX, dX2) and torch.equal(dB, dB2)


def test_row_bwd_split_with_bias_gradient_and_misaligned_scratch():
    # The bias-gradient column partials sit at the start of the workspace and the split planes after
    # them: both in one call.  Then the same call through a workspace 8 bytes off 16-byte alignment
    # (no bias gradient, which needs an aligned workspace): the schedule must not split, and the
    # results are those of the unsplit launch.
    M, N, K = 512, 128, 512   # this file's order: X_i [M, N], B_i [N, K], dZ [M, K]
    dtype = syn.BF16
    d = _inputs(dtype, M, N, K, 91, "none")
    dZ, Xi, Bi = dev(d["dZ"]), dev(d["dY"]), dev(d["B"])
    dX, dB, db = ops.row_bwd(dZ, Xi, Bi, want_db=True, split=True)
    torch.cuda.synchronize()
    rdX, rdB, rdb = oracle.row_bwd(d["dZ"].f64, d["dY"].f64, d["B"].f64)
    assert_close("dX", host64(dX), rdX, TOL[dtype])
    assert_close("dB", host64(dB), rdB, TOL[dtype])
    assert_close("db", host64(db), rdb, TOL[dtype])
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    n = tp.tp_row_bwd_workspace_bytes_split(tp.TP_BF16, M, K, N, cus)
    raw = torch.empty(n + 64, dtype=torch.uint8, device="cuda")
    off = (16 - raw.data_ptr() % 16) % 16 + 8   # 8 bytes past a 16-byte boundary
    dX2 = torch.empty_like(dX)
    dB2 = torch.empty_like(dB)
    dXu, dBu, _ = ops.row_bwd(dZ, Xi, Bi)     # unsplit reference launch
    tp.tp_row_bwd(tp.TP_BF16, M, K, N, dZ, dZ.stride(0), Xi, Xi.stride(0), Bi, Bi.stride(0), dX2, dX2.stride(0),
                  dB2, dB2.stride(0), None, raw.data_ptr() + off, n)
    torch.cuda.synchronize()
    assert torch.equal(dX2, dXu) and torch.equal(dB2, dBu)


@pytest.mark.parametrize("shape", [(512, 128, 512), (1024, 256, 1024)])
def test_column_bwd_split_contraction(shape):
    # the activation-free column backward's pair of GEMMs with its split workspace (and a bias gradient,
    # whose column partials come first in the workspace)
    M, N, K = shape
    dtype = syn.BF16
    d = _inputs(dtype, M, N, K, 71 + N, "none")
    dX, dA, _, db, _ = ops.column_bwd(dev(d["dY"]), dev(d["X"]), dev(d["A"]), act="none", want_db=True, split=True)
    torch.cuda.synchronize()
    r = oracle.column_bwd(d["dY"].f64, d["X"].f64, d["A"].f64, None, "none", None)
    assert_close("dXpart", host64(dX), r[0], TOL[dtype])
    assert_close("dA", host64(dA), r[1], TOL[dtype])
    assert_close("db", host64(db), r[3], TOL[dtype])


@pytest.mark.parametrize("act", ["none", "swiglu"])
def test_column_bwd_wgrad_narrow_tiles_two_rounds(act):
    # Weight gradient [2560, 7680] (per problem): 300 tiles of 256 x 256 or
    # 400 of 256 x 192 on 256 CUs -- two rounds either way, so the narrow
    # tiles are taken and workgroups run one or two tiles in a row.
    M, N, K = 64, 7680 // (2 if act == "swiglu" else 1), 2560
    dtype = syn.BF16
    d = _inputs(dtype, M, N, K, 23, act)
    sw = act == "swiglu"
    dX, dA, dA2, _, _ = ops.column_bwd(dev(d["dY"]), dev(d["X"]), dev(d["A"]),
                                       Pre=dev(d["Pre"]) if sw else None, act=act, A2=dev(d["A2"]) if sw else None)
    torch.cuda.synchronize()
    r = oracle.column_bwd(d["dY"].f64, d["X"].f64, d["A"].f64, d["Pre"].f64 if sw else None, act,
                          d["A2"].f64 if sw else None)
    assert_close("dXpart", host64(dX), r[0], TOL[dtype])
    assert_close("dA", host64(dA), r[1], TOL[dtype])
    if sw:
        assert_close("dA2", host64(dA2), r[2], TOL[dtype])


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("act", ["none", "gelu", "swiglu"])
def test_column_bwd_ragged(dtype, shape, act):
    M, N, K = shape
    d = _inputs(dtype, M, N, K, 11 + N, act)
    sw = act == "swiglu"
    dX, dA, dA2, db, db2 = ops.column_bwd(dev(d["dY"]), dev(d["X"]), dev(d["A"]),
                                          Pre=dev(d["Pre"]) if act != "none" else None, act=act,
                                          A2=dev(d["A2"]) if sw else None, want_db=True)
    torch.cuda.synchronize()
    r = oracle.column_bwd(d["dY"].f64, d["X"].f64, d["A"].f64, d["Pre"].f64 if act != "none" else None, act,
                          d["A2"].f64 if sw else None)
    assert_close("dXpart", host64(dX), r[0], TOL[dtype])
    assert_close("dA", host64(dA), r[1], TOL[dtype])
    assert_close("db", host64(db), r[3], TOL[dtype])
    if sw:
        assert_close("dA2", host64(dA2), r[2], TOL[dtype])
        assert_close("db2", host64(db2), r[4], TOL[dtype])


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("t", [1, 2, 3, 8])
def test_sum_partials_with_bias_once(dtype, t):
    M, N = 37, 70
    seeded = [syn.normal(50 + i, (M, N), 1.0, dtype) for i in range(t)]
    parts = [dev(p) for p in seeded]
    bias = syn.normal(49, (N,), 1.0, dtype)
    buf, n = ops.stack_partials(parts)
    Z = ops.sum_partials(buf, n, bias=dev(bias))
    Zin = ops.sum_partials(buf, n, out=buf[0, :, :n])      # exact aliasing of part 0 is allowed
    torch.cuda.synchronize()
    ref = oracle.sum_partials([p.f64 for p in seeded], bias=bias.f64)
    assert_close("Z", host64(Z), ref, TOL[dtype])
    assert_close("Z in place", host64(Zin), oracle.sum_partials([p.f64 for p in seeded]), TOL[dtype])


@pytest.mark.parametrize("dtype", DTYPES)
def test_sp_fig2_halves_on_gpu(dtype):
    # Fig. 2 as a reduce-scatter over token rows: rank 0 keeps 1 + 3, rank 1 keeps 2 + 4.
    g = _golden("v4_fig2_allreduce.json")
    parts = [_t(np.array(v, np.float32).reshape(2, 1), dtype) for v in g["gpu_inputs"]]
    buf, n = ops.stack_partials(parts)
    _, h0 = ops.sp_reduce_scatter_ln(buf, n, 0, 1)
    _, h1 = ops.sp_reduce_scatter_ln(buf, n, 1, 1)
    torch.cuda.synchronize()
    _exact(h0, [[g["reduce_scatter"]["gpu0_first_half"]]])
    _exact(h1, [[g["reduce_scatter"]["gpu1_second_half"]]])


# (t, M, N, r0, Mr): one column, ragged widths around the 8-wide vectors and the
# 2048-column chunk steps, the widest row, and rank blocks at both ends.
# (8, 64, 2048, ...) and (3, 20, 4096, ...): bf16 rows of whole chunks take the kernel's
# single-round-trip path (t <= 8 partials, 1 or 2 chunks of 8 columns per thread).
SP_CASES = [(1, 4, 1, 0, 4), (2, 6, 7, 2, 3), (3, 40, 70, 13, 27), (8, 64, 2048, 56, 8), (4, 33, 2049, 0, 11),
            (8, 24, 4100, 8, 8), (2, 9, 8191, 4, 5), (3, 5, 16384, 1, 3), (8, 16, 12345, 15, 1),
            (3, 20, 4096, 5, 7)]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("t,M,N,r0,Mr", SP_CASES)
def test_sp_reduce_scatter_ln_small(dtype, t, M, N, r0, Mr):
    seed = 7 * t + M + N
    seeded = [syn.normal(seed + i, (M, N), 1.0, dtype) for i in range(t)]
    bias = syn.normal(seed + 100, (N,), 0.5, dtype)
    resid = syn.normal(seed + 101, (Mr, N), 2.0, dtype)
    gamma = syn.normal(seed + 102, (N,), 1.0, dtype)
    beta = syn.normal(seed + 103, (N,), 0.5, dtype)
    buf, n = ops.stack_partials([dev(p) for p in seeded])
    y, h = ops.sp_reduce_scatter_ln(buf, n, r0, Mr, dev(bias), dev(resid), dev(gamma), dev(beta), eps=1e-5)
    y0, _ = ops.sp_reduce_scatter_ln(buf, n, r0, Mr, want_h=False)
    torch.cuda.synchronize()
    ry, rh = oracle.sp_reduce_scatter_ln([p.f64 for p in seeded], r0, Mr, bias.f64, resid.f64, gamma.f64, beta.f64,
                                         1e-5)
    assert_close("h", host64(h), rh, TOL[dtype])
    assert_close("y", host64(y), ry, TOL[dtype])
    ry0, _ = oracle.sp_reduce_scatter_ln([p.f64 for p in seeded], r0, Mr)
    assert_close("y (no bias/resid/gamma/beta)", host64(y0), ry0, TOL[dtype])


@pytest.mark.parametrize("dtype", DTYPES)
def test_sp_flow_reduce_scatter_gather_column(dtype):
    # The SP forward between two blocks: row partials -> each rank's block (+bias +resid,
    # LayerNorm) -> all-gather (a concatenation on one device) -> next column-parallel GEMM.
    t, M, N, Nc = 4, 96, 136, 40
    Mr = M // t
    seeded = [syn.normal(90 + i, (M, N), 1.0, dtype) for i in range(t)]
    bias = syn.normal(95, (N,), 0.5, dtype)
    resid = syn.normal(96, (M, N), 1.0, dtype)
    gamma = syn.normal(97, (N,), 1.0, dtype)
    beta = syn.normal(98, (N,), 0.5, dtype)
    A = syn.normal(99, (N, Nc), 0.2, dtype)
    buf, n = ops.stack_partials([dev(p) for p in seeded])
    R = dev(resid)
    ys = [ops.sp_reduce_scatter_ln(buf, n, r * Mr, Mr, dev(bias), R[r * Mr:(r + 1) * Mr], dev(gamma), dev(beta),
                                   eps=1e-5)[0] for r in range(t)]
    gathered = torch.cat(ys, dim=0)
    Y, _ = ops.column_fwd(gathered, dev(A))
    torch.cuda.synchronize()
    full = oracle.sum_partials([p.f64 for p in seeded], bias=bias.f64) + resid.f64
    ref_y = oracle.layer_norm(full, gamma.f64, beta.f64, 1e-5)
    assert_close("gathered y", host64(gathered), ref_y, TOL[dtype])
    assert_close("column after gather", host64(Y), oracle.column_fwd(ref_y, A.f64)[0], TOL[dtype])


def test_sp_reduce_scatter_ln_in_place_and_constant_rows():
    dtype = syn.BF16
    t, M, N, r0, Mr = 4, 12, 1000, 4, 4
    seeded = [syn.normal(60 + i, (M, N), 1.0, dtype) for i in range(t)]
    resid = syn.normal(65, (Mr, N), 1.0, dtype)
    buf, n = ops.stack_partials([dev(p) for p in seeded])
    r = ops.aligned(dev(resid))
    y, h = ops.sp_reduce_scatter_ln(buf, n, r0, Mr, resid=r, eps=1e-5, h_inplace=True)
    torch.cuda.synchronize()
    ry, rh = oracle.sp_reduce_scatter_ln([p.f64 for p in seeded], r0, Mr, resid=resid.f64, eps=1e-5)
    assert h.data_ptr() == r.data_ptr()
    assert_close("h in place", host64(r), rh, TOL[dtype])
    assert_close("y", host64(y), ry, TOL[dtype])
    # rows whose sum is constant: variance 0, so the output is beta exactly
    const = [syn.from_values(np.full((2, 24), v, np.float32), dtype) for v in (1.5, -0.25)]
    beta = syn.normal(66, (24,), 1.0, dtype)
    buf, n = ops.stack_partials([dev(p) for p in const])
    y, _ = ops.sp_reduce_scatter_ln(buf, n, 0, 2, beta=dev(beta), eps=1e-5)
    torch.cuda.synchronize()
    _exact(y, np.broadcast_to(beta.f64, (2, 24)))


# (2048, 18992, 40): 600 logit tiles on 256 CUs -- workgroups run two or three
# tiles in a row, and the last 88 tiles run as 176 half tiles; (2000, ...):
# the same without the half tiles (M not a multiple of 256), rows past M masked.
# K % 32 != 0 takes the kernels' K-tail variant, K % 32 == 0 the other one
# ((2048, 18992, 64): half tiles without a K tail).
@pytest.mark.parametrize("M,Vr,K", [(1, 1, 8), (37, 300, 72), (300, 600, 136), (260, 18992, 64),
                                    (2048, 18992, 40), (2048, 18992, 64), (2000, 18992, 72)])
def test_vocab_ce_small(M, Vr, K):
    rng = np.random.default_rng(M + Vr)
    H = syn.normal(70 + M, (M, K), 1.0, syn.BF16)
    W = syn.normal(71 + Vr, (Vr, K), 0.3, syn.BF16)
    v0 = 1000
    target = rng.integers(v0 - 50, v0 + Vr + 50, size=M).astype(np.int32)
    target[: min(M, 3)] = [v0, v0 + Vr - 1, -5][: min(M, 3)]
    m, s, tg = ops.vocab_ce_partials(dev(H), dev(W), torch.from_numpy(target).cuda(), v0)
    torch.cuda.synchronize()
    rm, rs, rt = oracle.vocab_ce_partials(H.f64, W.f64, target, v0)
    gl, gt, gloss = oracle.lse_recombine([(host64(m), host64(s), host64(tg))])
    rl, rt2, rloss = oracle.lse_recombine([(rm, rs, rt)])
    assert_close("lse", gl, rl, 1e-3)
    assert_close("tgt", gt, rt2, 1e-3)
    assert_close("loss", gloss, rloss, 1e-3)
    owned = (target >= v0) & (target < v0 + Vr)
    assert np.all(host64(tg)[~owned] == 0.0)


@pytest.mark.parametrize("M,Vr,K,use_g", [(1, 1, 8, False), (37, 300, 72, True), (300, 600, 136, False),
                                           (260, 1000, 64, True), (512, 768, 256, True)])
def test_vocab_ce_bwd_small(M, Vr, K, use_g):
    rng = np.random.default_rng(3 * M + Vr)
    H = syn.normal(80 + M, (M, K), 1.0, syn.BF16)
    W = syn.normal(81 + Vr, (Vr, K), 0.3, syn.BF16)
    v0 = 500
    target = rng.integers(v0 - 50, v0 + Vr + 50, size=M).astype(np.int32)
    target[: min(M, 3)] = [v0, v0 + Vr - 1, -5][: min(M, 3)]
    lse, _, _ = oracle.lse_recombine([oracle.vocab_ce_partials(H.f64, W.f64, target, v0)])
    lse32 = lse.astype(np.float32)
    g32 = syn.normal(82 + M, (M,), 1.0, syn.FP32).f32 if use_g else None
    dH, dW = ops.vocab_ce_bwd(dev(H), dev(W), torch.from_numpy(target).cuda(), v0, torch.from_numpy(lse32).cuda(),
                              torch.from_numpy(g32).cuda() if use_g else None)
    torch.cuda.synchronize()
    _, rdH, rdW = oracle.vocab_ce_bwd(H.f64, W.f64, target, v0, lse32, g32)
    assert_close("dH", host64(dH), rdH, TOL[syn.BF16])
    assert_close("dW", host64(dW), rdW, TOL[syn.BF16])


@pytest.mark.parametrize("R,M", [(1, 1), (3, 37), (8, 1000), (8, 8192)])
def test_vocab_ce_combine_small(R, M):
    # Seeded shard triples (max, sumexp >= 1, tgt); shard r owns token m's target
    # when m % R == r, the others report 0.  The device combine is fp64 with one
    # rounding to fp32, so it must agree with the float64 oracle to fp32 rounding.
    rng = np.random.default_rng(10 * R + M)
    mx = (rng.standard_normal((R, M)) * 3.0).astype(np.float32)
    se = (1.0 + rng.random((R, M)) * 5000.0).astype(np.float32)
    tg = np.zeros((R, M), dtype=np.float32)
    own = np.arange(M) % R
    tg[own, np.arange(M)] = (rng.standard_normal(M) * 2.0).astype(np.float32)
    mx[:, : min(M, 2)] = 1e4 if R == 1 else mx[:, : min(M, 2)]        # large maxima: no overflow
    lse, tgt, loss = ops.vocab_ce_combine(torch.from_numpy(mx).cuda(), torch.from_numpy(se).cuda(),
                                          torch.from_numpy(tg).cuda())
    torch.cuda.synchronize()
    rl, rt, rloss = oracle.lse_recombine([(mx[r], se[r], tg[r]) for r in range(R)])
    assert_close("lse", host64(lse), rl, 1e-6)
    assert_close("tgt", host64(tgt), rt, 1e-6)
    assert_close("loss", host64(loss), rloss, 1e-6)


def test_vocab_ce_chain_eight_shards_on_gpu_outputs():
    # The whole vocab-parallel CE path with every intermediate made on the GPU:
    # 8 shards' partials -> device recombination (lse) -> each shard's backward on
    # that lse -> dH summed over the shards (the all-reduce of the partial dH).
    # Shards of 2000 vocab rows (7 whole 256-column tiles and a ragged one).
    R, M, Vr, K = 8, 1024, 2000, 1024
    H = syn.normal(9100, (M, K), 1.0, syn.BF16)
    Ws = [syn.normal(9110 + r, (Vr, K), 0.05, syn.BF16) for r in range(R)]
    target = np.random.default_rng(9120).integers(0, R * Vr, size=M).astype(np.int32)
    g = syn.normal(9121, (M,), 1.0, syn.FP32).f32
    Hd, td, gd = dev(H), torch.from_numpy(target).cuda(), torch.from_numpy(g).cuda()
    parts = [ops.vocab_ce_partials(Hd, dev(Ws[r]), td, r * Vr) for r in range(R)]
    lse, tgt, loss = ops.vocab_ce_combine([p[0] for p in parts], [p[1] for p in parts], [p[2] for p in parts])
    dHs, dWs = [], []
    for r in range(R):
        dH, dW = ops.vocab_ce_bwd(Hd, dev(Ws[r]), td, r * Vr, lse, gd)
        dHs.append(dH)
        dWs.append(dW)
    buf, n = ops.stack_partials(dHs)
    dHsum = ops.sum_partials(buf, n)
    torch.cuda.synchronize()
    rparts = [oracle.vocab_ce_partials(H.f64, Ws[r].f64, target, r * Vr) for r in range(R)]
    rl, rt, rloss = oracle.lse_recombine(rparts)
    assert_close("lse", host64(lse), rl, 1e-3)
    assert_close("tgt", host64(tgt), rt, 1e-3)
    assert_close("loss", host64(loss), rloss, 1e-3)
    rdH = np.zeros((M, K))
    for r in range(R):
        _, rdHr, rdWr = oracle.vocab_ce_bwd(H.f64, Ws[r].f64, target, r * Vr, rl, g)
        rdH += rdHr
        assert_close(f"dW shard {r}", host64(dWs[r]), rdWr, TOL[syn.BF16])
    assert_close("dH summed", host64(dHsum), rdH, TOL[syn.BF16])


def _ids_dev(ids):
    return torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).cuda()


# (M, Vr, K, v0, kind): one row and one token, ragged widths, several 256-row blocks and
# 256-token chunks, ids all owned / none owned / heavily repeated.
EMB_CASES = [(1, 1, 8, 0, "uniform"), (5, 3, 7, 10, "uniform"), (300, 700, 136, 500, "uniform"),
             (1000, 300, 13, 0, "repeated"), (777, 1030, 4100, 2000, "uniform"), (513, 257, 64, 50, "none"),
             (2048, 600, 72, 0, "all")]


def _emb_ids(M, Vr, v0, kind, seed):
    rng = np.random.default_rng(seed)
    if kind == "none":
        return rng.integers(v0 + Vr, v0 + Vr + 1000, size=M).astype(np.int32)
    if kind == "all":
        return rng.integers(v0, v0 + Vr, size=M).astype(np.int32)
    ids = rng.integers(v0 - 2 * Vr, v0 + 3 * Vr, size=M).astype(np.int32)
    if kind == "repeated":                                   # half the tokens on two rows
        ids[rng.random(M) < 0.5] = v0 + min(Vr - 1, 5)
        ids[::7] = v0
    ids[: min(M, 3)] = [v0, v0 + Vr - 1, -1][: min(M, 3)]
    return ids


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("M,Vr,K,v0,kind", EMB_CASES)
def test_vocab_embed_fwd_bwd_small(dtype, M, Vr, K, v0, kind):
    seed = M + 3 * Vr + K
    ids = _emb_ids(M, Vr, v0, kind, seed)
    E = syn.normal(seed + 1, (Vr, K), 1.0, dtype)
    dout = syn.normal(seed + 2, (M, K), 1.0, dtype)
    out = ops.vocab_embed_fwd(_ids_dev(ids), dev(E), v0)
    dE = ops.vocab_embed_bwd(_ids_dev(ids), dev(dout), v0, Vr)
    dE2 = ops.vocab_embed_bwd(_ids_dev(ids), dev(dout), v0, Vr)
    torch.cuda.synchronize()
    _exact(out, oracle.vocab_embed_fwd(ids, E.f64, v0))          # rows copied bit for bit
    assert_close("dE", host64(dE), oracle.vocab_embed_bwd(ids, dout.f64, v0, Vr), TOL[dtype])
    assert torch.equal(dE.cpu(), dE2.cpu())                        # fixed summation order


def test_vocab_embed_shards_sum_to_full_lookup_on_gpu():
    # t = 4 ranks' lookups summed (the all-reduce on one device) give every token its own row.
    t, Vr, K, M = 4, 250, 72, 600
    E = syn.normal(77, (t * Vr, K), 1.0, syn.BF16)
    ids = np.random.default_rng(78).integers(0, t * Vr, size=M).astype(np.int32)
    Ed = dev(E)
    parts = [ops.vocab_embed_fwd(_ids_dev(ids), Ed[r * Vr:(r + 1) * Vr], r * Vr) for r in range(t)]
    buf, n = ops.stack_partials(parts)
    Z = ops.sum_partials(buf, n)
    torch.cuda.synchronize()
    _exact(Z, np.take(E.f64, ids, axis=0))


# (B, S, n_q, n_kv, causal): one token, ragged tails of the 64-key tiles and 32-row blocks,
# GQA groups 4 / 2 / 1 / 8, several sequences.
ATTN_CASES = [(1, 1, 1, 1, True), (1, 37, 4, 1, True), (1, 64, 4, 1, False), (1, 200, 4, 1, True),
              (1, 300, 2, 1, True), (1, 130, 2, 2, False), (1, 256, 8, 1, True), (3, 100, 4, 1, True),
              (2, 129, 4, 1, False), (1, 1100, 4, 1, True), (1, 2100, 2, 1, True), (2, 700, 8, 2, False)]
# (causal ranges beyond 1024 keys and short non-causal ones are cut into chunks merged afterwards)


@pytest.mark.parametrize("B,S,n_q,n_kv,causal", ATTN_CASES)
def test_attention_fwd_small(B, S, n_q, n_kv, causal):
    seed = 11 * S + n_q + 3 * B
    width = 128 * (n_q + 2 * n_kv)
    qkv = syn.normal(seed, (B * S, width), 1.0, syn.BF16)       # packed [q heads | k | v] like the QKV output
    d = dev(qkv)
    q, k, v = d[:, :128 * n_q], d[:, 128 * n_q:128 * (n_q + n_kv)], d[:, 128 * (n_q + n_kv):]
    O, lse = ops.attention_fwd(q, k, v, n_q, n_kv, causal=causal, B=B)
    torch.cuda.synchronize()
    X = qkv.f64
    for b in range(B):
        rs = slice(b * S, (b + 1) * S)
        ro, rl = oracle.attention_fwd(X[rs, :128 * n_q], X[rs, 128 * n_q:128 * (n_q + n_kv)],
                                      X[rs, 128 * (n_q + n_kv):], n_q, n_kv, causal=causal)
        assert_close(f"O seq {b}", host64(O[rs]), ro, TOL[syn.BF16])
        assert_close(f"lse seq {b}", host64(lse[b]), rl, 1e-3)


ATTN_BWD_CASES = [(1, 1, 1, 1, True), (1, 37, 4, 1, True), (1, 200, 4, 1, True), (1, 300, 2, 1, True),
                  (1, 130, 2, 2, False), (1, 256, 8, 1, True), (2, 100, 4, 1, True), (1, 1100, 4, 1, True),
                  (1, 2200, 4, 1, True), (2, 700, 8, 2, False), (1, 2300, 4, 1, False)]
# (beyond 1024 keys the dQ pass is cut into key chunks; beyond 2048 queries the dK/dV pass into
# query chunks, whole chunks launched before the shorter last ones)


@pytest.mark.parametrize("B,S,n_q,n_kv,causal", ATTN_BWD_CASES)
def test_attention_bwd_small(B, S, n_q, n_kv, causal):
    seed = 13 * S + n_q + 5 * B
    width = 128 * (n_q + 2 * n_kv)
    qkv = syn.normal(seed, (B * S, width), 1.0, syn.BF16)
    dO = syn.normal(seed + 1, (B * S, 128 * n_q), 1.0, syn.BF16)
    d = dev(qkv)
    q, k, v = d[:, :128 * n_q], d[:, 128 * n_q:128 * (n_q + n_kv)], d[:, 128 * (n_q + n_kv):]
    O, lse = ops.attention_fwd(q, k, v, n_q, n_kv, causal=causal, B=B)
    dq, dk, dv = ops.attention_bwd(q, k, v, O, lse, dev(dO), n_q, n_kv, causal=causal, B=B)
    dq2, dk2, dv2 = ops.attention_bwd(q, k, v, O, lse, dev(dO), n_q, n_kv, causal=causal, B=B)
    torch.cuda.synchronize()
    X, G = qkv.f64, dO.f64
    for b in range(B):
        rs = slice(b * S, (b + 1) * S)
        rq, rk, rv = oracle.attention_bwd(X[rs, :128 * n_q], X[rs, 128 * n_q:128 * (n_q + n_kv)],
                                          X[rs, 128 * (n_q + n_kv):], G[rs], n_q, n_kv, causal=causal)
        assert_close(f"dQ seq {b}", host64(dq[rs]), rq, TOL[syn.BF16])
        assert_close(f"dK seq {b}", host64(dk[rs]), rk, TOL[syn.BF16])
        assert_close(f"dV seq {b}", host64(dv[rs]), rv, TOL[syn.BF16])
    for x, y in ((dq, dq2), (dk, dk2), (dv, dv2)):                  # fixed summation order
        assert torch.equal(x.cpu(), y.cpu())


def test_deterministic_bitwise():
    d = _inputs(syn.BF16, 520, 300, 1030, 3, "swiglu")
    outs = []
    for _ in range(2):
        Y, Pre = ops.column_fwd(dev(d["X"]), dev(d["A"]), "swiglu", A2=dev(d["A2"]))
        dX, dA, dA2, _, _ = ops.column_bwd(dev(d["dY"]), dev(d["X"]), dev(d["A"]), Pre=dev(d["Pre"]),
                                           act="swiglu", A2=dev(d["A2"]))
        torch.cuda.synchronize()
        outs.append([x.cpu() for x in (Y, Pre, dX, dA, dA2)])
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
