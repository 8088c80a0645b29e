"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times.  Outputs too large for the float64 oracle are checked on
sampled rows / columns that the oracle computes one by one (the sample always
includes the first and last index and tile edges)."""
import numpy as np
import pytest

import oracle
import synthetic as syn

from .gpu_util import TOL, TOL_CE, assert_close, cols, dev, host64, rows, sample_idx, tile_sample_idx

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
ops = pytest.importorskip("tensor_transformer_linear_tp_amd.torch_ops")
tp = pytest.importorskip("tensor_transformer_linear_tp_amd")

BF = TOL[syn.BF16]


# ---------------------------------------------------------------------------
# c1: fp32 GeLU MLP, t shards of one full weight, with and without bias,
# against the unsharded layer (the pages' self-test recipe).
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("t", [1, 2, 4])
@pytest.mark.parametrize("bias", [False, True])
@pytest.mark.parametrize("dtype", [syn.FP32, syn.BF16])
def test_c1_sharded_mlp_matches_unsharded(t, bias, dtype):
    cfg = syn.C1
    M, H, F = cfg.M, cfg.H, cfg.F
    s = cfg.seed + 100
    X = syn.normal(s + 1, (M, H), 1.0, dtype)
    A = syn.normal(s + 2, (H, F), cfg.std_w, dtype)
    B = syn.normal(s + 3, (F, H), cfg.std_w, dtype)
    dZ = syn.normal(s + 4, (M, H), 1.0, dtype)
    bA = syn.normal(s + 5, (F,), 0.5, dtype) if bias else None
    bB = syn.normal(s + 6, (H,), 0.5, dtype) if bias else None

    Xd, dZd = dev(X), dev(dZ)
    Ad, Bd = dev(A), dev(B)
    zparts, dxparts, dAs, dBs, dbs = [], [], [], [], []
    dbrow = None
    for i in range(t):
        cs = oracle.column_slice(F, t, i)
        Y, Pre = ops.column_fwd(Xd, Ad[:, cs], "gelu", bias=dev(bA)[cs] if bias else None)
        zparts.append(ops.row_fwd(Y, Bd[cs, :]))
        dY, dB, db_row = ops.row_bwd(dZd, Y, Bd[cs, :], want_db=bias)
        dX, dA, _, db, _ = ops.column_bwd(dY, Xd, Ad[:, cs], Pre=Pre, act="gelu", want_db=bias)
        dxparts.append(dX)
        dAs.append(dA)
        dBs.append(dB)
        dbs.append(db)
        dbrow = db_row
    buf, N = ops.stack_partials(zparts)
    Z = ops.sum_partials(buf, N, bias=dev(bB) if bias else None)
    buf2, N2 = ops.stack_partials(dxparts)
    dXs = ops.sum_partials(buf2, N2)
    torch.cuda.synchronize()

    # Unsharded reference (t = 1 of the oracle).
    Yr, Pr = oracle.column_fwd(X.f64, A.f64, "gelu", bias=bA.f64 if bias else None)
    Zr = oracle.sum_partials([oracle.row_fwd(Yr, B.f64)], bias=bB.f64 if bias else None)
    dYr, dBr, dbrow_r = oracle.row_bwd(dZ.f64, Yr, B.f64)
    dXr, dAr, _, dbr, _ = oracle.column_bwd(dYr, X.f64, A.f64, Pr, "gelu")
    tol = TOL[dtype]
    assert_close("Z", host64(Z), Zr, tol)
    assert_close("dX", host64(dXs), dXr, tol)
    assert_close("dA", np.concatenate([host64(a) for a in dAs], axis=1), dAr, tol)
    assert_close("dB", np.concatenate([host64(b) for b in dBs], axis=0), dBr, tol)
    if bias:
        assert_close("db_col", np.concatenate([host64(b) for b in dbs]), dbr, tol)
        assert_close("db_row", host64(dbrow), dbrow_r, tol)


# ---------------------------------------------------------------------------
# c2: Qwen3-8B-shaped SwiGLU shard, t = 8.
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def c2():
    return syn.mlp_shard_inputs(syn.C2, shard=0)


def test_c2_shard_chain_sampled(c2):
    cfg = syn.C2
    X, A, A2, B, dZ = (c2[k] for k in ("X", "A", "A2", "B", "dZ"))
    Xd, Ad, A2d, Bd, dZd = (dev(c2[k]) for k in ("X", "A", "A2", "B", "dZ"))
    Y, Pre = ops.column_fwd(Xd, Ad, "swiglu", A2=A2d)
    Z = ops.row_fwd(Y, Bd)
    dY, dB, _ = ops.row_bwd(dZd, Y, Bd)
    dX, dA, dA2, _, _ = ops.column_bwd(dY, Xd, Ad, Pre=Pre, act="swiglu", A2=A2d)
    torch.cuda.synchronize()

    ms = tile_sample_idx(cfg.M, 256, 1, per_tile=2)    # token rows: two in every 256-row tile
    ks = tile_sample_idx(cfg.Fi, 192, 2, per_tile=2)   # intermediate columns: two per 192-wide tile
    Xf, Af, A2f, Bf, dZf = X.f64, A.f64, A2.f64, B.f64, dZ.f64
    # forward rows
    Yr, Prer = oracle.column_fwd(Xf[ms], Af, "swiglu", A2=A2f)
    assert_close("Y rows", rows(Y, ms), Yr, BF)
    assert_close("Pre rows", rows(Pre, ms), Prer, BF)
    assert_close("Z rows", rows(Z, ms), oracle.row_fwd(Yr, Bf), BF)
    # backward rows: dY, dX_part
    dYr = oracle.dgrad(dZf[ms], Bf)
    assert_close("dY rows", rows(dY, ms), dYr, BF)
    dXr = oracle.column_bwd(dYr, Xf[ms], Af, Prer, "swiglu", A2f)[0]
    assert_close("dXpart rows", rows(dX, ms), dXr, BF)
    # weight gradients on sampled intermediate columns (reductions over all tokens)
    Yk, Prek = oracle.column_fwd(Xf, Af[:, ks], "swiglu", A2=A2f[:, ks])
    assert_close("dB rows", rows(dB, ks), oracle.wgrad(Yk, dZf), BF)
    dYk = oracle.dgrad(dZf, Bf[ks, :])
    _, dAk, dA2k, _, _ = oracle.column_bwd(dYk, Xf, Af[:, ks], Prek, "swiglu", A2f[:, ks])
    assert_close("dA cols", cols(dA, ks), dAk, BF)
    assert_close("dA2 cols", cols(dA2, ks), dA2k, BF)


def test_c2_per_call_sampled(c2):
    """Each call on its own seeded inputs (none taken from another GPU call)."""
    cfg = syn.C2
    M, H, Fi = cfg.M, cfg.H, cfg.Fi
    Yin = syn.normal(2900, (M, Fi), 1.0, syn.BF16)
    dYin = syn.normal(2901, (M, Fi), 1.0, syn.BF16)
    Pin = syn.normal(2902, (M, 2 * Fi), 1.0, syn.BF16)
    X, A, A2, B, dZ = (c2[k] for k in ("X", "A", "A2", "B", "dZ"))
    Z = ops.row_fwd(dev(Yin), dev(B))
    dYo, dB, db = ops.row_bwd(dev(dZ), dev(Yin), dev(B), want_db=True)
    dX, dA, dA2, dbg, dbu = ops.column_bwd(dev(dYin), dev(X), dev(A), Pre=dev(Pin), act="swiglu", A2=dev(A2),
                                           want_db=True)
    torch.cuda.synchronize()
    ms = tile_sample_idx(M, 256, 3, per_tile=2)
    ks = tile_sample_idx(Fi, 192, 4, per_tile=2)
    ns = tile_sample_idx(H, 256, 5, per_tile=2)
    assert_close("Z", rows(Z, ms), oracle.row_fwd(Yin.f64[ms], B.f64), BF)
    assert_close("dY", rows(dYo, ms), oracle.dgrad(dZ.f64[ms], B.f64), BF)
    assert_close("dB", cols(dB, ns), oracle.wgrad(Yin.f64, dZ.f64[:, ns]), BF)
    assert_close("db_row", host64(db), dZ.f64.sum(axis=0), BF)
    P = Pin.f64
    r = oracle.column_bwd(dYin.f64[ms], X.f64[ms], A.f64, P[ms], "swiglu", A2.f64)
    assert_close("dXpart", rows(dX, ms), r[0], BF)
    Pk = np.concatenate([P[:, ks], P[:, Fi + ks]], axis=1)
    r = oracle.column_bwd(dYin.f64[:, ks], X.f64, A.f64[:, ks], Pk, "swiglu", A2.f64[:, ks])
    assert_close("dA", cols(dA, ks), r[1], BF)
    assert_close("dA2", cols(dA2, ks), r[2], BF)
    assert_close("db_gate", rows(dbg, ks), r[3], BF)
    assert_close("db_up", rows(dbu, ks), r[4], BF)


# ---------------------------------------------------------------------------
# c3: attention projection shard (QKV column, W_O row), t = 8.
# ---------------------------------------------------------------------------

def test_c3_attention_projections_sampled():
    cfg = syn.C3
    d = syn.attn_proj_inputs(cfg)
    QKV, _ = ops.column_fwd(dev(d["X"]), dev(d["Wqkv"]), "none")
    Z = ops.row_fwd(dev(d["attn"]), dev(d["Wo"]))
    dAttn, dWo, _ = ops.row_bwd(dev(d["dZ"]), dev(d["attn"]), dev(d["Wo"]))
    dX, dWqkv, _, _, _ = ops.column_bwd(dev(d["dQKV"]), dev(d["X"]), dev(d["Wqkv"]), act="none")
    torch.cuda.synchronize()
    ms = tile_sample_idx(cfg.M, 128, 6, per_tile=2)   # the narrow launches use 128-row tiles
    X, Wqkv, attn, Wo, dZ, dQKV = (d[k].f64 for k in ("X", "Wqkv", "attn", "Wo", "dZ", "dQKV"))
    assert_close("QKV", rows(QKV, ms), oracle.column_fwd(X[ms], Wqkv)[0], BF)
    assert_close("Z", rows(Z, ms), oracle.row_fwd(attn[ms], Wo), BF)
    assert_close("dAttn", rows(dAttn, ms), oracle.dgrad(dZ[ms], Wo), BF)
    ns = tile_sample_idx(cfg.H, 192, 7, per_tile=2)
    assert_close("dWo", cols(dWo, ns), oracle.wgrad(attn, dZ[:, ns]), BF)
    assert_close("dX", rows(dX, ms), oracle.dgrad(dQKV[ms], Wqkv), BF)
    assert_close("dWqkv", host64(dWqkv), oracle.wgrad(X, dQKV), BF)


def test_c3_attention_projection_backwards_split_sampled():
    # The backward calls as the bench makes them: with the workspace of their split-contraction
    # schedules (on 256 CUs, 256 x 256 tiles: the W_O backward cuts dW's 8192-token contraction into
    # 4 parts and dX's 4096 into 2; the QKV backward cuts dW's 8192-token contraction into 2).
    cfg = syn.C3
    d = syn.attn_proj_inputs(cfg)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if cus == 256:
        M, H, Na = cfg.M, d["Wo"].shape[1], d["Wo"].shape[0]
        need = tp.tp_row_bwd_workspace_bytes_split(tp.TP_BF16, M, H, Na, cus) - tp.tp_row_bwd_workspace_bytes(
            tp.TP_BF16, M, H)
        assert tp.tp_row_bwd_plan_split(M, H, Na, cus, need) == (0, 4, 2)
        Nq = d["Wqkv"].shape[1]   # the column backward's pair has the row backward's structure
        assert tp.tp_row_bwd_plan_split(M, Nq, H, cus, 1 << 40) == (0, 2, 1)
    dAttn, dWo, _ = ops.row_bwd(dev(d["dZ"]), dev(d["attn"]), dev(d["Wo"]), split=True)
    dX, dWqkv, _, _, _ = ops.column_bwd(dev(d["dQKV"]), dev(d["X"]), dev(d["Wqkv"]), act="none", split=True)
    torch.cuda.synchronize()
    ms = tile_sample_idx(cfg.M, 256, 6, per_tile=2)
    X, Wqkv, attn, Wo, dZ, dQKV = (d[k].f64 for k in ("X", "Wqkv", "attn", "Wo", "dZ", "dQKV"))
    assert_close("dAttn", rows(dAttn, ms), oracle.dgrad(dZ[ms], Wo), BF)
    ns = tile_sample_idx(d["Wo"].shape[1], 256, 7, per_tile=2)
    assert_close("dWo", cols(dWo, ns), oracle.wgrad(attn, dZ[:, ns]), BF)
    assert_close("dX", rows(dX, ms), oracle.dgrad(dQKV[ms], Wqkv), BF)
    assert_close("dWqkv", host64(dWqkv), oracle.wgrad(X, dQKV), BF)


# ---------------------------------------------------------------------------
# c4: GeLU shard at h = 8192, t = 4, and the 4-way partial sum.
# ---------------------------------------------------------------------------

def test_c4_gelu_shard_sampled():
    cfg = syn.C4
    d = syn.mlp_shard_inputs(cfg, shard=0)
    M, H, Fi = cfg.M, cfg.H, cfg.Fi
    Yin = syn.normal(4900, (M, Fi), 1.0, syn.BF16)
    Pin = syn.normal(4901, (M, Fi), 1.0, syn.BF16)
    dYin = syn.normal(4902, (M, Fi), 1.0, syn.BF16)
    X, A, B, dZ = (d[k] for k in ("X", "A", "B", "dZ"))
    Y, Pre = ops.column_fwd(dev(X), dev(A), "gelu")
    Z = ops.row_fwd(dev(Yin), dev(B))
    dYo, dB, _ = ops.row_bwd(dev(dZ), dev(Yin), dev(B))
    dX, dA, _, _, _ = ops.column_bwd(dev(dYin), dev(X), dev(A), Pre=dev(Pin), act="gelu")
    torch.cuda.synchronize()
    ms = tile_sample_idx(M, 256, 8, per_tile=2)
    ks = tile_sample_idx(Fi, 256, 9, per_tile=1)
    ns = tile_sample_idx(H, 256, 10, per_tile=1)
    Yr, Pr = oracle.column_fwd(X.f64[ms], A.f64, "gelu")
    assert_close("Y", rows(Y, ms), Yr, BF)
    assert_close("Pre", rows(Pre, ms), Pr, BF)
    assert_close("Z", rows(Z, ms), oracle.row_fwd(Yin.f64[ms], B.f64), BF)
    assert_close("dY", rows(dYo, ms), oracle.dgrad(dZ.f64[ms], B.f64), BF)
    assert_close("dB", cols(dB, ns), oracle.wgrad(Yin.f64, dZ.f64[:, ns]), BF)
    r = oracle.column_bwd(dYin.f64[ms], X.f64[ms], A.f64, Pin.f64[ms], "gelu")
    assert_close("dXpart", rows(dX, ms), r[0], BF)
    r = oracle.column_bwd(dYin.f64[:, ks], X.f64, A.f64[:, ks], Pin.f64[:, ks], "gelu")
    assert_close("dA", cols(dA, ks), r[1], BF)


def test_c4_four_shards_real_partials_summed():
    # The pages' self-test at c4's full size: the 4 shards of one full weight
    # (A = [A_0 .. A_3] [8192, 32768], B = [B_0; ..; B_3]) each run the GeLU
    # column forward and the row forward on the GPU; tp_sum_partials adds their
    # real bf16 partials, compared on tile-sampled token rows with the unsharded
    # layer GeLU(X A) B of the oracle.
    cfg = syn.C4
    shards = [syn.mlp_shard_inputs(cfg, shard=i) for i in range(cfg.t)]
    X = shards[0]["X"]
    Xd = dev(X)
    zparts = []
    for d in shards:
        Y, _ = ops.column_fwd(Xd, dev(d["A"]), "gelu")
        zparts.append(ops.row_fwd(Y, dev(d["B"])))
        del Y
    buf, N = ops.stack_partials(zparts)
    del zparts
    Z = ops.sum_partials(buf, N)
    torch.cuda.synchronize()
    ms = tile_sample_idx(cfg.M, 256, 11, per_tile=2)
    Afull = np.concatenate([d["A"].f64 for d in shards], axis=1)
    Yr, _ = oracle.column_fwd(X.f64[ms], Afull, "gelu")
    del Afull
    Bfull = np.concatenate([d["B"].f64 for d in shards], axis=0)
    assert_close("Z", rows(Z, ms), oracle.row_fwd(Yr, Bfull), BF)


def test_c2_all_eight_shards_chain_vs_unsharded():
    # The pages' self-test at c2's full size: the 8 shards of one full SwiGLU MLP
    # (gate/up [4096, 12288], down [12288, 4096]) run the whole shard chain on the
    # GPU; the forward partials and the input-gradient partials are summed with
    # tp_sum_partials, the weight gradients are concatenated; everything is
    # compared with the unsharded layer of the oracle (token rows: two in every
    # 256-row tile; weight columns/rows: two in every 192-wide tile of each shard).
    cfg = syn.C2
    t, M, H, Fi = cfg.t, cfg.M, cfg.H, cfg.Fi
    shards = [syn.mlp_shard_inputs(cfg, shard=i) for i in range(t)]
    X, dZ = shards[0]["X"], shards[0]["dZ"]
    Xd, dZd = dev(X), dev(dZ)
    ks_local = tile_sample_idx(Fi, 192, 31, per_tile=2)
    zparts, dxparts, dA_s, dA2_s, dB_s = [], [], [], [], []
    for d in shards:
        Ad, A2d, Bd = dev(d["A"]), dev(d["A2"]), dev(d["B"])
        Y, Pre = ops.column_fwd(Xd, Ad, "swiglu", A2=A2d)
        zparts.append(ops.row_fwd(Y, Bd))
        dY, dB, _ = ops.row_bwd(dZd, Y, Bd)
        dX, dA, dA2, _, _ = ops.column_bwd(dY, Xd, Ad, Pre=Pre, act="swiglu", A2=A2d)
        dxparts.append(dX)
        dA_s.append(cols(dA, ks_local))
        dA2_s.append(cols(dA2, ks_local))
        dB_s.append(rows(dB, ks_local))
        del Y, Pre, dY, dB, dA, dA2
    zb, n = ops.stack_partials(zparts)
    xb, n2 = ops.stack_partials(dxparts)
    del zparts, dxparts
    Z = ops.sum_partials(zb, n)
    dXs = ops.sum_partials(xb, n2)
    torch.cuda.synchronize()

    Af = np.concatenate([d["A"].f64 for d in shards], axis=1)
    A2f = np.concatenate([d["A2"].f64 for d in shards], axis=1)
    Bf = np.concatenate([d["B"].f64 for d in shards], axis=0)
    Xf, dZf = X.f64, dZ.f64
    ms = tile_sample_idx(M, 256, 30, per_tile=2)
    Yr, Prer = oracle.column_fwd(Xf[ms], Af, "swiglu", A2=A2f)
    assert_close("Z rows (8 partials summed)", rows(Z, ms), oracle.row_fwd(Yr, Bf), BF)
    dYr = oracle.dgrad(dZf[ms], Bf)
    dXr = oracle.column_bwd(dYr, Xf[ms], Af, Prer, "swiglu", A2f)[0]
    assert_close("dX rows (8 partials summed)", rows(dXs, ms), dXr, BF)
    ks = np.concatenate([i * Fi + ks_local for i in range(t)])   # the same local columns of every shard
    Yk, Prek = oracle.column_fwd(Xf, Af[:, ks], "swiglu", A2=A2f[:, ks])
    assert_close("dB rows (concatenated)", np.concatenate(dB_s, axis=0), oracle.wgrad(Yk, dZf), BF)
    dYk = oracle.dgrad(dZf, Bf[ks, :])
    _, dAk, dA2k, _, _ = oracle.column_bwd(dYk, Xf, Af[:, ks], Prek, "swiglu", A2f[:, ks])
    assert_close("dA cols (concatenated)", np.concatenate(dA_s, axis=1), dAk, BF)
    assert_close("dA2 cols (concatenated)", np.concatenate(dA2_s, axis=1), dA2k, BF)


def test_c2_sequence_parallel_boundary_sampled():
    # The 8 row partials of c2's down projection [8192, 4096], reduce-scattered
    # over token blocks of 1024 rows, + bias + residual, then LayerNorm.
    cfg = syn.C2
    t, M, N = cfg.t, cfg.M, cfg.H
    Mr = M // t
    seeded = [syn.normal(2950 + i, (M, N), 1.0, syn.BF16) for i in range(t)]
    bias = syn.normal(2960, (N,), 0.02, syn.BF16)
    gamma = syn.normal(2961, (N,), 1.0, syn.BF16)
    beta = syn.normal(2962, (N,), 0.1, syn.BF16)
    buf, n = ops.stack_partials([dev(p) for p in seeded])
    ms = sample_idx(Mr, 48, 13)
    part_rows = {}
    for rank in (0, 3, t - 1):
        r0 = rank * Mr
        resid = syn.normal(2970 + rank, (Mr, N), 1.0, syn.BF16)
        y, h = ops.sp_reduce_scatter_ln(buf, n, r0, Mr, dev(bias), dev(resid), dev(gamma), dev(beta), eps=1e-5)
        torch.cuda.synchronize()
        for i, p in enumerate(seeded):
            part_rows[i] = p.f64[r0 + ms]
        ry, rh = oracle.sp_reduce_scatter_ln([part_rows[i] for i in range(t)], 0, len(ms), bias.f64,
                                             resid.f64[ms], gamma.f64, beta.f64, 1e-5)
        assert_close(f"h rank {rank}", rows(h, ms), rh, BF)
        assert_close(f"y rank {rank}", rows(y, ms), ry, BF)


# ---------------------------------------------------------------------------
# c5: vocab-parallel LM head + CE partials.
# ---------------------------------------------------------------------------

def test_c5_shard0_full_size_sampled():
    cfg = syn.C5
    d = syn.vocab_inputs(cfg, shard=0)
    target = d["target"].copy()
    # two tokens in every 256-row tile; half of them get their target in shard 0
    ms = tile_sample_idx(cfg.M, 256, 12, per_tile=2)
    target[ms[::2]] = (ms[::2] * 7919) % cfg.Vr
    m, s, tg = ops.vocab_ce_partials(dev(d["H"]), dev(d["W"]), torch.from_numpy(target).cuda(), d["v0"])
    torch.cuda.synchronize()
    rm, rs, rt = oracle.vocab_ce_partials(d["H"].f64[ms], d["W"].f64, target[ms], d["v0"])
    gl, gt, gloss = oracle.lse_recombine([(host64(m)[ms], host64(s)[ms], host64(tg)[ms])])
    rl, rt2, rloss = oracle.lse_recombine([(rm, rs, rt)])
    assert_close("lse", gl, rl, TOL_CE)
    assert_close("tgt", gt, rt2, TOL_CE)
    assert_close("loss", gloss, rloss, TOL_CE)


def test_c5_ce_backward_full_size_sampled():
    cfg = syn.C5
    d = syn.vocab_inputs(cfg, shard=0)
    target = d["target"].copy()
    # token rows of dH and vocab rows of dW: two in every 256-row block (the GEMM tile), so that
    # every tile of the dz workspace and of both products enters the check
    ms = tile_sample_idx(cfg.M, 256, 13, per_tile=2)
    js = tile_sample_idx(cfg.Vr, 256, 14, per_tile=2)
    target[ms[::2]] = (ms[::2] * 7919) % cfg.Vr
    # lse near the shard's own log-sum-exp (ln 18992 + 1.28^2/2 ~ 10.7), so the softmax
    # term and the onehot term are both of order one; g: per-token upstream gradient
    lse = (10.7 + syn.normal(cfg.seed + 30, (cfg.M,), 0.3, syn.FP32).f32).astype(np.float32)
    g = syn.normal(cfg.seed + 31, (cfg.M,), 1.0, syn.FP32).f32
    dH, dW = ops.vocab_ce_bwd(dev(d["H"]), dev(d["W"]), torch.from_numpy(target).cuda(), d["v0"],
                              torch.from_numpy(lse).cuda(), torch.from_numpy(g).cuda())
    torch.cuda.synchronize()
    H64, W64 = d["H"].f64, d["W"].f64
    _, rdH, _ = oracle.vocab_ce_bwd(H64[ms], W64, target[ms], d["v0"], lse[ms], g[ms])
    assert_close("dH", host64(dH)[ms], rdH, TOL[syn.BF16])
    # dW rows j: dz[:, j] over all tokens, from the oracle restricted to vocab rows js
    dz_cols = np.empty((cfg.M, len(js)))
    for c, j in enumerate(js):
        dzc, _, _ = oracle.vocab_ce_bwd(H64, W64[j:j + 1], target, d["v0"] + j, lse, g)
        dz_cols[:, c] = dzc[:, 0]
    rdW = dz_cols.T @ H64
    assert_close("dW", host64(dW)[js], rdW, TOL[syn.BF16])


def test_c5_ce_chain_eight_shards_full_size_sampled():
    # c5's full vocabulary (8 shards of 18992) with every intermediate made on
    # the GPU: partials of all 8 shards -> tp_vocab_ce_combine -> each shard's
    # backward on that lse -> dH summed over the shards.  The oracle recombines
    # its own partials; lse, tgt, loss and dH are compared on two tokens of every
    # 256-row tile.
    cfg = syn.C5
    base = syn.vocab_inputs(cfg, shard=0)
    H, target = base["H"], base["target"]
    g = syn.normal(cfg.seed + 40, (cfg.M,), 1.0, syn.FP32).f32
    Hd, td, gd = dev(H), torch.from_numpy(target).cuda(), torch.from_numpy(g).cuda()
    ms = tile_sample_idx(cfg.M, 256, 41, per_tile=2)
    mstk = torch.empty(cfg.shards, cfg.M, dtype=torch.float32, device="cuda")
    sstk, tstk = torch.empty_like(mstk), torch.empty_like(mstk)
    rparts, rdH = [], np.zeros((len(ms), cfg.H))
    Ws = []
    for r in range(cfg.shards):
        W = syn.vocab_inputs(cfg, shard=r, M=1)["W"]
        m, s, tg = ops.vocab_ce_partials(Hd, dev(W), td, r * cfg.Vr)
        mstk[r].copy_(m)
        sstk[r].copy_(s)
        tstk[r].copy_(tg)
        rparts.append(oracle.vocab_ce_partials(H.f64[ms], W.f64, target[ms], r * cfg.Vr))
        Ws.append(W)
    lse, tgt, loss = ops.vocab_ce_combine(mstk, sstk, tstk)
    rl, rt, rloss = oracle.lse_recombine(rparts)
    dHs = []
    for r, W in enumerate(Ws):
        dH, _ = ops.vocab_ce_bwd(Hd, dev(W), td, r * cfg.Vr, lse, gd, want_dw=False)
        dHs.append(dH)
        rdH += oracle.vocab_ce_bwd(H.f64[ms], W.f64, target[ms], r * cfg.Vr, rl, g[ms])[1]
    buf, n = ops.stack_partials(dHs)
    del dHs
    dHsum = ops.sum_partials(buf, n)
    torch.cuda.synchronize()
    assert_close("lse", host64(lse)[ms], rl, TOL_CE)
    assert_close("tgt", host64(tgt)[ms], rt, TOL_CE)
    assert_close("loss", host64(loss)[ms], rloss, TOL_CE)
    assert_close("dH summed", rows(dHsum, ms), rdH, BF)


def test_c3_attention_core_full_size():
    # The rank's 4 query heads and 1 KV head over one 8192-token sequence, causal, read
    # straight from the packed QKV projection output [8192, 768].
    cfg = syn.C3
    S, n_q, n_kv = cfg.M, 4, 1
    qkv = syn.normal(3950, (S, cfg.n_qkv), 1.0, syn.BF16)
    d = dev(qkv)
    O, lse = ops.attention_fwd(d[:, :512], d[:, 512:640], d[:, 640:], n_q, n_kv, causal=True)
    torch.cuda.synchronize()
    X = qkv.f64
    ro, rl = oracle.attention_fwd(X[:, :512], X[:, 512:640], X[:, 640:], n_q, n_kv, causal=True)
    ms = sample_idx(S, 256, 19)
    assert_close("O", rows(O, ms), ro[ms], BF)
    assert_close("lse", host64(lse[0])[:, ms], rl[:, ms], 1e-3)


def test_c3_attention_backward_full_size():
    # Backward of the rank's attention core over the 8192-token sequence (causal, GQA 4:1).
    cfg = syn.C3
    S, n_q, n_kv = cfg.M, 4, 1
    qkv = syn.normal(3960, (S, cfg.n_qkv), 1.0, syn.BF16)
    dO = syn.normal(3961, (S, 512), 1.0, syn.BF16)
    d = dev(qkv)
    q, k, v = d[:, :512], d[:, 512:640], d[:, 640:]
    O, lse = ops.attention_fwd(q, k, v, n_q, n_kv, causal=True)
    dq, dk, dv = ops.attention_bwd(q, k, v, O, lse, dev(dO), n_q, n_kv, causal=True)
    torch.cuda.synchronize()
    X = qkv.f64
    rq, rk, rv = oracle.attention_bwd(X[:, :512], X[:, 512:640], X[:, 640:], dO.f64, n_q, n_kv, causal=True)
    ms = sample_idx(S, 512, 21)
    assert_close("dQ", rows(dq, ms), rq[ms], BF)
    assert_close("dK", rows(dk, ms), rk[ms], BF)
    assert_close("dV", rows(dv, ms), rv[ms], BF)


def test_c5_vocab_embedding_shard_full_size():
    # Embedding shard 0 of 8 of the 151936 x 4096 table (18992 rows), 8192 tokens with ids
    # uniform over the full vocabulary: lookup compared in full, backward on the rows that
    # received tokens plus sampled empty rows.
    cfg = syn.C5
    M, K, Vr, v0 = cfg.M, cfg.H, cfg.Vr, 0
    ids = syn.targets(5950, M, cfg.vocab)
    E = syn.normal(5951, (Vr, K), 0.02, syn.BF16)
    dout = syn.normal(5952, (M, K), 1.0, syn.BF16)
    idt = torch.from_numpy(ids).cuda()
    out = ops.vocab_embed_fwd(idt, dev(E), v0)
    dE = ops.vocab_embed_bwd(idt, dev(dout), v0, Vr)
    torch.cuda.synchronize()
    own = (ids >= v0) & (ids < v0 + Vr)
    ms = sample_idx(M, 256, 17)
    ms = np.unique(np.concatenate([ms, np.nonzero(own)[0][:64]]))
    assert np.array_equal(rows(out, ms), oracle.vocab_embed_fwd(ids[ms], E.f64, v0))
    used = np.unique(ids[own] - v0)
    vs = np.unique(np.concatenate([used, sample_idx(Vr, 128, 18)]))
    ref = oracle.vocab_embed_bwd(ids, dout.f64, v0, Vr)
    assert_close("dE", rows(dE, vs), ref[vs], BF)
    # rows no token uses are exactly zero
    empty = np.setdiff1d(np.arange(Vr), used)
    assert float(torch.count_nonzero(dE[torch.from_numpy(empty).cuda()]).item()) == 0.0


def test_c5_eight_shards_recombined():
    cfg = syn.C5
    Mt = 64
    base = syn.vocab_inputs(cfg, shard=0, M=cfg.M)
    H = base["H"]
    Hs = syn.Tensor(syn.BF16, np.ascontiguousarray(H.raw[:Mt]), (Mt, cfg.H))
    target = base["target"][:Mt].copy()
    Hd = dev(Hs)
    tgt_d = torch.from_numpy(target).cuda()
    gparts, rparts = [], []
    for r in range(cfg.shards):
        W = syn.vocab_inputs(cfg, shard=r, M=1)["W"]
        v0 = r * cfg.Vr
        m, s, tg = ops.vocab_ce_partials(Hd, dev(W), tgt_d, v0)
        torch.cuda.synchronize()
        gparts.append((host64(m), host64(s), host64(tg)))
        rparts.append(oracle.vocab_ce_partials(Hs.f64, W.f64, target, v0))
        del W
    gl, gt, gloss = oracle.lse_recombine(gparts)
    rl, rt, rloss = oracle.lse_recombine(rparts)
    assert_close("lse", gl, rl, TOL_CE)
    assert_close("tgt", gt, rt, TOL_CE)
    assert_close("loss", gloss, rloss, TOL_CE)
