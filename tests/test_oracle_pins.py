"""Pins of the CPU oracle against what the pages and mathematics fix.

Each test checks the oracle against something other than itself: the pages'
worked examples (tests/golden, each file cites its page and section),
textbook values, closed forms, finite differences and brute-force loops.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# Worked examples printed on the pages (exact).
# ---------------------------------------------------------------------------

def test_v1_column_and_row_split_of_2x2():
    g = _golden("v1_block_2x2.json")
    X, A = np.array(g["X"], float), np.array(g["A"], float)
    t = 2
    for i in range(t):
        cs = oracle.column_slice(2, t, i)
        Y, pre = oracle.column_fwd(X, A[:, cs])
        assert pre is None
        assert np.array_equal(Y, np.array(g["column_t2"]["shard_outputs"][i], float))
    parts = []
    for i in range(t):
        rs = oracle.row_slice(2, t, i)
        Z = oracle.row_fwd(X[:, rs], A[rs, :])
        assert np.array_equal(Z, np.array(g["row_t2"]["shard_partials"][i], float))
        parts.append(Z)
    assert np.array_equal(oracle.sum_partials(parts), np.array(g["row_t2"]["sum"], float))
    assert np.array_equal(oracle.sum_partials(parts), np.array(g["XA"], float))


def test_v2_column_t3_forward_backward():
    g = _golden("v2_column_t3.json")
    X, W, dY = (np.array(g[k], float) for k in ("X", "W", "dY"))
    t = g["t"]
    dx_parts = []
    for i in range(t):
        cs = oracle.column_slice(3, t, i)
        Y, _ = oracle.column_fwd(X, W[:, cs])
        assert np.array_equal(Y, np.array(g["Y_shards"][i], float))
        dXp, dA, dA2, db, db2 = oracle.column_bwd(dY[:, cs], X, W[:, cs])
        assert dA2 is None and db2 is None
        assert np.array_equal(dA, np.array(g["dW_shards"][i], float))
        assert np.array_equal(dXp, np.array(g["dX_parts"][i], float))
        assert np.array_equal(db, dY[0, cs])
        dx_parts.append(dXp)
    assert np.array_equal(oracle.sum_partials(dx_parts), np.array(g["dX"], float))


def test_v3_activation_never_acts_on_partials():
    g = _golden("v3_relu_partials.json")
    p = [np.array([[v]], float) for v in g["partials"]]
    relu = lambda x: np.maximum(x, 0.0)  # the page's own example activation
    assert oracle.sum_partials(p)[0, 0] == 1.0
    assert relu(oracle.sum_partials(p))[0, 0] == g["relu_of_sum"]
    assert oracle.sum_partials([relu(q) for q in p])[0, 0] == g["sum_of_relu"]
    # The same failure with the activations this library fuses.
    assert oracle.gelu(oracle.sum_partials(p))[0, 0] != pytest.approx(
        oracle.sum_partials([oracle.gelu(q) for q in p])[0, 0], rel=1e-3)
    # And the right order (column -> act -> row -> sum) equals the unsharded MLP.
    rng = np.random.default_rng(3)
    X = rng.standard_normal((5, 6))
    A = rng.standard_normal((6, 8))
    B = rng.standard_normal((8, 6))
    full = oracle.gelu(X @ A) @ B
    parts = []
    for i in range(2):
        cs = oracle.column_slice(8, 2, i)
        Y, _ = oracle.column_fwd(X, A[:, cs], act="gelu")
        parts.append(oracle.row_fwd(Y, B[cs, :]))
    np.testing.assert_allclose(oracle.sum_partials(parts), full, rtol=1e-12, atol=1e-12)


def test_v4_fig2_two_gpu_allreduce_result():
    g = _golden("v4_fig2_allreduce.json")
    parts = [np.array([v], float) for v in g["gpu_inputs"]]
    Z = oracle.sum_partials(parts)
    assert np.array_equal(Z, np.array([g["all_gather"][0]], float))
    assert Z[0, 0] == g["reduce_scatter"]["gpu0_first_half"]
    assert Z[0, 1] == g["reduce_scatter"]["gpu1_second_half"]


def test_v5_row_bias_added_once():
    # Page 'v4: Tensor Parallel and Sequence Parallel', section 'Self-test':
    # the row bias is not split; adding it on every card adds it t times.
    g = _golden("v1_block_2x2.json")
    parts = [np.array(p, float) for p in g["row_t2"]["shard_partials"]]
    b = np.array([10.0, 20.0])
    assert np.array_equal(oracle.sum_partials(parts, bias=b), np.array([[17.0, 30.0]]))
    wrong = oracle.sum_partials([p + b for p in parts])
    assert np.array_equal(wrong, oracle.sum_partials(parts, bias=b) + (len(parts) - 1) * b)


def test_v6_bias_gradients_by_hand():
    # Page 'v4: Tensor Parallel and Sequence Parallel', section 'Self-test':
    # bias gradients are among the quantities compared with one device.  Hand
    # case on the 2x2 block example split row-wise over t = 2 ranks, two
    # tokens, upstream gradient dZ = [[1, 2], [3, 4]].  The replicated row
    # bias b enters Z = X1 A1 + X2 A2 + b once, so dL/db = sum over tokens of
    # dZ = [4, 6] on EVERY rank (an all-reduce of it would give t times that).
    g = _golden("v1_block_2x2.json")
    X = np.array(g["X"] * 2, float)          # two identical tokens [1, 2]
    A = np.array(g["A"], float)
    dZ = np.array([[1.0, 2.0], [3.0, 4.0]])
    for i in range(2):
        rs = oracle.row_slice(2, 2, i)
        dXi, dAi, db = oracle.row_bwd(dZ, X[:, rs], A[rs, :])
        assert np.array_equal(db, np.array([4.0, 6.0]))
        # dX_i = dZ A_i^T, dA_i = X_i^T dZ, each entry by hand
        a = A[rs, :][0]                      # the rank's one row of A
        assert np.array_equal(dXi[:, 0], np.array([1 * a[0] + 2 * a[1], 3 * a[0] + 4 * a[1]]))
        x = X[0, rs][0]
        assert np.array_equal(dAi, np.array([[x * 4.0, x * 6.0]]))
    # Column-split SwiGLU with one token and one column per rank, zero gate:
    # G = 0 gives silu(0) = 0 and silu'(0) = 1/2, so with U = 3 and dY = 2 the
    # gate-bias gradient is dY * U * 1/2 = 3 and the up-bias gradient is
    # dY * silu(0) = 0; with G = ln 3 (sigmoid = 3/4, silu = (3/4) ln 3):
    # up-bias gradient = 2 * (3/4) ln 3.
    for gate, want_g, want_u in ((0.0, 3.0, 0.0),
                                 (math.log(3.0), 2 * 3.0 * (0.75 + math.log(3.0) * 0.75 * 0.25),
                                  2 * 0.75 * math.log(3.0))):
        Xo = np.array([[1.0]])
        _, Pre = oracle.column_fwd(Xo, np.array([[0.0]]), "swiglu", bias=np.array([gate]),
                                   A2=np.array([[0.0]]), bias2=np.array([3.0]))
        _, _, _, db, db2 = oracle.column_bwd(np.array([[2.0]]), Xo, np.array([[0.0]]), Pre, "swiglu",
                                             np.array([[0.0]]))
        assert db[0] == pytest.approx(want_g, rel=1e-15)
        assert db2[0] == pytest.approx(want_u, rel=1e-15, abs=0.0)


# ---------------------------------------------------------------------------
# Activations: textbook values, closed forms, finite differences.
# ---------------------------------------------------------------------------

# Standard normal CDF from tables: Phi(1), Phi(2), Phi(-1); logistic(1) = e/(1+e).
PHI1 = 0.8413447460685429
PHI2 = 0.9772498680518208
PHIM1 = 0.15865525393145707
SIG1 = 0.7310585786300049


def test_gelu_textbook_values():
    x = np.array([0.0, 1.0, -1.0, 2.0])
    np.testing.assert_allclose(oracle.gelu(x), [0.0, PHI1, -PHIM1, 2 * PHI2], rtol=1e-15, atol=0)
    # GeLU'(0) = Phi(0) = 1/2 ; GeLU'(1) = Phi(1) + phi(1)
    phi1 = math.exp(-0.5) / math.sqrt(2 * math.pi)
    np.testing.assert_allclose(oracle.gelu_grad(np.array([0.0, 1.0])), [0.5, PHI1 + phi1], rtol=1e-15)


def test_silu_textbook_values():
    x = np.array([0.0, 1.0, -1.0, 40.0, -40.0])
    np.testing.assert_allclose(oracle.sigmoid(x[:3]), [0.5, SIG1, 1 - SIG1], rtol=1e-15)
    np.testing.assert_allclose(oracle.silu(x[:3]), [0.0, SIG1, -(1 - SIG1)], rtol=1e-15, atol=0)
    # silu'(0) = 1/2; large |x| limits without overflow
    assert oracle.silu_grad(np.array([0.0]))[0] == 0.5
    np.testing.assert_allclose(oracle.silu(x[3:]), [40.0, -40.0 * math.exp(-40.0) / (1 + math.exp(-40.0))],
                               rtol=1e-13)


def test_activation_odd_part_identities():
    x = np.linspace(-6, 6, 121)
    np.testing.assert_allclose(oracle.gelu(x) - oracle.gelu(-x), x, rtol=0, atol=1e-14)
    np.testing.assert_allclose(oracle.silu(x) - oracle.silu(-x), x, rtol=0, atol=1e-14)


def test_activation_grads_by_central_differences():
    x = np.linspace(-5, 5, 101) + 0.0137
    h = 1e-5
    for f, df in ((oracle.gelu, oracle.gelu_grad), (oracle.silu, oracle.silu_grad)):
        fd = (f(x + h) - f(x - h)) / (2 * h)
        np.testing.assert_allclose(df(x), fd, rtol=0, atol=1e-9)


def test_activations_match_torch_cpu_fp64():
    torch = pytest.importorskip("torch")
    x = np.linspace(-8, 8, 1001)
    tx = torch.from_numpy(x)
    np.testing.assert_allclose(oracle.gelu(x), torch.nn.functional.gelu(tx, approximate="none").numpy(),
                               rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(oracle.silu(x), torch.nn.functional.silu(tx).numpy(), rtol=1e-14, atol=1e-15)


# ---------------------------------------------------------------------------
# GEMM building blocks against pure-Python loops (tiny shapes).
# ---------------------------------------------------------------------------

def _loop_mm(a, b):
    m, k = len(a), len(a[0])
    n = len(b[0])
    return [[sum(a[i][p] * b[p][j] for p in range(k)) for j in range(n)] for i in range(m)]


def _T(a):
    return [list(r) for r in zip(*a)]


def test_gemms_against_python_loops():
    rng = np.random.default_rng(11)
    X = rng.standard_normal((3, 5))
    A = rng.standard_normal((5, 4))
    dY = rng.standard_normal((3, 4))
    Xl, Al, dYl = X.tolist(), A.tolist(), dY.tolist()
    np.testing.assert_allclose(oracle.row_fwd(X, A), _loop_mm(Xl, Al), rtol=1e-13)
    Y, _ = oracle.column_fwd(X, A)
    np.testing.assert_allclose(Y, _loop_mm(Xl, Al), rtol=1e-13)
    np.testing.assert_allclose(oracle.dgrad(dY, A), _loop_mm(dYl, _T(Al)), rtol=1e-13)
    np.testing.assert_allclose(oracle.wgrad(X, dY), _loop_mm(_T(Xl), dYl), rtol=1e-13)
    # bias goes inside the linear, before the activation
    b = rng.standard_normal(4)
    Yg, P = oracle.column_fwd(X, A, act="gelu", bias=b)
    loop = _loop_mm(Xl, Al)
    for i in range(3):
        for j in range(4):
            p = loop[i][j] + b[j]
            assert P[i, j] == pytest.approx(p, rel=1e-13)
            assert Yg[i, j] == pytest.approx(0.5 * p * (1 + math.erf(p / math.sqrt(2))), rel=1e-12)


# ---------------------------------------------------------------------------
# Block-matrix invariants over shard counts, activations and bias.
# ---------------------------------------------------------------------------

def _mlp_full(X, A, A2, ba, ba2, B, bB, act):
    Y, _ = oracle.column_fwd(X, A, act=act, bias=ba, A2=A2, bias2=ba2)
    Z = Y @ B
    return Z + bB[None, :] if bB is not None else Z


@pytest.mark.parametrize("t", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("act", ["none", "gelu", "swiglu"])
@pytest.mark.parametrize("bias", [False, True])
def test_sharded_mlp_equals_unsharded(t, act, bias):
    rng = np.random.default_rng(100 * t + len(act) + bias)
    M, H, F = 7, 6, 24
    X = rng.standard_normal((M, H))
    A = rng.standard_normal((H, F)) * 0.5
    A2 = rng.standard_normal((H, F)) * 0.5 if act == "swiglu" else None
    B = rng.standard_normal((F, H)) * 0.5
    ba = rng.standard_normal(F) if bias else None
    ba2 = rng.standard_normal(F) if (bias and act == "swiglu") else None
    bB = rng.standard_normal(H) if bias else None
    dZ = rng.standard_normal((M, H))

    Yfull, _ = oracle.column_fwd(X, A, act=act, bias=ba, A2=A2, bias2=ba2)
    zparts, dxparts, dAs, dA2s, dbs, db2s, dBs, dbrows = [], [], [], [], [], [], [], []
    for i in range(t):
        cs = oracle.column_slice(F, t, i)
        Y, Pre = oracle.column_fwd(X, A[:, cs], act=act, bias=None if ba is None else ba[cs],
                                   A2=None if A2 is None else A2[:, cs],
                                   bias2=None if ba2 is None else ba2[cs])
        np.testing.assert_allclose(Y, Yfull[:, cs], rtol=1e-12, atol=1e-12)
        zparts.append(oracle.row_fwd(Y, B[cs, :]))
        dY, dBi, dbrow = oracle.row_bwd(dZ, Y, B[cs, :])
        dBs.append(dBi)
        dbrows.append(dbrow)
        dXp, dA, dA2, db, db2 = oracle.column_bwd(dY, X, A[:, cs], Pre, act, None if A2 is None else A2[:, cs])
        dxparts.append(dXp)
        dAs.append(dA)
        dA2s.append(dA2)
        dbs.append(db)
        db2s.append(db2)
    Z = oracle.sum_partials(zparts, bias=bB)
    np.testing.assert_allclose(Z, _mlp_full(X, A, A2, ba, ba2, B, bB, act), rtol=1e-11, atol=1e-11)

    # Unsharded backward via finite differences of L = <dZ, Z>.
    def loss(Xv=X, Av=A, A2v=A2, Bv=B):
        return float((dZ * _mlp_full(Xv, Av, A2v, ba, ba2, Bv, bB, act)).sum())

    dX = oracle.sum_partials(dxparts)
    h = 1e-6
    for (idx, arr, grad, key) in [((2, 3), X, dX, "Xv"),
                                  ((1, 5), A, np.concatenate(dAs, axis=1), "Av"),
                                  ((4, 2), B, np.concatenate(dBs, axis=0), "Bv")]:
        ap, am = arr.copy(), arr.copy()
        ap[idx] += h
        am[idx] -= h
        fd = (loss(**{key: ap}) - loss(**{key: am})) / (2 * h)
        assert grad[idx] == pytest.approx(fd, rel=1e-6, abs=1e-7)
    if act == "swiglu":
        ap, am = A2.copy(), A2.copy()
        ap[3, 7] += h
        am[3, 7] -= h
        fd = (loss(A2v=ap) - loss(A2v=am)) / (2 * h)
        assert np.concatenate(dA2s, axis=1)[3, 7] == pytest.approx(fd, rel=1e-6, abs=1e-7)
    # Bias gradients by central differences of L = <dZ, Z> over every entry
    # of each bias.  The replicated row bias enters Z once (after the sum), so
    # every shard's row-bias gradient must equal the full one (not 1/t of it,
    # and not counted t times); the column biases are split with the columns.
    def loss_b(ba_v, ba2_v, bB_v):
        return float((dZ * _mlp_full(X, A, A2, ba_v, ba2_v, B, bB_v, act)).sum())

    def fd_vec(vec, f):
        out = np.empty_like(vec)
        for j in range(vec.size):
            vp, vm = vec.copy(), vec.copy()
            vp[j] += h
            vm[j] -= h
            out[j] = (f(vp) - f(vm)) / (2 * h)
        return out

    if bias:
        fd_ba = fd_vec(ba, lambda v: loss_b(v, ba2, bB))
        np.testing.assert_allclose(np.concatenate(dbs), fd_ba, rtol=1e-6, atol=1e-7)
        fd_bB = fd_vec(bB, lambda v: loss_b(ba, ba2, v))
        for dbrow in dbrows:
            np.testing.assert_allclose(dbrow, fd_bB, rtol=1e-6, atol=1e-7)
        if act == "swiglu":
            fd_ba2 = fd_vec(ba2, lambda v: loss_b(ba, v, bB))
            np.testing.assert_allclose(np.concatenate(db2s), fd_ba2, rtol=1e-6, atol=1e-7)
        else:
            assert all(d is None for d in db2s)
    else:
        # Without a row bias in the model, its gradient is still defined as the
        # derivative of <dZ, Z + b> at b = 0; pin it the same way.
        zero = np.zeros(H)
        fd_b0 = fd_vec(zero, lambda v: float((dZ * (_mlp_full(X, A, A2, ba, ba2, B, None, act) + v[None, :])).sum()))
        for dbrow in dbrows:
            np.testing.assert_allclose(dbrow, fd_b0, rtol=1e-6, atol=1e-7)


# ---------------------------------------------------------------------------
# Vocab-parallel cross-entropy partials.
# ---------------------------------------------------------------------------

def test_ce_hand_example_ln6():
    # logits [0, ln 2, ln 3]: lse = ln 6; shard 0 owns id 0, shard 1 owns ids 1-2.
    H = np.array([[1.0]])
    W = np.array([[0.0], [math.log(2)], [math.log(3)]])
    p0 = oracle.vocab_ce_partials(H, W[0:1], np.array([1]), 0)
    p1 = oracle.vocab_ce_partials(H, W[1:3], np.array([1]), 1)
    assert (p0[0][0], p0[1][0], p0[2][0]) == (0.0, 1.0, 0.0)
    assert p1[0][0] == pytest.approx(math.log(3), rel=1e-15)
    assert p1[1][0] == pytest.approx(5.0 / 3.0, rel=1e-15)
    assert p1[2][0] == pytest.approx(math.log(2), rel=1e-15)
    lse, tgt, loss = oracle.lse_recombine([p0, p1])
    assert lse[0] == pytest.approx(math.log(6), rel=1e-15)
    assert tgt[0] == pytest.approx(math.log(2), rel=1e-15)
    assert loss[0] == pytest.approx(math.log(3), rel=1e-14)


def test_ce_partials_against_python_loops_and_full_vocab():
    rng = np.random.default_rng(5)
    M, K, V, R = 6, 5, 24, 4
    Hm = rng.standard_normal((M, K))
    W = rng.standard_normal((V, K))
    target = np.array([0, 5, 6, 23, 17, 11])
    vr = V // R
    parts = []
    for r in range(R):
        m, s, tg = oracle.vocab_ce_partials(Hm, W[r * vr:(r + 1) * vr], target, r * vr)
        for i in range(M):
            z = [sum(Hm[i, k] * W[r * vr + j, k] for k in range(K)) for j in range(vr)]
            mx = max(z)
            assert m[i] == pytest.approx(mx, rel=1e-13)
            assert s[i] == pytest.approx(sum(math.exp(v - mx) for v in z), rel=1e-13)
            own = r * vr <= target[i] < (r + 1) * vr
            assert tg[i] == (pytest.approx(z[target[i] - r * vr], rel=1e-13) if own else 0.0)
        parts.append((m, s, tg))
    lse, tgt, loss = oracle.lse_recombine(parts)
    for i in range(M):
        z = [sum(Hm[i, k] * W[j, k] for k in range(K)) for j in range(V)]
        mx = max(z)
        ref = mx + math.log(sum(math.exp(v - mx) for v in z))
        assert lse[i] == pytest.approx(ref, rel=1e-13)
        assert tgt[i] == pytest.approx(z[target[i]], rel=1e-13)
        assert loss[i] == pytest.approx(ref - z[target[i]], rel=1e-12, abs=1e-13)
    # single shard: lse = m + ln s
    lse1, _, _ = oracle.lse_recombine([parts[2]])
    np.testing.assert_allclose(lse1, parts[2][0] + np.log(parts[2][1]), rtol=1e-15)


def test_ce_target_out_of_range_contributes_zero():
    rng = np.random.default_rng(6)
    Hm = rng.standard_normal((4, 3))
    W = rng.standard_normal((5, 3))
    _, _, tg = oracle.vocab_ce_partials(Hm, W, np.array([-1, 4, 9, 10]), 5)
    z = Hm @ W.T
    assert tg[0] == 0.0 and tg[1] == 0.0 and tg[3] == 0.0
    assert tg[2] == pytest.approx(z[2, 4], rel=1e-14)


def test_ce_large_logits_do_not_overflow():
    Hm = np.array([[30.0], [-30.0]])
    W = np.array([[30.0], [29.0], [-5.0]])
    m, s, _ = oracle.vocab_ce_partials(Hm, W, np.array([0, 2]), 0)
    assert m[0] == 900.0 and np.isfinite(s).all()
    lse, _, _ = oracle.lse_recombine([(m, s, np.zeros(2))])
    assert lse[0] == pytest.approx(900.0 + math.log(1 + math.exp(-30.0) + math.exp(-1050.0)), rel=1e-15)


# ---- vocab-parallel CE backward -------------------------------------------------------------

def _full_loss(H, Ws, target, g):
    """Sum_m g_m (lse_m - z_m[target_m]) over the full vocabulary, written out directly."""
    z = np.concatenate([H @ W.T for W in Ws], axis=1)
    out = 0.0
    for m in range(H.shape[0]):
        row = z[m]
        mx = max(row)
        lse = mx + math.log(sum(math.exp(v - mx) for v in row))
        out += g[m] * (lse - row[target[m]])
    return out


def test_ce_bwd_hand_example():
    # z = [0, ln 2]: softmax (1/3, 2/3); target 1 -> dz = (1/3, -1/3)
    H = np.array([[1.0]])
    W = np.array([[0.0], [math.log(2.0)]])
    lse = np.array([math.log(3.0)])
    dz, dH, dW = oracle.vocab_ce_bwd(H, W, [1], 0, lse)
    assert np.allclose(dz, [[1 / 3, -1 / 3]], atol=1e-15)
    assert np.allclose(dH, [[-math.log(2.0) / 3]], atol=1e-15)
    assert np.allclose(dW, [[1 / 3], [-1 / 3]], atol=1e-15)


def test_ce_bwd_finite_differences_over_shards():
    rng = np.random.default_rng(7)
    M, K, vr, R = 3, 4, 5, 3
    H = rng.standard_normal((M, K))
    Ws = [rng.standard_normal((vr, K)) * 0.7 for _ in range(R)]
    target = np.array([2, 9, 14])          # owned by shards 0, 1, 2
    g = np.array([0.5, 1.0, 2.0])
    parts = [oracle.vocab_ce_partials(H, W, target, r * vr) for r, W in enumerate(Ws)]
    lse, _, _ = oracle.lse_recombine(parts)
    outs = [oracle.vocab_ce_bwd(H, W, target, r * vr, lse, g) for r, W in enumerate(Ws)]
    dH = sum(o[1] for o in outs)
    eps = 1e-6
    num_dH = np.zeros_like(H)
    for idx in np.ndindex(H.shape):
        Hp, Hm = H.copy(), H.copy()
        Hp[idx] += eps
        Hm[idx] -= eps
        num_dH[idx] = (_full_loss(Hp, Ws, target, g) - _full_loss(Hm, Ws, target, g)) / (2 * eps)
    assert np.allclose(dH, num_dH, atol=1e-7)
    for r in range(R):
        num_dW = np.zeros_like(Ws[r])
        for idx in np.ndindex(Ws[r].shape):
            Wp = [W.copy() for W in Ws]
            Wm = [W.copy() for W in Ws]
            Wp[r][idx] += eps
            Wm[r][idx] -= eps
            num_dW[idx] = (_full_loss(H, Wp, target, g) - _full_loss(H, Wm, target, g)) / (2 * eps)
        assert np.allclose(outs[r][2], num_dW, atol=1e-7)


def test_ce_bwd_rows_sum_to_zero_and_loops():
    rng = np.random.default_rng(8)
    M, K, vr, R = 4, 3, 6, 2
    H = rng.standard_normal((M, K))
    Ws = [rng.standard_normal((vr, K)) for _ in range(R)]
    target = np.array([0, 7, 11, -3])      # the last token's target is owned by no shard
    parts = [oracle.vocab_ce_partials(H, W, target, r * vr) for r, W in enumerate(Ws)]
    lse, _, _ = oracle.lse_recombine(parts)
    outs = [oracle.vocab_ce_bwd(H, W, target, r * vr, lse) for r, W in enumerate(Ws)]
    rowsum = sum(o[0].sum(axis=1) for o in outs)
    # softmax sums to one; the onehot subtracts one where some shard owns the target
    assert np.allclose(rowsum, [0.0, 0.0, 0.0, 1.0], atol=1e-12)
    for r, (dz, dH, dW) in enumerate(outs):
        for m in range(M):
            for k in range(K):
                assert abs(dH[m, k] - sum(dz[m, j] * Ws[r][j, k] for j in range(vr))) < 1e-12
        for j in range(vr):
            for k in range(K):
                assert abs(dW[j, k] - sum(dz[m, j] * H[m, k] for m in range(M))) < 1e-12


# ---- sequence-parallel reduce-scatter + residual + LayerNorm -------------------------------

def test_sp_reduce_scatter_fig2_halves():
    # Fig. 2 as a reduce-scatter over token rows: each GPU keeps the sum of its own half.
    g = _golden("v4_fig2_allreduce.json")
    parts = [np.array(v, float).reshape(2, 1) for v in g["gpu_inputs"]]   # one column, two token rows
    _, h0 = oracle.sp_reduce_scatter_ln(parts, 0, 1)
    _, h1 = oracle.sp_reduce_scatter_ln(parts, 1, 1)
    assert h0[0, 0] == g["reduce_scatter"]["gpu0_first_half"]
    assert h1[0, 0] == g["reduce_scatter"]["gpu1_second_half"]


def test_layer_norm_closed_forms():
    rng = np.random.default_rng(11)
    h = rng.standard_normal((5, 64)) * 3 + 2
    y = oracle.layer_norm(h, eps=0.0)
    assert np.allclose(y.mean(axis=1), 0.0, atol=1e-12)
    assert np.allclose((y ** 2).mean(axis=1), 1.0, atol=1e-12)
    # hand example: [1, 3] -> mean 2, var 1 -> [-1, 1]; gamma/beta scale and shift per column
    y2 = oracle.layer_norm(np.array([[1.0, 3.0]]), gamma=[2.0, 3.0], beta=[0.5, -1.0], eps=0.0)
    assert np.allclose(y2, [[-1.5, 2.0]], atol=1e-15)
    # eps enters under the square root: [0, 2] with eps = 3 -> var 1 -> +-1/2
    assert np.allclose(oracle.layer_norm(np.array([[0.0, 2.0]]), eps=3.0), [[-0.5, 0.5]], atol=1e-15)


def test_layer_norm_matches_torch_cpu_fp64():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(12)
    h = rng.standard_normal((7, 33))
    gam, bet = rng.standard_normal(33), rng.standard_normal(33)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(h), (33,), torch.from_numpy(gam), torch.from_numpy(bet),
                                         1e-5).numpy()
    assert np.allclose(oracle.layer_norm(h, gam, bet, 1e-5), ref, atol=1e-12)


def test_sp_ranks_concatenated_equal_allreduce_then_layernorm():
    rng = np.random.default_rng(13)
    t, M, N = 4, 12, 16
    parts = [rng.standard_normal((M, N)) for _ in range(t)]
    bias, resid = rng.standard_normal(N), rng.standard_normal((M, N))
    gam, bet = rng.standard_normal(N), rng.standard_normal(N)
    Mr = M // t
    ys, hs = [], []
    for r in range(t):
        y, h = oracle.sp_reduce_scatter_ln(parts, r * Mr, Mr, bias, resid[r * Mr:(r + 1) * Mr], gam, bet)
        ys.append(y)
        hs.append(h)
    full_h = sum(parts) + bias + resid
    assert np.allclose(np.concatenate(hs), full_h, atol=1e-12)
    assert np.allclose(np.concatenate(ys), oracle.layer_norm(full_h, gam, bet), atol=1e-12)



# ---------------------------------------------------------------------------
# Vocab-parallel embedding ("Embedding and LM head: split by vocab").
# ---------------------------------------------------------------------------

def test_vocab_embed_hand_example():
    # vocab 6, K = 2, t = 2 ranks of 3 rows; row v of the table is [10v, 10v + 1]
    E = np.array([[10.0 * v, 10.0 * v + 1] for v in range(6)])
    ids = [4, 0, 4, 7, -1, 2]                      # 7 and -1 are outside the table
    r0 = oracle.vocab_embed_fwd(ids, E[0:3], 0)
    r1 = oracle.vocab_embed_fwd(ids, E[3:6], 3)
    assert np.array_equal(r0, [[0, 0], [0, 1], [0, 0], [0, 0], [0, 0], [20, 21]])
    assert np.array_equal(r1, [[40, 41], [0, 0], [40, 41], [0, 0], [0, 0], [0, 0]])
    assert np.array_equal(r0 + r1, [[40, 41], [0, 1], [40, 41], [0, 0], [0, 0], [20, 21]])
    dout = np.array([[m, -m] for m in range(6)], float)
    assert np.array_equal(oracle.vocab_embed_bwd(ids, dout, 0, 3), [[1, -1], [0, 0], [5, -5]])
    assert np.array_equal(oracle.vocab_embed_bwd(ids, dout, 3, 3), [[0, 0], [2, -2], [0, 0]])


def test_vocab_embed_shards_sum_to_full_lookup():
    rng = np.random.default_rng(21)
    V, K, t, M = 40, 6, 4, 50
    E = rng.standard_normal((V, K))
    ids = rng.integers(0, V, size=M)
    Vr = V // t
    total = sum(oracle.vocab_embed_fwd(ids, E[r * Vr:(r + 1) * Vr], r * Vr) for r in range(t))
    assert np.array_equal(total, np.take(E, ids, axis=0))
    # each token is owned by exactly one rank
    owners = [np.any(oracle.vocab_embed_fwd(ids, np.ones((Vr, 1)), r * Vr) != 0, axis=1) for r in range(t)]
    assert np.array_equal(np.sum(owners, axis=0), np.ones(M))


def test_vocab_embed_bwd_is_the_adjoint_and_a_onehot_product():
    rng = np.random.default_rng(22)
    Vr, K, M, v0 = 9, 5, 60, 100
    ids = rng.integers(v0 - 10, v0 + Vr + 10, size=M)
    ids[:4] = [v0, v0 + Vr - 1, v0 + 3, v0 + 3]    # both block ends and a repeated id
    Er = rng.standard_normal((Vr, K))
    dout = rng.standard_normal((M, K))
    dE = oracle.vocab_embed_bwd(ids, dout, v0, Vr)
    # <lookup(E), dout> = <E, dE> for every E: dE is the gradient of that inner product
    assert np.isclose(np.sum(oracle.vocab_embed_fwd(ids, Er, v0) * dout), np.sum(Er * dE), rtol=1e-12)
    onehot = np.zeros((M, Vr))
    own = (ids >= v0) & (ids < v0 + Vr)
    onehot[np.nonzero(own)[0], ids[own] - v0] = 1.0
    assert np.allclose(dE, onehot.T @ dout, atol=1e-12)


def test_vocab_embed_bwd_shards_concatenate_to_full():
    rng = np.random.default_rng(23)
    V, K, t, M = 24, 3, 3, 80
    ids = rng.integers(-3, V + 3, size=M)
    dout = rng.standard_normal((M, K))
    Vr = V // t
    full = oracle.vocab_embed_bwd(ids, dout, 0, V)
    parts = np.concatenate([oracle.vocab_embed_bwd(ids, dout, r * Vr, Vr) for r in range(t)])
    assert np.array_equal(parts, full)


# ---------------------------------------------------------------------------
# Attention core ("Attention: split by head"), GQA.
# ---------------------------------------------------------------------------

def _attn_loops(Q, K, V, n_q, n_kv, causal, scale):
    """Pure-Python triple loops: softmax attention written element by element."""
    S, d = len(Q), len(Q[0]) // n_q
    group = n_q // n_kv
    O = [[0.0] * (n_q * d) for _ in range(S)]
    for h in range(n_q):
        g = h // group
        for i in range(S):
            keys = range(i + 1) if causal else range(S)
            sc = [sum(Q[i][h * d + c] * K[j][g * d + c] for c in range(d)) * scale for j in keys]
            mx = max(sc)
            w = [math.exp(x - mx) for x in sc]
            z = sum(w)
            for c in range(d):
                O[i][h * d + c] = sum(w[t] * V[j][g * d + c] for t, j in enumerate(keys)) / z
    return O


@pytest.mark.parametrize("causal", [True, False])
def test_attention_matches_loops(causal):
    rng = np.random.default_rng(31)
    S, d, n_q, n_kv = 5, 3, 4, 2
    Q = rng.standard_normal((S, n_q * d))
    K = rng.standard_normal((S, n_kv * d))
    V = rng.standard_normal((S, n_kv * d))
    O, lse = oracle.attention_fwd(Q, K, V, n_q, n_kv, causal=causal, scale=0.7)
    ref = _attn_loops(Q.tolist(), K.tolist(), V.tolist(), n_q, n_kv, causal, 0.7)
    assert np.allclose(O, ref, atol=1e-12)


def test_attention_closed_forms():
    rng = np.random.default_rng(32)
    S, d = 6, 4
    V = rng.standard_normal((S, d))
    K = rng.standard_normal((S, d))
    Z = np.zeros((S, d))
    # zero queries: uniform weights -> causal rows are prefix means, lse = log(i + 1)
    O, lse = oracle.attention_fwd(Z, K, V, 1, 1, causal=True)
    assert np.allclose(O, np.cumsum(V, axis=0) / np.arange(1, S + 1)[:, None], atol=1e-12)
    assert np.allclose(lse[0], np.log(np.arange(1, S + 1)), atol=1e-12)
    O, lse = oracle.attention_fwd(Z, K, V, 1, 1, causal=False)
    assert np.allclose(O, np.broadcast_to(V.mean(axis=0), (S, d)), atol=1e-12)
    # first row under the causal mask sees only key 0: O = V[0], lse = q.k * scale
    Q = rng.standard_normal((S, d))
    O, lse = oracle.attention_fwd(Q, K, V, 1, 1, causal=True)
    assert np.allclose(O[0], V[0], atol=1e-12)
    assert np.isclose(lse[0, 0], Q[0] @ K[0] / 2.0)          # default scale 1/sqrt(4)


def test_attention_matches_torch_sdpa_fp64():
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    rng = np.random.default_rng(33)
    S, d, n_q, n_kv = 9, 8, 4, 1
    Q = rng.standard_normal((S, n_q * d))
    K = rng.standard_normal((S, n_kv * d))
    V = rng.standard_normal((S, n_kv * d))
    dO = rng.standard_normal((S, n_q * d))
    for causal in (True, False):
        q = torch.tensor(Q.reshape(S, n_q, d).transpose(1, 0, 2), requires_grad=True)
        k = torch.tensor(K.reshape(S, n_kv, d).transpose(1, 0, 2), requires_grad=True)
        v = torch.tensor(V.reshape(S, n_kv, d).transpose(1, 0, 2), requires_grad=True)
        kr = k.repeat_interleave(n_q // n_kv, dim=0)
        vr = v.repeat_interleave(n_q // n_kv, dim=0)
        o = F.scaled_dot_product_attention(q, kr, vr, is_causal=causal)
        o.backward(torch.tensor(dO.reshape(S, n_q, d).transpose(1, 0, 2)))
        O, _ = oracle.attention_fwd(Q, K, V, n_q, n_kv, causal=causal)
        assert np.allclose(O, o.detach().numpy().transpose(1, 0, 2).reshape(S, n_q * d), atol=1e-12)
        dQ, dK, dV = oracle.attention_bwd(Q, K, V, dO, n_q, n_kv, causal=causal)
        assert np.allclose(dQ, q.grad.numpy().transpose(1, 0, 2).reshape(S, -1), atol=1e-12)
        assert np.allclose(dK, k.grad.numpy().transpose(1, 0, 2).reshape(S, -1), atol=1e-12)
        assert np.allclose(dV, v.grad.numpy().transpose(1, 0, 2).reshape(S, -1), atol=1e-12)


def test_attention_bwd_finite_differences():
    rng = np.random.default_rng(34)
    S, d, n_q, n_kv = 4, 3, 2, 1
    Q = rng.standard_normal((S, n_q * d))
    K = rng.standard_normal((S, n_kv * d))
    V = rng.standard_normal((S, n_kv * d))
    dO = rng.standard_normal((S, n_q * d))
    grads = oracle.attention_bwd(Q, K, V, dO, n_q, n_kv, causal=True)

    def loss(q, k, v):
        return float(np.sum(oracle.attention_fwd(q, k, v, n_q, n_kv, causal=True)[0] * dO))

    eps = 1e-6
    for which, X in enumerate((Q, K, V)):
        for idx in [(0, 0), (S - 1, X.shape[1] - 1), (2, 1)]:
            args = [Q.copy(), K.copy(), V.copy()]
            args[which][idx] += eps
            up = loss(*args)
            args[which][idx] -= 2 * eps
            dn = loss(*args)
            assert np.isclose(grads[which][idx], (up - dn) / (2 * eps), rtol=1e-6, atol=1e-8)


def test_attention_gqa_equals_replicated_kv():
    rng = np.random.default_rng(35)
    S, d, n_q = 7, 4, 4
    Q = rng.standard_normal((S, n_q * d))
    K = rng.standard_normal((S, d))
    V = rng.standard_normal((S, d))
    dO = rng.standard_normal((S, n_q * d))
    O1, l1 = oracle.attention_fwd(Q, K, V, n_q, 1)
    O4, l4 = oracle.attention_fwd(Q, np.tile(K, 4), np.tile(V, 4), n_q, n_q)
    assert np.allclose(O1, O4, atol=1e-12) and np.allclose(l1, l4, atol=1e-12)
    _, dK1, dV1 = oracle.attention_bwd(Q, K, V, dO, n_q, 1)
    _, dK4, dV4 = oracle.attention_bwd(Q, np.tile(K, 4), np.tile(V, 4), dO, n_q, n_q)
    assert np.allclose(dK1, dK4.reshape(S, 4, d).sum(axis=1), atol=1e-12)
    assert np.allclose(dV1, dV4.reshape(S, 4, d).sum(axis=1), atol=1e-12)
