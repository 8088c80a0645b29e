"""Plain float64 definitions of what one tensor-parallel shard computes.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

Citations name the source page and its section:
  [TP/SP]  page "v4: Tensor Parallel and Sequence Parallel" (infra lesson v4)
  [TPcomm] page "TP communication: how many all-reduces per layer, how much data"

Conventions (the math layout of Y = XA, weights [K, N], all row-major):
  * X [M, K] tokens x features; column weight shard A_i [K, N_i];
    row weight shard B_i [K_i, N]; LM-head shard W_r [V_r, K] (vocab rows).
  * Shard i of t owns the i-th contiguous block, in shard order.
Every function takes numpy arrays (any float dtype) and returns float64.
Parity status: every function below is pinned by tests/test_oracle_*.py
(worked examples of the pages, closed forms, textbook values, brute force);
none is "parity unpinned".
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf

_SQRT2 = math.sqrt(2.0)
_INV_SQRT_2PI = 1.0 / math.sqrt(2.0 * math.pi)


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------------------
# Shard maps.  [TP/SP] "Full flow: column parallel, t = 3" (GPU i takes column
# i) and "Where column and row communicate" (column: [k, n/t] per card; row:
# [k/t, n] per card).  Contiguous blocks in shard order.
# ---------------------------------------------------------------------------

def column_slice(n_full: int, t: int, i: int) -> slice:
    """Output columns owned by column-parallel shard i of t."""
    if n_full % t:
        raise ValueError("width not divisible by t")
    w = n_full // t
    return slice(i * w, (i + 1) * w)


def row_slice(k_full: int, t: int, i: int) -> slice:
    """Inner-dimension rows (and input columns) owned by row-parallel shard i of t."""
    return column_slice(k_full, t, i)


# ---------------------------------------------------------------------------
# Activations.  [TP/SP] "MLP: column first, then row" names GeLU (elementwise,
# local to the shard) and Qwen3's SwiGLU (gate and up both column-split,
# multiplied elementwise on the shard).  The pages give neither formula; the
# readings are the exact erf GeLU, x * Phi(x), and SwiGLU = silu(gate) * up.
# ---------------------------------------------------------------------------

def gelu(x):
    """GeLU(x) = x * Phi(x) with the exact normal CDF Phi(x) = (1 + erf(x/sqrt 2)) / 2."""
    x = _f64(x)
    return 0.5 * x * (1.0 + erf(x / _SQRT2))


def gelu_grad(x):
    """d/dx GeLU = Phi(x) + x * phi(x), phi the standard normal density."""
    x = _f64(x)
    cdf = 0.5 * (1.0 + erf(x / _SQRT2))
    pdf = _INV_SQRT_2PI * np.exp(-0.5 * x * x)
    return cdf + x * pdf


def sigmoid(x):
    """Logistic function 1 / (1 + e^-x), evaluated without overflow."""
    x = _f64(x)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    e = np.exp(x[~pos])
    out[~pos] = e / (1.0 + e)
    return out


def silu(x):
    """silu(x) = x * sigmoid(x)."""
    x = _f64(x)
    return x * sigmoid(x)


def silu_grad(x):
    """d/dx silu = sigmoid(x) * (1 + x * (1 - sigmoid(x)))."""
    x = _f64(x)
    s = sigmoid(x)
    return s * (1.0 + x * (1.0 - s))


# ---------------------------------------------------------------------------
# Forward.
# ---------------------------------------------------------------------------

def column_fwd(X, A, act="none", bias=None, A2=None, bias2=None):
    """Column-parallel shard forward: Y_i = act(X A_i + b_i).

    [TP/SP] "TP math: block matrix multiplication": X[A_1, A_2] = [XA_1, XA_2],
    so a column shard takes the full X (f is the identity in the forward,
    "Full flow: column parallel, t = 3") and emits its own output columns.
    The column bias is split with the columns and added inside the linear,
    before the activation ("Full flow", ColumnParallelLinear).
    "MLP: column first, then row": GeLU acts on the shard's columns;
    SwiGLU: gate (A) and up (A2) shards of the same block, Y = silu(G) * U.

    Returns (Y, Pre): Pre is the pre-activation kept for the backward:
    None for act="none", P for "gelu", [G | U] (concatenated on columns) for
    "swiglu".
    """
    X, A, A2 = _f64(X), _f64(A), _f64(A2)
    P = X @ A
    if bias is not None:
        P = P + _f64(bias)[None, :]
    if act == "none":
        return P, None
    if act == "gelu":
        return gelu(P), P
    if act == "swiglu":
        if A2 is None:
            raise ValueError("swiglu needs the up-projection shard A2")
        U = X @ A2
        if bias2 is not None:
            U = U + _f64(bias2)[None, :]
        return silu(P) * U, np.concatenate([P, U], axis=1)
    raise ValueError(f"unknown activation {act!r}")


def row_fwd(Xi, Bi):
    """Row-parallel shard forward: the full-shape partial Z_i = X_i B_i.

    [TP/SP] "TP math": [X_1, X_2][A_1; A_2] = X_1 A_1 + X_2 A_2; each shard's
    output has the full shape and only part of the value.  No bias (added once
    after the sum) and no activation ("MLP": an activation cannot act on
    partial sums).
    """
    return _f64(Xi) @ _f64(Bi)


def sum_partials(parts, bias=None):
    """Sum of the t shard partials in ascending shard order, bias added once.

    This is the value g's forward all-reduce (and f's backward all-reduce)
    leaves on every rank: [TP/SP] "Full flow" (f/g) and "Self-test" (the row
    bias is not split and is added once after the all-reduce, else it is added
    t times); [TPcomm] Fig. 2 (two GPUs holding [1,2] and [3,4] both end with
    [4,6]).
    """
    parts = [_f64(p) for p in parts]
    if not parts:
        raise ValueError("need at least one partial")
    Z = np.zeros_like(parts[0])
    for p in parts:
        Z = Z + p
    if bias is not None:
        Z = Z + _f64(bias)[None, :]
    return Z


# ---------------------------------------------------------------------------
# Backward.  [TP/SP] "Where column and row communicate": column dX is a partial
# sum (dX = dY_1 A_1^T + dY_2 A_2^T, summed by f's backward); the row shard
# holds the full dY (g's backward is the identity) and dX_i = dY A_i^T is
# local.  "Full flow, t = 3": dW_i = X^T dY_i is complete on its own card.
# ---------------------------------------------------------------------------

def dgrad(dY, W):
    """dX = dY W^T for a layer Y = X W (W [K, N], dY [M, N] -> dX [M, K])."""
    return _f64(dY) @ _f64(W).T


def wgrad(X, dY):
    """dW = X^T dY for a layer Y = X W (X [M, K], dY [M, N] -> dW [K, N])."""
    return _f64(X).T @ _f64(dY)


def row_bwd(dZ, Xi, Bi):
    """Row-parallel shard backward.

    Returns (dX_i, dB_i, dbias): dX_i = dZ B_i^T (local), dB_i = X_i^T dZ, and
    the gradient of the replicated row bias, sum over tokens of dZ.
    """
    dZ = _f64(dZ)
    return dgrad(dZ, Bi), wgrad(Xi, dZ), dZ.sum(axis=0)


def act_bwd(dY, Pre, act):
    """Gradient through the column epilogue: dP from dY and the saved Pre.

    GeLU: dP = dY * GeLU'(P).  SwiGLU with Pre = [G | U]:
    dG = dY * U * silu'(G), dU = dY * silu(G); returns [dG | dU].
    """
    dY = _f64(dY)
    if act == "none":
        return dY
    Pre = _f64(Pre)
    if act == "gelu":
        return dY * gelu_grad(Pre)
    if act == "swiglu":
        n = dY.shape[1]
        G, U = Pre[:, :n], Pre[:, n:2 * n]
        return np.concatenate([dY * U * silu_grad(G), dY * silu(G)], axis=1)
    raise ValueError(f"unknown activation {act!r}")


def column_bwd(dY, X, A, Pre=None, act="none", A2=None):
    """Column-parallel shard backward.

    Returns (dX_part, dA, dA2, dbias, dbias2):
      dP = act_bwd(dY, Pre);
      dX_part = dP_gate A^T (+ dP_up A2^T): this shard's term of dX, a partial
      that f's backward sums over shards;
      dA = X^T dP_gate, dA2 = X^T dP_up (None unless SwiGLU);
      dbias = sum over tokens of dP_gate, dbias2 likewise for up.
    """
    dP = act_bwd(dY, Pre, act)
    if act == "swiglu":
        n = _f64(dY).shape[1]
        dPg, dPu = dP[:, :n], dP[:, n:2 * n]
        dXp = dgrad(dPg, A) + dgrad(dPu, A2)
        return dXp, wgrad(X, dPg), wgrad(X, dPu), dPg.sum(axis=0), dPu.sum(axis=0)
    return dgrad(dP, A), wgrad(X, dP), None, dP.sum(axis=0), None


# ---------------------------------------------------------------------------
# Vocab-parallel LM head and cross-entropy partials.
# [TP/SP] "Embedding and LM head: split by vocab": the LM head is split by
# vocab (column parallel over the vocabulary, 151936 / 8 = 18992 ids per
# rank); cross-entropy never gathers the logits, each token all-reduces only
# three numbers: the max, the sum of e^z and the target logit.
# Reading: the sum is taken relative to the shard's own max, and a target the
# shard does not own contributes 0.
# ---------------------------------------------------------------------------

def vocab_ce_partials(H, W, target, v0):
    """Per-token (max, sum exp(z - max), target logit) over one vocab shard.

    z = H W^T with W [V_r, K] holding vocab ids [v0, v0 + V_r).
    Returns three float64 arrays of length M.
    """
    H, W = _f64(H), _f64(W)
    target = np.asarray(target, dtype=np.int64)
    z = H @ W.T
    if not np.all(np.isfinite(z)):
        raise ValueError("non-finite logits")
    m = z.max(axis=1)
    s = np.exp(z - m[:, None]).sum(axis=1)
    vr = W.shape[0]
    owned = (target >= v0) & (target < v0 + vr)
    tgt = np.zeros(H.shape[0], dtype=np.float64)
    rows = np.nonzero(owned)[0]
    tgt[rows] = z[rows, target[rows] - v0]
    return m, s, tgt


def lse_recombine(parts):
    """Combine per-shard (max, sumexp, tgt) triples into per-token CE terms.

    M* = max_r m_r, S* = sum_r s_r e^(m_r - M*), lse = M* + ln S*,
    tgt* = sum_r tgt_r (exactly one shard owns each target), loss = lse - tgt*.
    Returns (lse, tgt, loss), float64.
    """
    ms = np.stack([_f64(p[0]) for p in parts])
    ss = np.stack([_f64(p[1]) for p in parts])
    ts = np.stack([_f64(p[2]) for p in parts])
    mstar = ms.max(axis=0)
    sstar = (ss * np.exp(ms - mstar[None, :])).sum(axis=0)
    lse = mstar + np.log(sstar)
    tgt = ts.sum(axis=0)
    return lse, tgt, lse - tgt


def vocab_ce_bwd(H, W, target, v0, lse, gscale=None):
    """Backward of the vocab-parallel cross entropy for one vocab shard.

    [TP/SP] "Embedding and LM head: split by vocab": each rank owns the
    logits z = H W_r^T of its vocab rows; with the per-token log-sum-exp
    recombined over all shards (lse, as lse_recombine returns it), the
    gradient of the per-token loss lse - z[target] w.r.t. the shard's logits
    is softmax(z) - onehot(target), the onehot entry present only on the shard
    that owns the target.  gscale [M] (default 1) is the upstream gradient of
    each token's loss.  The shard's weight gradient dW_r = dz^T H completes
    locally; dH_r = dz W_r is this shard's partial of dH (summed over shards).
    Returns (dz [M, V_r], dH_r [M, K], dW_r [V_r, K]), float64.
    """
    H, W = _f64(H), _f64(W)
    lse = _f64(lse)
    target = np.asarray(target, dtype=np.int64)
    g = np.ones(H.shape[0]) if gscale is None else _f64(gscale)
    z = H @ W.T
    dz = np.exp(z - lse[:, None])
    vr = W.shape[0]
    owned = (target >= v0) & (target < v0 + vr)
    rows = np.nonzero(owned)[0]
    dz[rows, target[rows] - v0] -= 1.0
    dz *= g[:, None]
    return dz, dz @ W, dz.T @ H


def layer_norm(h, gamma=None, beta=None, eps=1e-5):
    """LayerNorm over the last axis: (h - mean) / sqrt(var + eps) * gamma + beta, var biased (1/N)."""
    h = _f64(h)
    mu = h.mean(axis=-1, keepdims=True)
    var = ((h - mu) ** 2).mean(axis=-1, keepdims=True)
    y = (h - mu) / np.sqrt(var + eps)
    if gamma is not None:
        y = y * _f64(gamma)
    if beta is not None:
        y = y + _f64(beta)
    return y


def sp_reduce_scatter_ln(parts, r0, Mr, bias=None, resid=None, gamma=None, beta=None, eps=1e-5):
    """Sequence-parallel block boundary of one rank, on one device.

    [TP/SP] "SP: shard the activations that TP leaves whole": the all-reduce after the row-parallel layer
    becomes a reduce-scatter -- each rank keeps the sum for its own block of
    tokens -- and the residual add and LayerNorm that follow run on that
    block only; an all-gather rebuilds the full sequence before the next
    column-parallel layer.  Rank rows [r0, r0 + Mr):
      h = sum_i parts[i][r0:r0+Mr] (ascending i) + bias (once) + resid
      y = LayerNorm(h) * gamma + beta
    resid is the rank's own [Mr, N] block.  Returns (y, h), float64.
    """
    h = sum_partials([_f64(p)[r0:r0 + Mr] for p in parts], bias)
    if resid is not None:
        h = h + _f64(resid)
    return layer_norm(h, gamma, beta, eps), h


def vocab_embed_fwd(ids, E_r, v0):
    """Vocab-parallel embedding lookup of one rank.

    [TP/SP] "Embedding and LM head: split by vocab": the table is split by
    rows (vocab ids) into t blocks; rank r holds E_r = rows [v0, v0 + Vr).
    A token whose id falls in the block gets that row; any other token
    (another rank's id, or an id outside the table) gets a zero row, so the
    all-reduce (sum over ranks) leaves every token exactly its own row.
    ids: integer [M]; E_r: [Vr, K].  Returns [M, K] float64.
    """
    E = _f64(E_r)
    ids = np.asarray(ids, dtype=np.int64)
    out = np.zeros((ids.shape[0], E.shape[1]))
    own = (ids >= v0) & (ids < v0 + E.shape[0])
    out[own] = E[ids[own] - v0]
    return out


def vocab_embed_bwd(ids, dout, v0, Vr):
    """Gradient of the rank's table block under the lookup above.

    The lookup copies row id - v0 to token m, so the block's gradient row v
    is the sum of dout[m] over the tokens m whose id is v0 + v (added in
    ascending m); rows no token uses are zero.  Tokens the rank does not own
    contribute nothing.  ids: integer [M]; dout: [M, K].  Returns [Vr, K].
    """
    d = _f64(dout)
    ids = np.asarray(ids, dtype=np.int64)
    dE = np.zeros((Vr, d.shape[1]))
    for m in range(ids.shape[0]):
        if v0 <= ids[m] < v0 + Vr:
            dE[ids[m] - v0] += d[m]
    return dE


def _attn_heads(Q, K, V, n_q, n_kv):
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    d = Q.shape[1] // n_q
    if Q.shape[1] != n_q * d or K.shape[1] != n_kv * d or V.shape[1] != n_kv * d or n_q % n_kv != 0:
        raise ValueError("head layout does not match")
    return Q, K, V, d, n_q // n_kv


def _attn_scores(Qh, Kg, causal, scale):
    s = (Qh @ Kg.T) * scale
    if causal:
        S = s.shape[0]
        s = np.where(np.arange(S)[None, :] > np.arange(S)[:, None], -np.inf, s)
    return s


def attention_fwd(Q, K, V, n_q, n_kv, causal=True, scale=None):
    """Attention core of one rank's heads, between the QKV and W_O projections.

    [TP/SP] "Attention: split by head": every head is computed on its own, so
    the rank runs scaled dot-product attention for its n_q query heads; with
    GQA (32 query / 8 KV heads at t = 8: 4 query heads and 1 KV head per rank)
    query head h reads KV head h // (n_q / n_kv).  Per head:
      s = Q_h K_g^T * scale (scale = 1/sqrt(d)), keys after the query masked
      when causal, P = softmax(s) over keys, O_h = P V_g, lse = log sum exp s.
    Q [S, n_q*d], K and V [S, n_kv*d] (head h in columns [h*d, (h+1)*d)).
    Returns O [S, n_q*d] and lse [n_q, S], float64.
    """
    Q, K, V, d, group = _attn_heads(Q, K, V, n_q, n_kv)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    S = Q.shape[0]
    O = np.zeros((S, n_q * d))
    lse = np.zeros((n_q, S))
    for h in range(n_q):
        g = h // group
        s = _attn_scores(Q[:, h * d:(h + 1) * d], K[:, g * d:(g + 1) * d], causal, scale)
        mx = s.max(axis=1, keepdims=True)
        e = np.exp(s - mx)
        tot = e.sum(axis=1, keepdims=True)
        O[:, h * d:(h + 1) * d] = (e / tot) @ V[:, g * d:(g + 1) * d]
        lse[h] = (mx + np.log(tot))[:, 0]
    return O, lse


def attention_bwd(Q, K, V, dO, n_q, n_kv, causal=True, scale=None):
    """Gradients of the attention core above (the pages print no backward).

    Textbook softmax-attention gradients per head, with P recomputed from s:
      dV_g += P^T dO_h,  dP = dO_h V_g^T,
      dS = P * (dP - rowsum(P * dP)),
      dQ_h = dS K_g * scale,  dK_g += dS^T Q_h * scale.
    A KV head's gradient sums over the query heads that read it (ascending h).
    Returns dQ [S, n_q*d], dK, dV [S, n_kv*d], float64.
    """
    Q, K, V, d, group = _attn_heads(Q, K, V, n_q, n_kv)
    dO = _f64(dO)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    dQ, dK, dV = np.zeros_like(Q), np.zeros_like(K), np.zeros_like(V)
    for h in range(n_q):
        g = h // group
        qs, ks = slice(h * d, (h + 1) * d), slice(g * d, (g + 1) * d)
        s = _attn_scores(Q[:, qs], K[:, ks], causal, scale)
        e = np.exp(s - s.max(axis=1, keepdims=True))
        P = e / e.sum(axis=1, keepdims=True)
        dV[:, ks] += P.T @ dO[:, qs]
        dP = dO[:, qs] @ V[:, ks].T
        dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
        dQ[:, qs] = dS @ K[:, ks] * scale
        dK[:, ks] += dS.T @ Q[:, qs] * scale
    return dQ, dK, dV
