"""Seeded synthetic inputs shared by the HIP path's tests/bench and the CPU oracle.

This module holds no arithmetic of the method: it only draws seeded random
tensors (numpy PCG64), rounds them to the storage dtype (bf16 by
round-to-nearest-even, or fp32), and describes the workload shapes.  Both sides
receive the same bytes: the GPU gets the raw bf16/fp32 words, the oracle gets
the same values widened to float64 (exact, since every bf16 value is an fp32
value and every fp32 value is an fp64 value).

Workloads (all inputs synthetic; no dataset or trained weight is involved):

* ``c1`` fp32 GeLU MLP, t=4 simulated shards: X[64,256] ~N(0,1),
  A[256,1024] and B[1024,256] ~N(0,0.02), dY ~N(0,1).
* ``c2`` Qwen3-8B-shaped SwiGLU MLP shard, t=8: X[8192,4096], gate/up
  [4096,1536], down [1536,4096], dZ[8192,4096]; bf16.
* ``c3`` attention projection shard, t=8 (GQA 32 q / 8 kv heads, head_dim 128):
  QKV column [4096,768], W_O row [512,4096]; bf16.
* ``c4`` GeLU MLP shard, t=4 at h=8192: X[4096,8192], A_i and B_i
  [8192,8192] ~N(0,0.01); bf16.
* ``c5`` vocab-parallel LM head shard (one of 8): H[8192,4096],
  W_r[18992,4096] ~N(0,0.02), targets uniform int32 in [0,151936).

The second argument of N(0, s) is the standard deviation.
"""
from __future__ import annotations

import dataclasses

import numpy as np

BF16 = "bf16"
FP32 = "fp32"


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the 16-bit patterns as uint16.  Inputs here are finite draws, so
    NaN handling is not needed; a non-finite input raises.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("bf16 rounding expects finite values")
    u = x.view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float32 exactly."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class Tensor:
    """A seeded input tensor: storage words for the GPU and exact values for the oracle."""

    dtype: str          # BF16 or FP32
    raw: np.ndarray     # uint16 (bf16 bit patterns) or float32, C-contiguous
    shape: tuple

    @property
    def f64(self) -> np.ndarray:
        if self.dtype == BF16:
            return bf16_bits_to_f32(self.raw).astype(np.float64)
        return self.raw.astype(np.float64)

    @property
    def f32(self) -> np.ndarray:
        if self.dtype == BF16:
            return bf16_bits_to_f32(self.raw)
        return self.raw


def normal(seed: int, shape, std: float, dtype: str) -> Tensor:
    """N(0, std) draws from PCG64(seed), stored as ``dtype``."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if dtype == BF16:
        return Tensor(BF16, bf16_bits_from_f32(x), tuple(shape))
    if dtype == FP32:
        return Tensor(FP32, np.ascontiguousarray(x), tuple(shape))
    raise ValueError(dtype)


def small_ints(seed: int, shape, lo: int, hi: int, dtype: str) -> Tensor:
    """Uniform integers in [lo, hi] stored as ``dtype`` (exact in bf16 for |v| <= 256)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.integers(lo, hi + 1, size=shape).astype(np.float32)
    if dtype == BF16:
        return Tensor(BF16, bf16_bits_from_f32(x), tuple(shape))
    return Tensor(FP32, x, tuple(shape))


def targets(seed: int, n: int, vocab: int) -> np.ndarray:
    """Uniform int32 token ids in [0, vocab)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(0, vocab, size=n, dtype=np.int64).astype(np.int32)


def from_values(values, dtype: str) -> Tensor:
    """Wrap exact small values (worked examples) as a Tensor of ``dtype``."""
    x = np.asarray(values, dtype=np.float32)
    if dtype == BF16:
        bits = bf16_bits_from_f32(x)
        if not np.array_equal(bf16_bits_to_f32(bits), x):
            raise ValueError("value not exact in bf16")
        return Tensor(BF16, bits, x.shape)
    return Tensor(FP32, np.ascontiguousarray(x), x.shape)


# ---------------------------------------------------------------------------
# Workload descriptions.  Seeds follow 1000*config + tensor index.
# ---------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class MLPShape:
    name: str
    dtype: str
    act: str            # "gelu" | "swiglu" | "none"
    t: int              # tensor-parallel degree (number of simulated shards)
    M: int              # tokens
    H: int              # model width (column K, row N)
    F: int              # full intermediate width (column N summed over shards)
    std_x: float
    std_w: float
    std_dy: float
    seed: int

    @property
    def Fi(self) -> int:
        return self.F // self.t


C1 = MLPShape("c1_fp32_gelu_t4", FP32, "gelu", 4, 64, 256, 1024, 1.0, 0.02, 1.0, 1000)
C2 = MLPShape("c2_qwen3_8b_swiglu_t8", BF16, "swiglu", 8, 8192, 4096, 12288, 1.0, 0.02, 1.0, 2000)
C4 = MLPShape("c4_gelu_t4_h8192", BF16, "gelu", 4, 4096, 8192, 32768, 1.0, 0.01, 1.0, 4000)


@dataclasses.dataclass(frozen=True)
class AttnProjShape:
    name: str = "c3_attn_proj_t8"
    M: int = 8192
    H: int = 4096
    n_qkv: int = 768     # (4 q + 1 k + 1 v) heads x 128 per shard
    k_o: int = 512       # 4 q heads x 128 per shard
    std_w: float = 0.02
    seed: int = 3000


C3 = AttnProjShape()


@dataclasses.dataclass(frozen=True)
class VocabShape:
    name: str = "c5_lm_head_ce_shard"
    M: int = 8192
    H: int = 4096
    vocab: int = 151936
    shards: int = 8
    std_w: float = 0.02
    seed: int = 5000

    @property
    def Vr(self) -> int:
        return self.vocab // self.shards


C5 = VocabShape()


def mlp_shard_inputs(cfg: MLPShape, shard: int, M: int | None = None):
    """Inputs of one shard of an MLP block, drawn independently per shard.

    The full weight is never drawn: shard ``i`` of the column weight and
    shard ``i`` of the row weight get their own seeds, so any single shard can
    be generated without the others (the full-weight invariants are tested on
    small shapes where all shards are drawn and concatenated).
    Returns a dict of Tensor: X, A (gate for SwiGLU), A2 (up, SwiGLU only),
    B (row weight shard), dZ.
    """
    M = cfg.M if M is None else M
    s = cfg.seed
    out = {
        "X": normal(s + 1, (M, cfg.H), cfg.std_x, cfg.dtype),
        "A": normal(s + 10 + 3 * shard, (cfg.H, cfg.Fi), cfg.std_w, cfg.dtype),
        "B": normal(s + 12 + 3 * shard, (cfg.Fi, cfg.H), cfg.std_w, cfg.dtype),
        "dZ": normal(s + 2, (M, cfg.H), cfg.std_dy, cfg.dtype),
    }
    if cfg.act == "swiglu":
        out["A2"] = normal(s + 11 + 3 * shard, (cfg.H, cfg.Fi), cfg.std_w, cfg.dtype)
    return out


def attn_proj_inputs(cfg: AttnProjShape = C3, M: int | None = None):
    M = cfg.M if M is None else M
    s = cfg.seed
    return {
        "X": normal(s + 1, (M, cfg.H), 1.0, BF16),
        "Wqkv": normal(s + 2, (cfg.H, cfg.n_qkv), cfg.std_w, BF16),
        "attn": normal(s + 3, (M, cfg.k_o), 1.0, BF16),
        "Wo": normal(s + 4, (cfg.k_o, cfg.H), cfg.std_w, BF16),
        "dZ": normal(s + 5, (M, cfg.H), 1.0, BF16),
        "dQKV": normal(s + 6, (M, cfg.n_qkv), 1.0, BF16),
    }


def vocab_inputs(cfg: VocabShape = C5, shard: int = 0, M: int | None = None, Vr: int | None = None):
    M = cfg.M if M is None else M
    Vr = cfg.Vr if Vr is None else Vr
    s = cfg.seed
    return {
        "H": normal(s + 1, (M, cfg.H), 1.0, BF16),
        "W": normal(s + 10 + shard, (Vr, cfg.H), cfg.std_w, BF16),
        "target": targets(s + 2, M, cfg.vocab),
        "v0": shard * Vr,
    }
