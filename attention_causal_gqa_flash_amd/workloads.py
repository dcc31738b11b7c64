"""Seeded synthetic workloads for causal grouped-query attention.

This module only draws inputs: it holds none of attention's arithmetic, so
that the GPU path and the CPU oracle can both take their inputs from it
without sharing any computation.

Shapes come from the pages' workloads:
  * GQA 12/4 heads with head dim 64 at batch x sequence 4 x 1024 is the
    RustingBrain dense transformer ("RustingBrain" docs, "Where it stands
    against PyTorch and TensorFlow").
  * Sequences of 128 and 512 tokens are those of tang's forward+backward and
    transformer-block results ("tang -- differentiable computing in Rust",
    hero line and "A transformer").
  * The 4k context is tang-llm's 4k-context decode ("An LLM").
  * 32 query heads, 8 key/value heads and head dim 128 are the long-context
    and decode shapes used throughout.

Values are i.i.d. standard normal, drawn in float32 from
``numpy.random.default_rng(seed)`` in the order Q, K, V, dO (decode: q, K
cache, V cache).  bf16 workloads round each drawn value to the nearest bf16
(ties to even) after any scaling; both the GPU and the oracle receive exactly
these rounded values.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class TrainConfig:
    """A causal fwd+bwd workload."""
    name: str
    dtype: str          # "f32" or "bf16": the dtype of q, k, v and dO
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    seed: int
    dout_scale: float = 1.0
    causal: bool = True

    @property
    def scale(self) -> float:
        # the softmax scale 1/sqrt(d), as the float32 value handed to the GPU
        return float(np.float32(1.0 / math.sqrt(self.d)))

    @property
    def pairs(self) -> int:
        """Unmasked (query, key) pairs over all batches and query heads."""
        per_head = self.N * (self.N + 1) // 2 if self.causal else self.N * self.N
        return self.B * self.Hq * per_head

    @property
    def fwd_flop(self) -> int:
        # 4*d per unmasked pair: QK^T and PV, 2 flop per multiply-add each
        return 4 * self.d * self.pairs

    @property
    def bwd_flop(self) -> int:
        # 10*d per pair: recomputed QK^T, dO V^T, P^T dO, dS^T Q, dS K
        return 10 * self.d * self.pairs


@dataclass(frozen=True)
class DecodeConfig:
    """A one-token split-KV decode workload against a full cache."""
    name: str
    dtype: str
    B: int
    Hq: int
    Hkv: int
    L: int
    d: int
    n_splits: int
    seed: int

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.d)))

    def algorithmic_bytes(self) -> int:
        """K and V caches + q read once, O (f32) and LSE (f32) written once."""
        esz = 2 if self.dtype == "bf16" else 4
        kv = 2 * self.B * self.Hkv * self.L * self.d * esz
        q = self.B * self.Hq * self.d * esz
        out = self.B * self.Hq * self.d * 4 + self.B * self.Hq * 4
        return kv + q + out


@dataclass(frozen=True)
class DecodeAppendConfig:
    """One decode step of B sequences of their own lengths against caches of
    capacity L_cap, appending the new token (lengths: seq_lens)."""
    name: str
    dtype: str
    B: int
    Hq: int
    Hkv: int
    L_cap: int
    d: int
    n_splits: int
    seq_lens: tuple
    seed: int

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.d)))

    def algorithmic_bytes(self) -> int:
        """Per sequence: its n cached K and V rows and the new k, v read, the new
        row written to both caches, q read, O (f32) and LSE (f32) written."""
        esz = 2 if self.dtype == "bf16" else 4
        row = self.Hkv * self.d * esz                 # one token of one cache
        kv = sum(2 * n * row for n in self.seq_lens)
        new = self.B * 2 * row * 2                    # k_new, v_new read; cache rows written
        q = self.B * self.Hq * self.d * esz
        out = self.B * self.Hq * self.d * 4 + self.B * self.Hq * 4
        return kv + new + q + out


@dataclass(frozen=True)
class ChunkConfig:
    """A causal forward of Nq new tokens against Nk >= Nq keys (the queries are
    the last Nq positions: a prefill chunk against a cache)."""
    name: str
    dtype: str
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nk: int
    d: int
    seed: int

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.d)))

    @property
    def pairs(self) -> int:
        """Visible (query, key) pairs: query i sees keys 0 .. i + Nk - Nq."""
        off = self.Nk - self.Nq
        return self.B * self.Hq * (self.Nq * (off + 1) + self.Nq * (self.Nq - 1) // 2)

    @property
    def fwd_flop(self) -> int:
        return 4 * self.d * self.pairs


C1 = TrainConfig("tiny_f32_b1_h2x1_n64_d16", "f32", 1, 2, 1, 64, 16, seed=1001)
C2 = TrainConfig("gqa12x4_b4_n1024_d64", "bf16", 4, 12, 4, 1024, 64, seed=1002, dout_scale=0.1)
C3_128 = TrainConfig("gqa32x8_b1_n128_d128", "bf16", 1, 32, 8, 128, 128, seed=1003)
C3_512 = TrainConfig("gqa32x8_b1_n512_d128", "bf16", 1, 32, 8, 512, 128, seed=1003)
C4 = TrainConfig("gqa32x8_b1_n4096_d128", "bf16", 1, 32, 8, 4096, 128, seed=1004)
C5 = DecodeConfig("decode_gqa32x8_l4096_d128_s16", "bf16", 1, 32, 8, 4096, 128, 16, seed=1005)

# 8 sequences of 512, 1024, ..., 4096 tokens after the step (a length mix over
# the 4k context of the decode workload)
C6 = DecodeAppendConfig("decode_append_gqa32x8_b8_lc4096_d128_s16", "bf16", 8, 32, 8, 4096, 128, 16,
                        tuple(512 * (b + 1) - 1 for b in range(8)), seed=1006)

# the last 512 tokens of the 4k context prefilled against the first 3584
C7 = ChunkConfig("chunk_gqa32x8_nq512_nk4096_d128", "bf16", 1, 32, 8, 512, 4096, 128, seed=1007)

TRAIN_CONFIGS = {c.name: c for c in (C1, C2, C3_128, C3_512, C4)}
DECODE_CONFIGS = {C5.name: C5}


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32.

    Input preparation only: the rounded values are the inputs both sides see.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def _draw(rng: np.random.Generator, shape, dtype: str, mul: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if mul != 1.0:
        x = (x * np.float32(mul)).astype(np.float32)
    return round_bf16(x) if dtype == "bf16" else x


def train_inputs(cfg: TrainConfig, seed: int | None = None) -> dict:
    """q, k, v, dout as float32 arrays (bf16-representable when cfg.dtype is bf16)."""
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    q = _draw(rng, (cfg.B, cfg.Hq, cfg.N, cfg.d), cfg.dtype)
    k = _draw(rng, (cfg.B, cfg.Hkv, cfg.N, cfg.d), cfg.dtype)
    v = _draw(rng, (cfg.B, cfg.Hkv, cfg.N, cfg.d), cfg.dtype)
    do = _draw(rng, (cfg.B, cfg.Hq, cfg.N, cfg.d), cfg.dtype, cfg.dout_scale)
    return {"q": q, "k": k, "v": v, "dout": do}


def decode_inputs(cfg: DecodeConfig, seed: int | None = None) -> dict:
    """q [B,Hq,d] and the caches [B,Hkv,L,d] as float32 arrays."""
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    q = _draw(rng, (cfg.B, cfg.Hq, cfg.d), cfg.dtype)
    kc = _draw(rng, (cfg.B, cfg.Hkv, cfg.L, cfg.d), cfg.dtype)
    vc = _draw(rng, (cfg.B, cfg.Hkv, cfg.L, cfg.d), cfg.dtype)
    return {"q": q, "k_cache": kc, "v_cache": vc}


def decode_append_inputs(cfg: DecodeAppendConfig, seed: int | None = None) -> dict:
    """q [B,Hq,d], k_new / v_new [B,Hkv,d], the caches [B,Hkv,L_cap,d] as float32
    arrays and seq_lens [B] int32."""
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    q = _draw(rng, (cfg.B, cfg.Hq, cfg.d), cfg.dtype)
    kn = _draw(rng, (cfg.B, cfg.Hkv, cfg.d), cfg.dtype)
    vn = _draw(rng, (cfg.B, cfg.Hkv, cfg.d), cfg.dtype)
    kc = _draw(rng, (cfg.B, cfg.Hkv, cfg.L_cap, cfg.d), cfg.dtype)
    vc = _draw(rng, (cfg.B, cfg.Hkv, cfg.L_cap, cfg.d), cfg.dtype)
    return {"q": q, "k_new": kn, "v_new": vn, "k_cache": kc, "v_cache": vc,
            "seq_lens": np.asarray(cfg.seq_lens, dtype=np.int32)}


def chunk_inputs(cfg: ChunkConfig, seed: int | None = None) -> dict:
    """q [B,Hq,Nq,d] and k, v [B,Hkv,Nk,d] as float32 arrays."""
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    q = _draw(rng, (cfg.B, cfg.Hq, cfg.Nq, cfg.d), cfg.dtype)
    k = _draw(rng, (cfg.B, cfg.Hkv, cfg.Nk, cfg.d), cfg.dtype)
    v = _draw(rng, (cfg.B, cfg.Hkv, cfg.Nk, cfg.d), cfg.dtype)
    return {"q": q, "k": k, "v": v}


def random_train(B, Hq, Hkv, N, d, dtype="bf16", seed=0, dout_scale=1.0) -> dict:
    """Inputs of an arbitrary shape, same recipe (used for extra parity shapes)."""
    cfg = TrainConfig("adhoc", dtype, B, Hq, Hkv, N, d, seed=seed, dout_scale=dout_scale)
    return train_inputs(cfg)
