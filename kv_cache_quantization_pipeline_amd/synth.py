"""Seeded synthetic inputs shared by the oracle-side and GPU-side tests and the bench.

This module holds none of the method's arithmetic: it only draws random K/V
activations, queries, page tables and lengths, in numpy, host memory.

K/V statistics (one draw for K, then one for V, per workload):
  base  ~ N(0, 1)                      [n_tok, Hkv, 128]
  tok   = exp(0.5 * N(0, 1))           [n_tok, Hkv]       (log-normal(0, 0.5) per-token scale)
  4 outlier channels per head, fixed for the whole workload, scaled x20
  X = base * tok[..., None], outliers x20, cast float32 -> float16 (round to nearest even)
These mimic the two properties the pages build the method around: a few
outlier channels (spread by the Hadamard rotation) and uneven per-token scales
(removed by the row/column normalisation).
"""
from __future__ import annotations

import numpy as np

HEAD_DIM = 128
BLOCK = 128


def gen_kv_one(rng: np.random.Generator, n_tok: int, n_kv_heads: int) -> np.ndarray:
    base = rng.standard_normal((n_tok, n_kv_heads, HEAD_DIM), dtype=np.float32)
    tok = np.exp(np.float32(0.5) * rng.standard_normal((n_tok, n_kv_heads), dtype=np.float32))
    base *= tok[..., None]
    for h in range(n_kv_heads):
        ch = rng.choice(HEAD_DIM, 4, replace=False)
        base[:, h, ch] *= np.float32(20.0)
    return base.astype(np.float16)


def gen_kv(seed: int, n_tok: int, n_kv_heads: int):
    """(k, v) float16 [n_tok, Hkv, 128]."""
    rng = np.random.default_rng(seed)
    k = gen_kv_one(rng, n_tok, n_kv_heads)
    v = gen_kv_one(rng, n_tok, n_kv_heads)
    return k, v


def gen_q(seed: int, batch: int, n_q_heads: int) -> np.ndarray:
    """float16 [B, Hq, 128] ~ N(0, 1); drawn from its own stream (seed + 1000)."""
    rng = np.random.default_rng(seed + 1000)
    return rng.standard_normal((batch, n_q_heads, HEAD_DIM), dtype=np.float32).astype(np.float16)


def gen_page_perm(seed: int, total_pages: int) -> np.ndarray:
    rng = np.random.default_rng(seed + 2000)
    return rng.permutation(total_pages).astype(np.int32)


def gen_lengths(seed: int, n: int, lo: int, hi: int) -> np.ndarray:
    rng = np.random.default_rng(seed + 3000)
    return rng.integers(lo, hi + 1, size=n).astype(np.int32)


def gen_formats(seed: int, n: int) -> np.ndarray:
    """Per-sequence format choice for mixed-format workloads: 0 = k4v2, 1 = k8v8."""
    rng = np.random.default_rng(seed + 4000)
    return (rng.random(n) < 0.5).astype(np.int32)


def tiles_view(x: np.ndarray) -> np.ndarray:
    """[n_tok, Hkv, 128] -> [n_tok/128, 128, Hkv, 128] (the quantizer's input layout)."""
    n_tok, hkv, d = x.shape
    assert n_tok % BLOCK == 0
    return x.reshape(n_tok // BLOCK, BLOCK, hkv, d)


# Workloads (sizes of the pages' settings: Qwen3-32B at TP=2 with 16K context,
# Llama-3-70B at long context, a ragged continuous-batching step).
WORKLOADS = {
    "single_tile": dict(seed=0, n_kv_heads=1, n_q_heads=1, batch=1, ctx=128),
    "bulk_quantize_qwen3_32b_tp2": dict(seed=1, n_kv_heads=4, batch=8, ctx=16384),
    "decode_gqa8_b32_ctx16k": dict(seed=2, n_kv_heads=4, n_q_heads=32, batch=32, ctx=16384),
    "decode_long_b4_ctx128k": dict(seed=3, n_kv_heads=1, n_q_heads=8, batch=4, ctx=131072),
    "ragged_mixed_64seq": dict(seed=4, n_kv_heads=4, n_q_heads=32, batch=64, ctx_lo=1024, ctx_hi=32768),
}
