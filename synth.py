"""Seeded synthetic inputs shared by the oracle-side and device-side tests and the bench.

This module holds no arithmetic of the attention method: it only draws
standard-normal tensors from a counter-keyed NumPy generator and rounds them to
the storage type (bf16 with round-to-nearest-even, or fp32).  Both sides consume
the resulting bit patterns unchanged.

Workload shapes follow the pages: a LingBot-Map frame carries 256 patch tokens
and 6 special tokens (camera/register/scale) ("LingBot-Map Paged KV Cache",
section 2, the page-type table), and a VGGT image becomes about 1374 tokens
(vLLM-Omni RFC #2727, section 2.2, the architecture figure).  The pages stream
real videos; normal draws of those shapes stand in for them.
"""
from __future__ import annotations

import numpy as np

KIND_Q, KIND_K, KIND_V = 0, 1, 2


def rng_for(seed: int, layer: int, unit: int, kind: int) -> np.random.Generator:
    """Independent stream per (seed, layer, unit, tensor kind)."""
    return np.random.default_rng([int(seed), int(layer), int(unit), int(kind)])


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round-to-nearest-even) and return the 16-bit patterns (uint16).

    NaN inputs map to a quiet NaN pattern.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r = r.copy()
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32 (for building inputs only)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_tokens(seed: int, layer: int, unit: int, kind: int, tokens: int, heads: int,
                  head_dim: int, dtype: str = "bf16", scale: float = 1.0) -> np.ndarray:
    """[tokens, heads, head_dim] draws ~ N(0, scale^2).

    dtype "bf16" returns uint16 bit patterns; "f32" returns float32.
    """
    x = rng_for(seed, layer, unit, kind).standard_normal((tokens, heads, head_dim), dtype=np.float32)
    if scale != 1.0:
        x = (x * np.float32(scale)).astype(np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "f32":
        return x
    raise ValueError(f"unknown dtype {dtype!r}")


def frame_qkv(seed: int, layer: int, unit: int, tokens: int, heads: int, head_dim: int,
              dtype: str = "bf16", q_scale: float = 1.0):
    """(q, k, v) for one appended unit, each [tokens, heads, head_dim]."""
    q = normal_tokens(seed, layer, unit, KIND_Q, tokens, heads, head_dim, dtype, q_scale)
    k = normal_tokens(seed, layer, unit, KIND_K, tokens, heads, head_dim, dtype)
    v = normal_tokens(seed, layer, unit, KIND_V, tokens, heads, head_dim, dtype)
    return q, k, v
