"""Oracle attention in float64 (test infrastructure).

What is computed: each query token of the current frame or chunk attends to
every visible KV token with plain softmax attention, no mask, scale
1/sqrt(head_dim) unless given ("LingBot-Map Paged KV Cache", section 1: a new
frame attends to the cached KV of earlier frames; section 2: the visible page
table needs no custom mask; "vLLM-Omni RFC #2727: Reconstruction Engine",
section 1: global attention over the tokens of the most recent
sliding_window_num chunks including the current one, and section 2.2: VGGT's
global self-attention over all frame tokens).

    O[q, h] = sum_k softmax_k(s * <Q[q, h], K[h, k]>) V[h, k]
    lse[q, h] = log sum_k exp(s * <Q[q, h], K[h, k]>)

Query rows are processed in blocks so that no Lq x Lk matrix larger than
block x Lk exists (the RFC's 100-frame example is a 137,400-token sequence
whose score matrix would need about 35 GB, section 2.3).  An empty key set
gives O = 0 and lse = -inf (the pages do not cover it; this is the reading
used on both sides).
"""
from __future__ import annotations

import math
from typing import Iterable, List, Sequence, Tuple

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns as float64 (bf16 is the top half of an fp32)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def to_f64(x: np.ndarray) -> np.ndarray:
    """Store-dtype array (uint16 bf16 patterns or float32) to float64, exactly."""
    if x.dtype == np.uint16:
        return bf16_bits_to_f64(x)
    return np.asarray(x, dtype=np.float64)


def attention_f64(q: np.ndarray, k: np.ndarray, v: np.ndarray, sm_scale: float | None = None,
                  block: int = 1024) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax attention in float64.

    q: [Lq, H, d]; k, v: [H, Lk, d] (any real dtype; converted to float64).
    Returns O [Lq, H, d] and lse [Lq, H] (natural log of the sum of exp of
    scaled scores).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    lq, nh, d = q.shape
    assert k.shape[0] == nh and k.shape[2] == d and v.shape == k.shape
    s = (1.0 / math.sqrt(d)) if sm_scale is None else float(sm_scale)
    out = np.zeros((lq, nh, d), np.float64)
    lse = np.full((lq, nh), -np.inf, np.float64)
    if k.shape[1] == 0:
        return out, lse
    for h in range(nh):
        kh, vh = k[h], v[h]
        for r0 in range(0, lq, block):
            qb = q[r0:r0 + block, h, :]
            sc = s * (qb @ kh.T)                    # [b, Lk]
            m = sc.max(axis=1, keepdims=True)
            p = np.exp(sc - m)
            l = p.sum(axis=1, keepdims=True)
            out[r0:r0 + block, h, :] = (p @ vh) / l
            lse[r0:r0 + block, h] = (m + np.log(l))[:, 0]
    return out, lse


def brute_attention(q: Sequence, k: Sequence, v: Sequence, sm_scale: float) -> List:
    """Scalar loops straight from the definition (tiny shapes only).

    q: [Lq][H][d], k, v: [H][Lk][d] nested sequences of floats.
    Returns (O as nested lists [Lq][H][d], lse [Lq][H]).
    """
    lq, nh, d = len(q), len(q[0]), len(q[0][0])
    out = [[[0.0] * d for _ in range(nh)] for _ in range(lq)]
    lse = [[-math.inf] * nh for _ in range(lq)]
    for i in range(lq):
        for h in range(nh):
            lk = len(k[h])
            if lk == 0:
                continue
            scores = []
            for j in range(lk):
                acc = 0.0
                for c in range(d):
                    acc += float(q[i][h][c]) * float(k[h][j][c])
                scores.append(sm_scale * acc)
            w = [math.exp(x) for x in scores]
            z = math.fsum(w)
            for c in range(d):
                out[i][h][c] = math.fsum(w[j] * float(v[h][j][c]) for j in range(lk)) / z
            lse[i][h] = math.log(z)
    return out, lse


def merge_partials(parts: Iterable[Tuple[np.ndarray, np.ndarray]]) -> Tuple[np.ndarray, np.ndarray]:
    """Combine attention results computed over disjoint key subsets.

    Each part is (O_i [.., d] normalised over its subset, lse_i [..]).  With
    lse = log sum_i exp(lse_i), the full result is O = sum_i exp(lse_i - lse) O_i.
    Parts with lse_i = -inf (empty subsets) contribute nothing.
    """
    parts = list(parts)
    lses = np.stack([np.asarray(p[1], np.float64) for p in parts])
    outs = np.stack([np.asarray(p[0], np.float64) for p in parts])
    m = lses.max(axis=0)
    finite = np.isfinite(m)
    msafe = np.where(finite, m, 0.0)
    w = np.where(np.isfinite(lses), np.exp(lses - msafe[None]), 0.0)
    z = w.sum(axis=0)
    lse = np.where(finite, msafe + np.log(np.where(z > 0, z, 1.0)), -np.inf)
    o = (w[..., None] * outs).sum(axis=0) / np.where(z > 0, z, 1.0)[..., None]
    return o, lse


def dense_history_attention(q: np.ndarray, history_k: List[np.ndarray], history_v: List[np.ndarray],
                            patch_tokens: int, num_scale: int, window: int,
                            sm_scale: float | None = None) -> Tuple[np.ndarray, np.ndarray]:
    """Attention over tokens selected straight from the unit history, no pages involved.

    history_k/v: the cached units in append order, each [patch + special, H, d]
    (store dtype).  Visible tokens ("LingBot-Map Paged KV Cache", section 2):
    patch tokens of the first num_scale units, patch tokens of the last
    `window` non-scale units (all of them when window <= 0), then the special
    tokens of every cached unit, in append order.
    """
    n = len(history_k)
    scale_ids = list(range(min(n, num_scale)))
    rest = list(range(min(n, num_scale), n))
    win_ids = rest if window <= 0 else rest[-window:] if rest else []
    ks, vs = [], []
    for i in scale_ids + win_ids:
        ks.append(history_k[i][:patch_tokens])
        vs.append(history_v[i][:patch_tokens])
    for i in range(n):
        ks.append(history_k[i][patch_tokens:])
        vs.append(history_v[i][patch_tokens:])
    k = to_f64(np.concatenate(ks, axis=0)).transpose(1, 0, 2)
    v = to_f64(np.concatenate(vs, axis=0)).transpose(1, 0, 2)
    return attention_f64(to_f64(q), k, v, sm_scale)
