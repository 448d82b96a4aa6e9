"""Parity at the exact shapes bench.py's optional workloads time, against the oracle.

* stream_batched: 6 LingBot-shaped streams (16 heads, 256 + 6 tokens per
  frame, 8 scale frames, 64-frame window) streamed for 1,000 frames each,
  one kvc_attend_batch launch over all six (576 table entries): every
  stream's 262 queries at the last frame against the oracle.
* chunked with per-layer page subsets (`--keep-ratio 0.25`, "vLLM-Omni RFC
  #2727", section 3.4: AVGGT random KV subsets): 10,992 queries against a
  quarter of the 172 pages of a 43,968-key window, sampled rows.
* chunked with FP8 pages (`--kv-dtype fp8`, RFC #2727 section 3.4 item 5):
  10,992 queries against 43,968 keys of E4M3 pages, sampled rows including
  the 512-row tile boundaries.
Inputs cycle a small bank of seeded frames (values do not change the launch
configuration); the oracle appends exactly the same bits.
"""
import numpy as np
import pytest

import synth
from gpu_helpers import check_attention, log, to_dev
from oracle import OracleCache, OracleConfig, attention_f64, subset_table
from oracle import to_f64 as bits_f64

pytestmark = pytest.mark.gpu

CHUNK_ROWS = [0, 1, 31, 32, 255, 256, 511, 512, 513, 1023, 1024, 5119, 5120, 10239, 10240, 10991]


def _chunk_rows(tokens, seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([rng.choice(tokens, 40, replace=False), CHUNK_ROWS]))


def test_stream_batched_six_streams_1000_frames():
    import torch
    from paged_sliding_window_kv_amd import attend_batch, shared_pool_caches
    B, H, P, X, S, W, frames = 6, 16, 256, 6, 8, 64, 1000
    log(f"stream_batched: {B} streams x {frames} frames, one launch")
    kw = dict(num_heads=H, dtype="bf16", patch_tokens=P, special_tokens=X, num_scale_units=S, window_units=W,
              max_units=frames)
    caches = shared_pool_caches(B, "cuda", **kw)
    oracles = [OracleCache(OracleConfig(num_heads=H, head_dim=64, patch_tokens=P, special_tokens=X,
                                        num_scale_units=S, window_units=W, max_units=frames, store_dtype="bf16"))
               for _ in range(B)]
    bank = [synth.frame_qkv(71, 0, i, P + X, H, 64, "bf16") for i in range(7)]
    dev_bank = [tuple(to_dev(x, "bf16") for x in f) for f in bank]
    for t in range(frames):
        for i in range(B):
            b = (t + 3 * i) % len(bank)
            oracles[i].append(bank[b][1], bank[b][2])
            caches[i].append(dev_bank[b][1], dev_bank[b][2])
        if t % 250 == 0:
            log(f"  frame {t}")
    qs = [bank[(5 * i + 1) % len(bank)][0] for i in range(B)]
    qo = np.arange(0, B * (P + X) + 1, P + X, dtype=np.int32)
    assert sum(len(c.visible_table()[0]) for c in caches) == 576
    o, lse = attend_batch(caches, to_dev(np.concatenate(qs), "bf16"), qo)
    torch.cuda.synchronize()
    for i in range(B):
        gk, gv = oracles[i].gather()
        assert gk.shape[1] == 24432
        assert caches[i].visible_table()[0].tolist() == oracles[i].visible_table()[0]
        ro, rl = attention_f64(bits_f64(qs[i]), bits_f64(gk), bits_f64(gv))
        check_attention(o[qo[i]:qo[i + 1]], lse[qo[i]:qo[i + 1]], ro, rl, "bf16", f"stream {i} Lk=24432")


def _chunk_caches(dtype, seed):
    from paged_sliding_window_kv_amd import KvCache
    H, T, W = 16, 8 * 1374, 4
    dc = KvCache(num_heads=H, dtype=dtype, patch_tokens=T, special_tokens=0, num_scale_units=0, window_units=W,
                 max_units=W + 1, device="cuda")
    oc = OracleCache(OracleConfig(num_heads=H, head_dim=64, patch_tokens=T, special_tokens=0, num_scale_units=0,
                                  window_units=W, max_units=W + 1, store_dtype=dtype))
    bank = [synth.frame_qkv(seed, 0, i, T, H, 64, "bf16") for i in range(2)]
    for c in range(W + 1):
        _, k, v = bank[c % 2]
        oc.append(k, v)
        dc.append(to_dev(k, "bf16"), to_dev(v, "bf16"))
    return dc, oc, bank[(W + 1) % 2][0]


def test_chunked_page_subset_keep_quarter_full_size():
    """bench --keep-ratio 0.25: layer l attends to kvc_attend_subset(keep 0.25, seed l) of its 172 pages."""
    import torch
    dc, oc, q = _chunk_caches("bf16", 72)
    log("chunked subset keep 0.25, 10,992 queries")
    ids, lens = oc.visible_table()
    assert len(ids) == 172
    for layer in (0, 17):
        si, sl = subset_table(ids, lens, 0.25, layer, 0, 0)
        assert len(si) == 43
        dids, dlens = dc.subset_table(0.25, layer)
        assert dids.tolist() == si and dlens.tolist() == sl
        o, lse = dc.attend_subset(to_dev(q, "bf16"), 0.25, layer)
        torch.cuda.synchronize()
        gk, gv = oc.gather(si, sl)
        rows = _chunk_rows(q.shape[0], layer)
        ro, rl = attention_f64(bits_f64(q[rows]), bits_f64(gk), bits_f64(gv))
        r = torch.from_numpy(rows).cuda()
        check_attention(o[r], lse[r], ro, rl, "bf16", f"layer seed {layer}: {len(si)} pages, Lk={gk.shape[1]}")


def test_chunked_fp8_pages_full_size():
    """bench --kv-dtype fp8 on the chunked step: E4M3 pages, 512-row FP8 tiles, sampled rows."""
    import torch
    dc, oc, q = _chunk_caches("fp8", 73)
    log("chunked FP8 pages, 10,992 queries x 43,968 keys")
    o, lse = dc.attend(to_dev(q, "bf16"))
    torch.cuda.synchronize()
    gk, gv = oc.gather()  # dequantised values
    assert gk.shape[1] == 43968
    rows = _chunk_rows(q.shape[0], 5)
    ro, rl = attention_f64(bits_f64(q[rows]), gk, gv)
    r = torch.from_numpy(rows).cuda()
    check_attention(o[r], lse[r], ro, rl, "bf16", f"fp8 chunk, {len(rows)} rows")
