"""Paged attention on the GPU against the fp64 oracle.

Covers the streaming step (current frame's 262 queries against scale, window
and special pages), keyframe rollback, chunk units with ragged tails, several
sequences in one call, empty and one-token key sets, partial pages with
NaN-poisoned stale slots, forced key splits, page-order invariance, peaky
scores and the split merge on its own.
"""
import math

import numpy as np
import pytest

import synth
from gpu_helpers import check_attention, log, to_dev, to_f64, v_pool_device_layout, v_positions
from oracle import OracleCache, OracleConfig, attention_f64, is_keyframe, merge_partials
from oracle import to_f64 as bits_f64

pytestmark = pytest.mark.gpu


def _dev_cache(dtype, H, P, X, S, W, frames, **kw):
    from paged_sliding_window_kv_amd import KvCache
    return KvCache(num_heads=H, head_dim=64, dtype=dtype, patch_tokens=P, special_tokens=X, num_scale_units=S,
                   window_units=W, max_units=frames, device="cuda", **kw)


def _oracle(dtype, H, P, X, S, W, frames):
    return OracleCache(OracleConfig(num_heads=H, head_dim=64, patch_tokens=P, special_tokens=X,
                                    num_scale_units=S, window_units=W, max_units=frames, store_dtype=dtype))


def _stream(dtype, H, P, X, S, W, frames, interval=1, check_every=1, seed=7, q_scale=1.0, num_splits=0,
            poison=True):
    import torch
    dc = _dev_cache(dtype, H, P, X, S, W, frames)
    oc = _oracle(dtype, H, P, X, S, W, frames)
    if poison:
        dc.k_pool.fill_(float("nan"))
        dc.v_pool.fill_(float("nan"))
    for t in range(frames):
        q, k, v = synth.frame_qkv(seed, 0, t, P + X, H, 64, dtype, q_scale)
        oc.append(k, v)
        dc.append(to_dev(k, dtype), to_dev(v, dtype))
        if t % check_every == 0 or t == frames - 1:
            o, lse = dc.attend(to_dev(q, dtype), num_splits=num_splits)
            gk, gv = oc.gather()
            ro, rl = attention_f64(bits_f64(q), bits_f64(gk), bits_f64(gv))
            check_attention(o, lse, ro, rl, dtype, f"t={t} Lk={gk.shape[1]}")
        if not is_keyframe(t, S, interval):
            oc.rollback()
            dc.rollback()
    torch.cuda.synchronize()


def test_tiny_streaming_f32():
    # 1 layer, 4 heads x 64, fp32; 256 patch + 6 special; S=2, W=4; 12 frames; every step checked
    log("tiny fp32 stream")
    _stream("f32", 4, 256, 6, 2, 4, 12)


def test_tiny_streaming_bf16():
    log("tiny bf16 stream")
    _stream("bf16", 4, 256, 6, 2, 4, 12)


def test_keyframe_stream_f32():
    log("keyframe fp32 stream (N=4)")
    _stream("f32", 4, 256, 6, 2, 4, 60, interval=4, check_every=5)


def test_lingbot_shaped_stream_bf16_reduced():
    # 16 heads, S=8, W=16 (window shortened so the oracle stays fast), 120 frames, sampled steps
    log("lingbot-shaped bf16 stream (W=16)")
    _stream("bf16", 16, 256, 6, 8, 16, 120, check_every=13)


def test_stream_forced_splits_and_peaky():
    log("forced splits 1/3/7, peaky Q")
    for ns in (1, 3, 7):
        _stream("bf16", 4, 256, 6, 2, 4, 9, check_every=4, num_splits=ns, q_scale=4.0)


def test_chunk_units_with_tails():
    # 2-frame chunks of 1374 tokens: 11 pages per unit, tail 188; window 2 chunks; query = the chunk
    log("chunk units bf16")
    _stream("bf16", 4, 2 * 1374, 0, 0, 2, 4)


def _random_tables(rng, page_counts, pool_pages, P):
    """Distinct pages across all sequences, lengths from a set of edge values."""
    total = sum(page_counts)
    pages = rng.choice(pool_pages, size=total, replace=False)
    lens = rng.choice([1, 5, 63, 64, 65, 127, 200, P - 1, P, P], size=total)
    kv = np.concatenate([[0], np.cumsum(page_counts)])
    return pages.astype(np.int32), lens.astype(np.int32), kv.astype(np.int32)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_multi_sequence_ragged(dtype):
    import torch
    from paged_sliding_window_kv_amd import paged_attention
    log(f"multi-sequence ragged {dtype}")
    rng = np.random.default_rng(21)
    H, P, N = 3, 256, 64
    qlens = [1, 31, 33, 262, 0, 300, 64, 129]
    counts = [3, 6, 0, 5, 2, 6, 1, 4]          # sequence 2 has no keys at all
    ns = len(qlens)
    ids, lens, kv = _random_tables(rng, counts, N, P)
    qo = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    kpool = synth.normal_tokens(3, 0, 0, 1, N * H * P, 1, 64, dtype).reshape(N, H, P, 64)
    vpool = synth.normal_tokens(3, 0, 0, 2, N * H * P, 1, 64, dtype).reshape(N, H, P, 64)
    q = synth.normal_tokens(3, 0, 0, 0, int(qo[-1]), H, 64, dtype)
    kd = to_dev(kpool, dtype)
    vd = to_dev(v_pool_device_layout(vpool), dtype)
    # stale slots past each page's length become NaN on the device
    pos = torch.from_numpy(v_positions(P)).cuda()
    for p, n in zip(ids, lens):
        kd[p, :, n:] = float("nan")
        vd[p][:, :, pos[n:]] = float("nan")
    dev = lambda a: torch.from_numpy(a).cuda()
    for splits in (0, 1, 4):
        o, lse = paged_attention(to_dev(q, dtype), kd, vd, dev(ids), dev(lens), dev(qo), dev(kv),
                                 max_qo_len=max(qlens), max_kv_pages=int(np.diff(kv).max()), num_splits=splits)
        for s in range(ns):
            a, b = qo[s], qo[s + 1]
            sel = list(zip(ids[kv[s]:kv[s + 1]], lens[kv[s]:kv[s + 1]]))
            if sel:
                gk = np.concatenate([kpool[p, :, :n] for p, n in sel], axis=1)
                gv = np.concatenate([vpool[p, :, :n] for p, n in sel], axis=1)
            else:
                gk = gv = np.zeros((H, 0, 64), kpool.dtype)
            ro, rl = attention_f64(bits_f64(q[a:b]), bits_f64(gk), bits_f64(gv))
            check_attention(o[a:b], lse[a:b], ro, rl, dtype, f"splits={splits} seq={s} q={b - a} Lk={gk.shape[1]}")
            if not sel:
                assert (to_f64(o[a:b]) == 0).all()


@pytest.mark.parametrize("qn", [1, 32, 33, 100, 224, 256, 257, 262, 271, 272, 273, 288, 289, 545, 1025, 1100, 1536, 1600])
def test_query_counts_across_tile_shapes(qn):
    """One sequence whose query count walks through every workgroup shape: 1..8
    32-row blocks, the 272-row tile with its 16-row extra block, 256-row tiles
    (the pipelined kernel) and 512-row tiles (two blocks per wave, above 1024
    queries), with partial last tiles; keys from ragged pages, with and
    without key splits."""
    import torch
    from paged_sliding_window_kv_amd import paged_attention
    log(f"query count {qn}")
    rng = np.random.default_rng(1000 + qn)
    H, P, N = 2, 256, 16
    ids, lens, kv = _random_tables(rng, [7], N, P)
    qo = np.array([0, qn], np.int32)
    kpool = synth.normal_tokens(4, 0, qn, 1, N * H * P, 1, 64, "bf16").reshape(N, H, P, 64)
    vpool = synth.normal_tokens(4, 0, qn, 2, N * H * P, 1, 64, "bf16").reshape(N, H, P, 64)
    q = synth.normal_tokens(4, 0, qn, 0, qn, H, 64, "bf16")
    kd = to_dev(kpool, "bf16")
    vd = to_dev(v_pool_device_layout(vpool), "bf16")
    pos = torch.from_numpy(v_positions(P)).cuda()
    for p_, n in zip(ids, lens):
        kd[p_, :, n:] = float("nan")
        vd[p_][:, :, pos[n:]] = float("nan")
    dev = lambda a: torch.from_numpy(a).cuda()
    gk = np.concatenate([kpool[p_, :, :n] for p_, n in zip(ids, lens)], axis=1)
    gv = np.concatenate([vpool[p_, :, :n] for p_, n in zip(ids, lens)], axis=1)
    ro, rl = attention_f64(bits_f64(q), bits_f64(gk), bits_f64(gv))
    for splits in (1, 3):
        o, lse = paged_attention(to_dev(q, "bf16"), kd, vd, dev(ids), dev(lens), dev(qo), dev(kv),
                                 max_qo_len=qn, max_kv_pages=7, num_splits=splits)
        check_attention(o, lse, ro, rl, "bf16", f"q={qn} splits={splits} Lk={gk.shape[1]}")


@pytest.mark.parametrize("splits", [0, 1, 5])
@pytest.mark.parametrize("wide", [False, True])
def test_large_tiles_short_and_empty_key_ranges(splits, wide):
    """256-row query tiles (the 8-wave software-pipelined kernel) and 512-row
    tiles (two 32-row blocks per wave, above 1024 queries) against key ranges
    that leave the key loop nearly or entirely empty: no keys at all (O = 0,
    lse = -inf), one token, one page shorter than a 64-key tile, one exactly
    full tile, and a 5-page range whose forced splits leave whole splits with
    a single tile; NaN-poisoned stale slots."""
    import torch
    from paged_sliding_window_kv_amd import paged_attention
    log(f"large tiles (wide={wide}), short key ranges, splits={splits}")
    rng = np.random.default_rng(55)
    H, P, N = 2, 256, 16
    qlens = [1100, 1025, 1600, 530, 1100] if wide else [300, 257, 512, 300, 270]
    page_lens = [[], [1], [37], [64], [256, 64, 200, 1, 65]]
    counts = [len(x) for x in page_lens]
    ids = rng.choice(N, size=sum(counts), replace=False).astype(np.int32)
    lens = np.array([n for x in page_lens for n in x], np.int32)
    kv = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    qo = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    kpool = synth.normal_tokens(6, 0, 0, 1, N * H * P, 1, 64, "bf16").reshape(N, H, P, 64)
    vpool = synth.normal_tokens(6, 0, 0, 2, N * H * P, 1, 64, "bf16").reshape(N, H, P, 64)
    q = synth.normal_tokens(6, 0, 0, 0, int(qo[-1]), H, 64, "bf16")
    kd = to_dev(kpool, "bf16")
    vd = to_dev(v_pool_device_layout(vpool), "bf16")
    pos = torch.from_numpy(v_positions(P)).cuda()
    for p_, n in zip(ids, lens):
        kd[p_, :, n:] = float("nan")
        vd[p_][:, :, pos[n:]] = float("nan")
    dev = lambda a: torch.from_numpy(a).cuda()
    o, lse = paged_attention(to_dev(q, "bf16"), kd, vd, dev(ids), dev(lens), dev(qo), dev(kv),
                             max_qo_len=max(qlens), max_kv_pages=max(counts), num_splits=splits)
    for s_ in range(len(qlens)):
        a, b = qo[s_], qo[s_ + 1]
        sel = list(zip(ids[kv[s_]:kv[s_ + 1]], lens[kv[s_]:kv[s_ + 1]]))
        if sel:
            gk = np.concatenate([kpool[p_, :, :n] for p_, n in sel], axis=1)
            gv = np.concatenate([vpool[p_, :, :n] for p_, n in sel], axis=1)
        else:
            gk = gv = np.zeros((H, 0, 64), kpool.dtype)
        ro, rl = attention_f64(bits_f64(q[a:b]), bits_f64(gk), bits_f64(gv))
        check_attention(o[a:b], lse[a:b], ro, rl, "bf16", f"splits={splits} seq={s_} q={b - a} Lk={gk.shape[1]}")
        if not sel:
            assert (to_f64(o[a:b]) == 0).all()


@pytest.mark.parametrize("qn", [262, 256, 1100])
def test_late_keys_outgrow_running_maximum(qn):
    """Scores of later pages exceed every earlier one by far more than 16 log2
    units, so the kernel's rescale path (tile maximum taken again, O and row sum
    rescaled) runs, on the 32-row blocks and on the 16-row extra block (262
    queries); partial first pages exercise the first-tile maximum with masked
    keys."""
    import torch
    from paged_sliding_window_kv_amd import paged_attention
    log(f"late large scores q={qn}")
    rng = np.random.default_rng(77)
    H, P, N = 2, 256, 16
    ids = rng.choice(N, size=6, replace=False).astype(np.int32)
    lens = np.array([37, 256, 130, 256, 256, 200], np.int32)
    kv = np.array([0, 6], np.int32)
    qo = np.array([0, qn], np.int32)
    kpool = synth.normal_tokens(9, 0, qn, 1, N * H * P, 1, 64, "f32").reshape(N, H, P, 64)
    vpool = synth.normal_tokens(9, 0, qn, 2, N * H * P, 1, 64, "bf16").reshape(N, H, P, 64)
    q = synth.normal_tokens(9, 0, qn, 0, qn, H, 64, "f32")
    # every query shares a component along a unit direction u (per head), and the
    # keys of the last three pages are long along u: their scores exceed the
    # first pages' by tens of natural-log units
    u = rng.standard_normal((H, 64))
    u /= np.linalg.norm(u, axis=-1, keepdims=True)
    q = (q + 4.0 * u[None]).astype(np.float32)
    for j, p_ in enumerate(ids[3:]):
        kpool[p_] += ((30.0 + 6 * j) * u[:, None, :]).astype(np.float32)
    kb = synth.f32_to_bf16_bits(kpool)
    qb = synth.f32_to_bf16_bits(q)
    kd = to_dev(kb, "bf16")
    vd = to_dev(v_pool_device_layout(vpool), "bf16")
    dev = lambda a: torch.from_numpy(a).cuda()
    gk = np.concatenate([kb[p_, :, :n] for p_, n in zip(ids, lens)], axis=1)
    gv = np.concatenate([vpool[p_, :, :n] for p_, n in zip(ids, lens)], axis=1)
    ro, rl = attention_f64(bits_f64(qb), bits_f64(gk), bits_f64(gv))
    # the late keys dominate: for most rows the maximum exceeds the first page's by
    # more than 12 (natural log), i.e. more than 16 log2 units
    s = np.einsum("qhd,hkd->hqk", bits_f64(qb), bits_f64(gk)) / 8.0
    gap = s.max(axis=-1) - s[:, :, :37].max(axis=-1)
    assert (gap > 12.0).mean() > 0.75
    for splits in (1, 2):
        o, lse = paged_attention(to_dev(qb, "bf16"), kd, vd, dev(ids), dev(lens), dev(qo), dev(kv),
                                 max_qo_len=qn, max_kv_pages=6, num_splits=splits)
        check_attention(o, lse, ro, rl, "bf16", f"q={qn} splits={splits}")


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_split_partials_with_values_beyond_fp16_range(dtype):
    """V scaled by 2^20 (exact in bf16): the split partials, kept in fp16 with a
    per-row power-of-two scale, must not overflow; O / 2^20 matches the oracle's.
    262 queries (32-row blocks and the 16-row extra block), forced key splits."""
    import torch
    from paged_sliding_window_kv_amd import KvCache
    log(f"values beyond fp16 range, {dtype}")
    H, P, X, S, W, frames = 2, 256, 6, 1, 2, 5
    dc = KvCache(num_heads=H, dtype=dtype, patch_tokens=P, special_tokens=X, num_scale_units=S, window_units=W,
                 max_units=frames, device="cuda")
    oc = _oracle(dtype, H, P, X, S, W, frames)
    big = 2.0 ** 20
    for t in range(frames):
        q, k, v = synth.frame_qkv(31, 0, t, P + X, H, 64, "bf16")
        vb = synth.f32_to_bf16_bits((synth.bf16_bits_to_f32(v) * np.float32(big)).astype(np.float32))
        oc.append(k, vb)
        dc.append(to_dev(k, "bf16"), to_dev(vb, "bf16"))
    for splits in (2, 3):
        o, lse = dc.attend(to_dev(q, "bf16"), num_splits=splits)
        gk, gv = oc.gather()
        ro, rl = attention_f64(bits_f64(q), bits_f64(gk), bits_f64(gv))
        assert np.abs(ro).max() > 32768.0 * 4
        got = to_f64(o)
        assert np.isfinite(got).all()
        check_attention(torch.from_numpy(got / big), lse, ro / big, rl, "bf16", f"{dtype} splits={splits}")


def test_page_order_and_placement_invariance():
    import torch
    from paged_sliding_window_kv_amd import paged_attention
    log("page placement invariance")
    rng = np.random.default_rng(5)
    H, P, N, npg = 2, 256, 24, 9
    kpool = synth.normal_tokens(8, 0, 0, 1, N * H * P, 1, 64, "bf16").reshape(N, H, P, 64)
    vpool = synth.normal_tokens(8, 0, 0, 2, N * H * P, 1, 64, "bf16").reshape(N, H, P, 64)
    q = synth.normal_tokens(8, 0, 0, 0, 200, H, 64, "bf16")
    ids = rng.choice(N, npg, replace=False).astype(np.int32)
    lens = np.array([256, 256, 100, 256, 7, 256, 256, 256, 252], np.int32)
    # the same tokens placed in other pages, in another order
    perm = rng.permutation(npg)
    new_ids = rng.choice(N, npg, replace=False).astype(np.int32)
    kpool2 = np.zeros_like(kpool)
    vpool2 = np.zeros_like(vpool)
    for j, i in enumerate(perm):
        kpool2[new_ids[j]] = kpool[ids[i]]
        vpool2[new_ids[j]] = vpool[ids[i]]
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    qo, kv = np.array([0, 200], np.int32), np.array([0, npg], np.int32)
    gk = np.concatenate([kpool[p, :, :n] for p, n in zip(ids, lens)], axis=1)
    gv = np.concatenate([vpool[p, :, :n] for p, n in zip(ids, lens)], axis=1)
    ro, rl = attention_f64(bits_f64(q), bits_f64(gk), bits_f64(gv))
    for kp, vp, ii, ll in ((kpool, vpool, ids, lens), (kpool2, vpool2, new_ids, lens[perm])):
        o, lse = paged_attention(to_dev(q, "bf16"), to_dev(kp, "bf16"), to_dev(v_pool_device_layout(vp), "bf16"),
                                 dev(ii), dev(ll), dev(qo), dev(kv), max_qo_len=200, max_kv_pages=npg)
        check_attention(o, lse, ro, rl, "bf16", "placement")


def test_merge_kernel_against_oracle_merge():
    import torch
    from paged_sliding_window_kv_amd import merge_partials as dev_merge
    log("merge kernel")
    rng = np.random.default_rng(9)
    parts, rows, H = 5, 37, 3
    po = rng.standard_normal((parts, rows, H, 64)).astype(np.float32)
    pl = (rng.standard_normal((parts, rows, H)) * 3).astype(np.float32)
    pl[1, :5] = -np.inf          # empty parts
    pl[:, 7] = -np.inf           # a row where every part is empty
    ref_o, ref_l = merge_partials([(po[i].astype(np.float64), pl[i].astype(np.float64)) for i in range(parts)])
    for dtype in ("f32", "bf16"):
        import torch
        out = torch.empty((rows, H, 64), dtype=torch.float32 if dtype == "f32" else torch.bfloat16, device="cuda")
        lse = torch.empty((rows, H), dtype=torch.float32, device="cuda")
        dev_merge(torch.from_numpy(po).cuda(), torch.from_numpy(pl).cuda(), out, lse)
        o = to_f64(out)
        tol = 1e-5 if dtype == "f32" else 1e-2
        assert np.abs(o - ref_o).max() <= tol * max(1.0, np.abs(ref_o).max())
        l = to_f64(lse)
        fin = np.isfinite(ref_l)
        assert np.abs(l[fin] - ref_l[fin]).max() <= 1e-5 and np.isneginf(l[~fin]).all()
        assert (o[7] == 0).all()
