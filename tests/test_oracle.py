"""Pins of the oracle against what the pages and mathematics fix (CPU only).

Each check is written as a function returning a bool so that the planted-
mistake tests at the end can show that a plausible error in the oracle makes
one of them fail.
"""
import json
import math
import os

import numpy as np
import pytest

import synth
from oracle import (CONTIGUOUS, FRAME_ALIGNED, NoUndo, OracleCache, OracleConfig, OutOfPages,
                    attention_f64, brute_attention, dense_history_attention, is_keyframe,
                    merge_partials, required_pages, to_f64)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _tiny_cfg(**kw):
    base = dict(num_heads=2, head_dim=8, page_size=4, patch_tokens=6, special_tokens=3,
                num_scale_units=1, window_units=2, max_units=10, store_dtype="f32")
    base.update(kw)
    return OracleConfig(**base)


def _unit(cfg, seed, t, kind):
    tok = cfg.patch_tokens + cfg.special_tokens
    return synth.normal_tokens(seed, 0, t, kind, tok, cfg.num_heads, cfg.head_dim, cfg.store_dtype)


# ---------------------------------------------------------------------------
# attention value pins
# ---------------------------------------------------------------------------
def check_brute_force(att=attention_f64) -> bool:
    """Paged oracle attention == scalar triple loop on a tiny multi-page stream."""
    cfg = _tiny_cfg()
    c = OracleCache(cfg)
    ok = True
    for t in range(10):
        c.append(_unit(cfg, 1, t, 1), _unit(cfg, 1, t, 2))
        q = _unit(cfg, 1, t, 0)
        k, v = c.gather()
        o, lse = att(to_f64(q), to_f64(k), to_f64(v), 0.35)
        ob, lb = brute_attention(to_f64(q).tolist(), to_f64(k).tolist(), to_f64(v).tolist(), 0.35)
        ok &= np.allclose(o, np.array(ob), rtol=0, atol=1e-12)
        ok &= np.allclose(lse, np.array(lb), rtol=0, atol=1e-12)
    return bool(ok)


def test_brute_force():
    assert check_brute_force()


def check_library_attention(att=attention_f64) -> bool:
    """Oracle attention == PyTorch's scaled_dot_product_attention (CPU, float64) for O, and
    == torch.logsumexp of the scaled scores for lse: library routines that share no code with the
    oracle.  Shapes span one query to several 1,024-row query blocks of the oracle, uneven key
    counts, and a row of planted large scores (peaky softmax)."""
    import torch
    rng = np.random.default_rng(11)
    ok = True
    for lq, lk, h, d, scale in ((1, 7, 2, 8, None), (37, 300, 3, 16, 0.21), (2100, 517, 2, 64, None)):
        q = rng.standard_normal((lq, h, d))
        k = rng.standard_normal((h, lk, d))
        v = rng.standard_normal((h, lk, d))
        q[0] *= 6.0  # peaky first row
        o, lse = att(q, k, v, scale)
        s = (1.0 / math.sqrt(d)) if scale is None else scale
        tq = torch.from_numpy(q).permute(1, 0, 2)        # [H, Lq, d]
        tk, tv = torch.from_numpy(k), torch.from_numpy(v)  # [H, Lk, d]
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=s).permute(1, 0, 2).numpy()
        ref_lse = torch.logsumexp(s * (tq @ tk.transpose(1, 2)), dim=-1).transpose(0, 1).numpy()
        ok &= np.allclose(o, ref, rtol=0, atol=1e-12)
        ok &= np.allclose(lse, ref_lse, rtol=0, atol=1e-12)
    return bool(ok)


def test_library_attention():
    assert check_library_attention()


def test_closed_forms():
    rng = np.random.default_rng(5)
    h, d, lk = 3, 16, 37
    v = rng.standard_normal((h, lk, d))
    # all keys equal -> output is the mean of V, lse = s<q,k> + log Lk
    k = np.broadcast_to(rng.standard_normal((h, 1, d)), (h, lk, d)).copy()
    q = rng.standard_normal((5, h, d))
    o, lse = attention_f64(q, k, v, 0.125)
    assert np.allclose(o, np.broadcast_to(v.mean(axis=1)[None], o.shape), atol=1e-13)
    ref = 0.125 * np.einsum("qhd,hd->qh", q, k[:, 0, :]) + math.log(lk)
    assert np.allclose(lse, ref, atol=1e-12)
    # Q = 0 -> mean of V as well
    o0, _ = attention_f64(np.zeros((2, h, d)), rng.standard_normal((h, lk, d)), v)
    assert np.allclose(o0, np.broadcast_to(v.mean(axis=1)[None], o0.shape), atol=1e-13)
    # one visible token -> O = V
    o1, l1 = attention_f64(q, k[:, :1], v[:, :1])
    assert np.allclose(o1, np.broadcast_to(v[:, 0][None], o1.shape), atol=1e-15)
    # planted key with a score margin of 60 -> O equals its V to fp64 precision
    kk = rng.standard_normal((h, lk, d)) * 0.01
    qq = np.zeros((1, h, d))
    qq[0, :, 0] = 1.0
    kk[:, 11, 0] = 60.0 / 0.125
    op, _ = attention_f64(qq, kk, v, 0.125)
    assert np.allclose(op[0], v[:, 11], rtol=0, atol=1e-20)
    # empty key set
    oe, le = attention_f64(q, k[:, :0], v[:, :0])
    assert (oe == 0).all() and np.isneginf(le).all()


def test_key_order_invariance_and_default_scale():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((7, 2, 64))
    k = rng.standard_normal((2, 50, 64))
    v = rng.standard_normal((2, 50, 64))
    perm = rng.permutation(50)
    o, lse = attention_f64(q, k, v)
    o2, lse2 = attention_f64(q, k[:, perm], v[:, perm])
    assert np.allclose(o, o2, atol=1e-13) and np.allclose(lse, lse2, atol=1e-12)
    o3, _ = attention_f64(q, k, v, 1.0 / 8.0)     # head_dim 64 -> 1/sqrt(64)
    assert np.array_equal(o, o3)


def test_blocking_does_not_change_result():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((300, 2, 16))
    k = rng.standard_normal((2, 90, 16))
    v = rng.standard_normal((2, 90, 16))
    a, la = attention_f64(q, k, v, block=1024)
    b, lb = attention_f64(q, k, v, block=7)
    assert np.allclose(a, b, atol=1e-14) and np.allclose(la, lb, atol=1e-13)


def check_merge(merge=merge_partials) -> bool:
    rng = np.random.default_rng(8)
    q = rng.standard_normal((9, 2, 16))
    k = rng.standard_normal((2, 120, 16))
    v = rng.standard_normal((2, 120, 16))
    o, lse = attention_f64(q, k, v)
    cuts = [0, 13, 13, 70, 120]            # includes an empty part
    parts = [attention_f64(q, k[:, a:b], v[:, a:b]) for a, b in zip(cuts[:-1], cuts[1:])]
    om, lm = merge(parts)
    return bool(np.allclose(o, om, atol=1e-13) and np.allclose(lse, lm, atol=1e-12))


def test_merge_partials():
    assert check_merge()
    o, l = merge_partials([(np.ones((2, 3)), np.full(2, -np.inf))])
    assert np.isneginf(l).all() and (o == 0).all()


# ---------------------------------------------------------------------------
# paged gather == tokens selected straight from the history
# ---------------------------------------------------------------------------
def _run_history_check(cfg, frames, keyframe_interval=1, seed=3) -> bool:
    cfg.max_units = max(cfg.max_units, frames)
    c = OracleCache(cfg)
    hk, hv = [], []
    ok = True
    for t in range(frames):
        k, v = _unit(cfg, seed, t, 1), _unit(cfg, seed, t, 2)
        q = _unit(cfg, seed, t, 0)
        c.append(k, v)
        hk.append(k)
        hv.append(v)
        # gathered bytes equal the history selection, byte for byte
        gk, gv = c.gather()
        n = len(hk)
        sel = list(range(min(n, cfg.num_scale_units)))
        rest = list(range(min(n, cfg.num_scale_units), n))
        sel += rest if cfg.window_units <= 0 else rest[-cfg.window_units:]
        ek = np.concatenate([hk[i][:cfg.patch_tokens] for i in sel] + [hk[i][cfg.patch_tokens:] for i in range(n)])
        ok &= np.array_equal(gk, ek.transpose(1, 0, 2))
        o, lse = attention_f64(to_f64(q), to_f64(gk), to_f64(gv))
        od, ld = dense_history_attention(q, hk, hv, cfg.patch_tokens, cfg.num_scale_units, cfg.window_units)
        ok &= np.allclose(o, od, atol=1e-12) and np.allclose(lse, ld, atol=1e-12)
        if not is_keyframe(t, cfg.num_scale_units, keyframe_interval):
            c.rollback()
            hk.pop()
            hv.pop()
    return bool(ok)


def test_paged_equals_history_selection():
    assert _run_history_check(_tiny_cfg(), 10)
    assert _run_history_check(_tiny_cfg(window_units=1, num_scale_units=0), 8)
    assert _run_history_check(_tiny_cfg(window_units=0), 9)
    assert _run_history_check(_tiny_cfg(special_packing=CONTIGUOUS, special_tokens=3), 12)
    assert _run_history_check(_tiny_cfg(), 14, keyframe_interval=3)


def test_window_one_is_independent_chunks():
    # sliding_window_num = 1: each chunk attends to itself only (RFC #2727, section 2.3 table).
    cfg = _tiny_cfg(special_tokens=0, num_scale_units=0, window_units=1, patch_tokens=7)
    c = OracleCache(cfg)
    for t in range(4):
        k, v, q = _unit(cfg, 9, t, 1), _unit(cfg, 9, t, 2), _unit(cfg, 9, t, 0)
        c.append(k, v)
        gk, gv = c.gather()
        o, _ = attention_f64(to_f64(q), to_f64(gk), to_f64(gv))
        oself, _ = attention_f64(to_f64(q), to_f64(k).transpose(1, 0, 2), to_f64(v).transpose(1, 0, 2))
        assert np.allclose(o, oself, atol=1e-14)


def test_unbounded_window_is_full_attention():
    # sliding_window_num = infinity: full global attention over every appended token (RFC section 2.3).
    cfg = _tiny_cfg(special_tokens=0, num_scale_units=0, window_units=0, patch_tokens=5)
    c = OracleCache(cfg)
    ks, vs = [], []
    for t in range(6):
        k, v = _unit(cfg, 10, t, 1), _unit(cfg, 10, t, 2)
        c.append(k, v)
        ks.append(k)
        vs.append(v)
    allk = to_f64(np.concatenate(ks)).transpose(1, 0, 2)
    allv = to_f64(np.concatenate(vs)).transpose(1, 0, 2)
    q = to_f64(np.concatenate(ks))           # every token as a query: global self-attention
    gk, gv = c.gather()
    a, _ = attention_f64(q, to_f64(gk), to_f64(gv))
    b, _ = attention_f64(q, allk, allv)
    assert np.allclose(a, b, atol=1e-14)


# ---------------------------------------------------------------------------
# page-table pins
# ---------------------------------------------------------------------------
def check_config1_trace(cache_cls=OracleCache) -> bool:
    g = _golden("config1_trace.json")
    gc = g["config"]
    cfg = OracleConfig(num_heads=1, head_dim=1, page_size=gc["page_size"], patch_tokens=gc["patch_tokens"],
                       special_tokens=gc["special_tokens"], num_scale_units=gc["num_scale_units"],
                       window_units=gc["window_units"], num_pages=gc["num_pages"], max_units=12)
    c = cache_cls(cfg, with_pool=False)
    ok = True
    for st in g["steps"]:
        c.append()
        ids, lens = c.visible_table()
        ok &= ids == st["page_ids"]
        ok &= lens[-1] == st["last_page_len"] and sum(lens) == st["lk"]
        ok &= all(x == 256 for x in lens[:-1])
        ok &= c.free == st["free_bottom_to_top"]
    return bool(ok)


def test_config1_trace():
    assert check_config1_trace()


def test_page_constants_from_the_pages():
    g = _golden("page_constants.json")
    page = g["page_size_tokens"]["value"]
    x = g["special_tokens_per_frame"]["value"]
    cfg = OracleConfig(num_heads=1, head_dim=1, page_size=page, patch_tokens=g["patch_tokens_per_frame"]["value"],
                       special_tokens=x, num_scale_units=g["scale_pages"]["value"],
                       window_units=g["window_pages"]["value"], max_units=1000)
    assert cfg.frames_per_special_page == g["frames_per_special_page"]["value"]
    assert cfg.unit_pages == 1                       # 256 patch tokens fill exactly one page
    # chunk form: sequence_length = sliding_window_num x chunk_size frames
    cs, w = g["rfc_chunk_size"]["value"], g["rfc_sliding_window_num"]["value"]
    ccfg = OracleConfig(num_heads=1, head_dim=1, page_size=page,
                        patch_tokens=cs * g["vggt_tokens_per_image"]["value"], special_tokens=0,
                        num_scale_units=0, window_units=w, max_units=20)
    c = OracleCache(ccfg, with_pool=False)
    for _ in range(12):
        c.append()
    _, lens = c.visible_table()
    assert sum(lens) == g["rfc_sequence_length_frames"]["value"] * g["vggt_tokens_per_image"]["value"]
    # 100 frames x 1374 tokens: one bf16 score matrix is about 35 GB (35.16 GiB)
    n = 100 * g["vggt_tokens_per_image"]["value"]
    assert round(n * n * 2 / 2 ** 30) == g["attention_matrix_gb_at_100_frames"]["value"]


def _stream_invariants(cfg, frames, interval=1, check_every=1):
    c = OracleCache(cfg, with_pool=False)
    u = cfg.unit_pages
    f = cfg.frames_per_special_page
    for t in range(frames):
        before = c.state()
        c.append()
        # conservation, no duplicates
        st = c.state()
        used = st["scale_pages"] + st["window_pages"] + st["special_pages"]
        assert len(set(used)) == len(used) and not set(used) & set(st["free"])
        assert len(used) + len(st["free"]) == c.num_pages
        if t % check_every == 0:
            ids, lens = c.visible_table()
            n = c.n
            if cfg.window_units > 0 and n > cfg.num_scale_units + cfg.window_units:
                assert c.patch_page_count() == (cfg.num_scale_units + cfg.window_units) * u
            if cfg.special_tokens and cfg.special_packing == FRAME_ALIGNED:
                ns = -(-n // f)
                assert len(c.special_pages) == ns
                assert lens[-1] == cfg.special_tokens * (n - f * (ns - 1))
                assert all(x == cfg.special_tokens * f for x in lens[len(lens) - ns:-1])
        if not is_keyframe(t, cfg.num_scale_units, interval):
            c.rollback()
            assert c.state() == {**before, "has_undo": False}
    return c


def test_lingbot_stream_invariants():
    cfg = OracleConfig(num_heads=1, head_dim=1, num_scale_units=8, window_units=64, max_units=1000)
    c = _stream_invariants(cfg, 1000)
    ids, lens = c.visible_table()
    assert len(ids) == 72 + 24 and sum(lens) == 72 * 256 + 6 * 1000


def test_keyframe_stream_10000():
    cfg = OracleConfig(num_heads=1, head_dim=1, num_scale_units=2, window_units=4, max_units=10000)
    c = _stream_invariants(cfg, 10000, interval=4, check_every=7)
    # growth ~ 1/N: n = S + ceil((T - S) / N)
    assert c.n == 2 + -(-(10000 - 2) // 4) == 2502
    assert len(c.special_pages) == 60 and c.last_page_len() == 144
    assert c.patch_page_count() == 6


def test_contiguous_special_packing():
    cfg = OracleConfig(num_heads=1, head_dim=1, num_scale_units=2, window_units=4, max_units=10000,
                       special_packing=CONTIGUOUS)
    c = _stream_invariants(cfg, 10000, interval=4, check_every=97)
    assert len(c.special_pages) == -(-2502 * 6 // 256) == 59
    ids, lens = c.visible_table()
    assert all(x == 256 for x in lens[-59:-1]) and lens[-1] == 2502 * 6 - 58 * 256


def test_chunk_config_table():
    cfg = OracleConfig(num_heads=1, head_dim=1, patch_tokens=8 * 1374, special_tokens=0,
                       num_scale_units=0, window_units=4, max_units=12)
    c = OracleCache(cfg, with_pool=False)
    for _ in range(12):
        c.append()
    ids, lens = c.visible_table()
    assert len(ids) == 172 and sum(lens) == 43968
    assert [lens[i] for i in (42, 85, 128, 171)] == [240] * 4
    assert c.num_pages == 5 * 43


def test_rollback_restores_bytes_exactly():
    cfg = OracleConfig(num_heads=2, head_dim=8, page_size=8, patch_tokens=8, special_tokens=3,
                       num_scale_units=1, window_units=2, max_units=60, store_dtype="bf16")
    c = OracleCache(cfg)
    for t in range(60):
        tok = 11
        k = synth.normal_tokens(2, 0, t, 1, tok, 2, 8)
        v = synth.normal_tokens(2, 0, t, 2, tok, 2, 8)
        st = c.state()
        gk0, gv0 = c.gather()
        c.append(k, v)
        if not is_keyframe(t, 1, 3):
            c.rollback()
            gk1, gv1 = c.gather()
            assert c.state() == {**st, "has_undo": False}
            assert np.array_equal(gk0, gk1) and np.array_equal(gv0, gv1)


def test_errors_leave_state_unchanged():
    cfg = OracleConfig(num_heads=1, head_dim=1, num_scale_units=1, window_units=2, num_pages=3, max_units=50)
    c = OracleCache(cfg, with_pool=False)
    c.append()
    c.append()
    st = c.state()
    with pytest.raises(OutOfPages):
        c.append()
    assert c.state() == st
    c.rollback()
    with pytest.raises(NoUndo):
        c.rollback()
    assert required_pages(OracleConfig(num_heads=1, head_dim=1, num_scale_units=2, window_units=4,
                                       max_units=12)) == 8


def test_keyframe_rule():
    assert [is_keyframe(t, 2, 4) for t in range(9)] == [True, True, True, False, False, False, True, False, False]


# ---------------------------------------------------------------------------
# planted mistakes: each must make a pin above fail
# ---------------------------------------------------------------------------
def test_planted_mistakes_are_caught(monkeypatch):
    # 1. V and K swapped inside the attention
    def swapped(q, k, v, sm_scale=None, block=1024):
        return attention_f64(q, v, k, sm_scale, block)
    assert not check_brute_force(swapped)
    assert not check_library_attention(swapped)
    # 2. scale applied twice (dropped/duplicated factor)
    def twice(q, k, v, sm_scale=None, block=1024):
        return attention_f64(q, k, v, (sm_scale or 1.0) ** 2, block)
    assert not check_brute_force(twice)
    # 2b. default scale 1/d instead of 1/sqrt(d)
    def wrong_default(q, k, v, sm_scale=None, block=1024):
        return attention_f64(q, k, v, sm_scale if sm_scale is not None else 1.0 / q.shape[2], block)
    assert not check_library_attention(wrong_default)
    # 2c. lse missing the running maximum (log of the shifted sum only)
    def lse_no_max(q, k, v, sm_scale=None, block=1024):
        o, lse = attention_f64(q, k, v, sm_scale, block)
        s = (1.0 / math.sqrt(q.shape[2])) if sm_scale is None else sm_scale
        m = np.stack([(s * np.einsum('qd,kd->qk', q[:, h], k[h])).max(axis=1) for h in range(k.shape[0])], axis=1)
        return o, lse - m
    assert not check_library_attention(lse_no_max)
    # 3. merge that forgets to renormalise
    def bad_merge(parts):
        parts = list(parts)
        o = sum(np.asarray(p[0]) for p in parts)
        return o, merge_partials(parts)[1]
    assert not check_merge(bad_merge)

    # 4. eviction done before the new unit's pages are popped
    class EvictFirst(OracleCache):
        def append(self, k_unit=None, v_unit=None):
            cfg = self.cfg
            if self.n >= cfg.num_scale_units and 0 < cfg.window_units <= len(self.window):
                for p in reversed(self.window.popleft()):
                    self.free.append(p)
            super().append(k_unit, v_unit)
    assert not check_config1_trace(EvictFirst)

    # 5. special page opened before the patch page
    class SpecialFirst(OracleCache):
        def append(self, k_unit=None, v_unit=None):
            new, _ = self._special_slots()
            if new:
                self.free[-1], self.free[-2] = self.free[-2], self.free[-1]
            super().append(k_unit, v_unit)
    assert not check_config1_trace(SpecialFirst)
