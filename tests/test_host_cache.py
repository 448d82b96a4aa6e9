"""The C++ page manager behind the C ABI against the oracle, bit-exact (CPU only).

Host-only handles (no device pools) run exactly the planning code that the
device path uses, so these tests need no GPU.
"""
import ctypes as C
import os
import re

import numpy as np
import pytest

from oracle import CONTIGUOUS, FRAME_ALIGNED, OracleCache, OracleConfig, OutOfPages as OOut, NoUndo as ONo
from oracle import is_keyframe
from paged_sliding_window_kv_amd import KvCache, NoUndo, OutOfPages
from paged_sliding_window_kv_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_library_exports_every_declared_symbol():
    """Every function declared in include/*.h is exported by libkvc.so and bound in _lib."""
    hdr = ""
    for name in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if name.endswith(".h"):
            with open(os.path.join(ROOT, "include", name)) as f:
                hdr += f.read()
    declared = set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(\w+)\s*\(", hdr, re.M))
    assert len(declared) >= 30
    assert declared == set(L.EXPORTED), declared ^ set(L.EXPORTED)
    lib = L.lib()
    for name in declared:
        assert hasattr(lib, name), name
    assert lib.kvc_version() >= 300


def _pair(**kw):
    packing = kw.pop("special_packing", FRAME_ALIGNED)
    ocfg = OracleConfig(num_heads=1, head_dim=1, special_packing=packing, **kw)
    oc = OracleCache(ocfg, with_pool=False)
    hc = KvCache(num_heads=1, head_dim=1, page_size=ocfg.page_size, patch_tokens=ocfg.patch_tokens,
                 special_tokens=ocfg.special_tokens, num_scale_units=ocfg.num_scale_units,
                 window_units=ocfg.window_units,
                 special_packing="contiguous" if packing == CONTIGUOUS else "frame_aligned",
                 max_units=ocfg.max_units, num_pages=ocfg.num_pages)
    return oc, hc


def _same(oc, hc):
    ids, lens = hc.visible_table()
    oids, olens = oc.visible_table()
    assert ids.tolist() == oids and lens.tolist() == olens
    assert hc.state() == oc.state()


STREAMS = [
    dict(num_scale_units=8, window_units=64, max_units=300),                       # LingBot-Map frames
    dict(num_scale_units=2, window_units=4, max_units=200),                        # tiny stream
    dict(num_scale_units=2, window_units=4, max_units=200, special_packing=CONTIGUOUS),
    dict(num_scale_units=0, window_units=4, patch_tokens=8 * 1374, special_tokens=0, max_units=40),  # chunks
    dict(num_scale_units=0, window_units=0, patch_tokens=1374, special_tokens=0, max_units=60),      # unbounded
    dict(num_scale_units=1, window_units=2, page_size=4, patch_tokens=6, special_tokens=3, max_units=90),
    dict(num_scale_units=1, window_units=2, page_size=8, patch_tokens=5, special_tokens=5, max_units=90,
         special_packing=CONTIGUOUS),
    dict(num_scale_units=3, window_units=1, page_size=64, patch_tokens=64, special_tokens=64, max_units=50),
]


@pytest.mark.parametrize("kw", STREAMS)
def test_random_ops_bit_exact(kw):
    oc, hc = _pair(**kw)
    rng = np.random.default_rng(11)
    for step in range(600):
        r = rng.random()
        if r < 0.65:
            try:
                oc.append()
                o_ok = True
            except OOut:
                o_ok = False
            try:
                hc.append()
                h_ok = True
            except OutOfPages:
                h_ok = False
            assert o_ok == h_ok
        elif r < 0.9:
            try:
                oc.rollback()
                o_ok = True
            except ONo:
                o_ok = False
            try:
                hc.rollback()
                h_ok = True
            except NoUndo:
                h_ok = False
            assert o_ok == h_ok
        elif r < 0.93:
            oc.reset()
            hc.reset()
        _same(oc, hc)


def test_keyframe_stream_10000_bit_exact():
    oc, hc = _pair(num_scale_units=2, window_units=4, max_units=10000)
    for t in range(10000):
        oc.append()
        hc.append()
        if not is_keyframe(t, 2, 4):
            oc.rollback()
            hc.rollback()
        if t % 97 == 0 or t > 9990:
            _same(oc, hc)
    st = hc.state()
    assert st["num_units"] == 2502 and len(st["special_pages"]) == 60
    assert hc.visible_table()[1][-1] == 144


def test_required_pages_matches_oracle():
    from oracle import required_pages
    for kw in STREAMS:
        kw = dict(kw)
        packing = kw.pop("special_packing", FRAME_ALIGNED)
        ocfg = OracleConfig(num_heads=1, head_dim=1, special_packing=packing, **kw)
        hc = KvCache(num_heads=1, head_dim=1, page_size=ocfg.page_size, patch_tokens=ocfg.patch_tokens,
                     special_tokens=ocfg.special_tokens, num_scale_units=ocfg.num_scale_units,
                     window_units=ocfg.window_units,
                     special_packing="contiguous" if packing == CONTIGUOUS else "frame_aligned",
                     max_units=ocfg.max_units)
        assert hc.num_pages == required_pages(ocfg)


def test_error_paths():
    lib = L.lib()
    cfg = L.KvcConfig(1, 64, 256, 0, 256, 6, 1, 2, 0, 10, 3)
    h = C.c_void_p()
    assert lib.kvc_create(C.byref(cfg), None, None, C.byref(h)) == 0
    assert lib.kvc_rollback_last_frame(h) == L.KVC_ERR_NO_UNDO
    assert lib.kvc_append_frame(h, None, None, None) == 0
    assert lib.kvc_append_frame(h, None, None, None) == 0
    assert lib.kvc_append_frame(h, None, None, None) == L.KVC_ERR_OUT_OF_PAGES   # 3 pages only
    assert b"pages" in lib.kvc_last_error()
    n = C.c_int32()
    ids = (C.c_int32 * 1)()
    lens = (C.c_int32 * 1)()
    assert lib.kvc_build_visible_table(h, ids, lens, 1, C.byref(n), None) == L.KVC_ERR_BUFFER_TOO_SMALL
    assert n.value == 3
    # host-only handle refuses data pointers
    assert lib.kvc_append_frame(h, C.c_void_p(16), C.c_void_p(16), None) == L.KVC_ERR_INVALID_ARGUMENT
    assert lib.kvc_destroy(h) == 0
    bad = L.KvcConfig(0, 64, 256, 0, 256, 6, 1, 2, 0, 10, 0)
    assert lib.kvc_create(C.byref(bad), None, None, C.byref(h)) == L.KVC_ERR_INVALID_ARGUMENT
    # device pools need head_dim 64 and page_size multiple of 64
    odd = L.KvcConfig(1, 32, 256, 0, 256, 6, 1, 2, 0, 10, 0)
    assert lib.kvc_create(C.byref(odd), C.c_void_p(256), C.c_void_p(256), C.byref(h)) == L.KVC_ERR_UNSUPPORTED
    # attention argument checks run on the host
    a = L.PagedAttnArgs()
    a.dtype, a.num_heads, a.head_dim, a.page_size, a.sm_scale = 0, 1, 128, 256, 0.1
    sz = C.c_size_t()
    assert lib.paged_attn_workspace_size(C.byref(a), C.byref(sz)) == L.KVC_ERR_UNSUPPORTED
    a.head_dim = 64
    a.sm_scale = float("nan")
    assert lib.paged_attn_workspace_size(C.byref(a), C.byref(sz)) == L.KVC_ERR_INVALID_ARGUMENT
    # device pointers must be 16-byte aligned (checked before any device work)
    a.sm_scale = 0.125
    assert lib.paged_attn_workspace_size(C.byref(a), C.byref(sz)) == 0
    for field in ("q", "k_pool", "v_pool", "o", "workspace"):
        setattr(a, field, C.c_void_p(4096 + 8))
        assert lib.paged_attn_workspace_size(C.byref(a), C.byref(sz)) == L.KVC_ERR_INVALID_ARGUMENT, field
        setattr(a, field, C.c_void_p(4096))
        assert lib.paged_attn_workspace_size(C.byref(a), C.byref(sz)) == 0, field
    # the public merge checks its vectors' alignment before launching anything
    f32 = C.c_void_p(4096 + 4)
    assert lib.paged_attn_merge(L.KVC_DTYPE_F32, 2, 4, 1, 64, f32, C.c_void_p(4096), C.c_void_p(4096), None,
                                None) == L.KVC_ERR_INVALID_ARGUMENT


def test_split_choice_and_workspace():
    lib = L.lib()
    a = L.PagedAttnArgs()
    a.dtype, a.num_heads, a.head_dim, a.page_size, a.sm_scale = 0, 16, 64, 256, 0.125
    a.num_seqs, a.total_q, a.max_qo_len, a.max_kv_pages, a.num_pool_pages = 1, 262, 262, 96, 97
    ns = C.c_int32()
    assert lib.paged_attn_num_splits(C.byref(a), C.byref(ns)) == 0
    assert 1 < ns.value <= 48
    sz = C.c_size_t()
    assert lib.paged_attn_workspace_size(C.byref(a), C.byref(sz)) == 0
    assert sz.value >= ns.value * 262 * 16 * 65 * 4
    a.num_splits = 1
    assert lib.paged_attn_workspace_size(C.byref(a), C.byref(sz)) == 0 and sz.value == 0
    # a 10,992-query chunk over 172 pages: 352 query tiles of 512 rows fill 1.375
    # rounds of the chip unsplit; 5 splits give 7 rounds, the last 88% full
    a.num_splits, a.total_q, a.max_qo_len, a.max_kv_pages = 0, 10992, 10992, 172
    assert lib.paged_attn_num_splits(C.byref(a), C.byref(ns)) == 0 and ns.value == 5
    # 100 frames x 1374 queries over 600 pages (100 one-frame units of 6 pages):
    # 4,304 tiles nearly fill 17 rounds, no split
    a.total_q, a.max_qo_len, a.max_kv_pages = 137400, 137400, 600
    assert lib.paged_attn_num_splits(C.byref(a), C.byref(ns)) == 0 and ns.value == 1


def test_attend_batch_argument_checks():
    """kvc_attend_batch validates the batch on the host (no pool memory is touched here)."""
    lib = L.lib()
    H, P, d = 2, 256, 64
    cfg = L.KvcConfig(H, d, P, 0, 256, 6, 1, 2, 0, 10, 0)
    n = C.c_int32()
    assert lib.kvc_required_pages(C.byref(cfg), C.byref(n)) == 0
    page_bytes = H * P * d * 2
    base_k, base_v = 1 << 32, 1 << 33          # placeholder addresses, never dereferenced
    hs = []
    for i in range(3):
        h = C.c_void_p()
        assert lib.kvc_create(C.byref(cfg), C.c_void_p(base_k + i * n.value * page_bytes),
                              C.c_void_p(base_v + i * n.value * page_bytes), C.byref(h)) == 0
        hs.append(h)
    for h in hs:
        assert lib.kvc_append_frame(h, None, None, None) in (0, L.KVC_ERR_INVALID_ARGUMENT)
    arr = (C.c_void_p * 3)(*[h.value for h in hs])
    qo = (C.c_int32 * 4)(0, 262, 262, 400)
    sz = C.c_size_t()
    assert lib.kvc_attend_batch_workspace_size(arr, 3, qo, C.byref(sz)) == 0
    # bad offsets, counts and sizes
    assert lib.kvc_attend_batch_workspace_size(arr, 0, qo, C.byref(sz)) == L.KVC_ERR_INVALID_ARGUMENT
    assert lib.kvc_attend_batch_workspace_size(arr, 17, qo, C.byref(sz)) == L.KVC_ERR_UNSUPPORTED
    bad_qo = (C.c_int32 * 4)(1, 262, 262, 400)
    assert lib.kvc_attend_batch_workspace_size(arr, 3, bad_qo, C.byref(sz)) == L.KVC_ERR_INVALID_ARGUMENT
    dec_qo = (C.c_int32 * 4)(0, 262, 100, 400)
    assert lib.kvc_attend_batch_workspace_size(arr, 3, dec_qo, C.byref(sz)) == L.KVC_ERR_INVALID_ARGUMENT
    # NULL q with a valid batch is rejected before anything is launched
    assert lib.kvc_attend_batch(arr, 3, None, qo, 0.0, None, None, None, 0, None) == L.KVC_ERR_INVALID_ARGUMENT
    # a pool that is not a whole number of pages into the shared allocation
    odd = C.c_void_p()
    assert lib.kvc_create(C.byref(cfg), C.c_void_p(base_k + 3 * n.value * page_bytes + 128),
                          C.c_void_p(base_v + 3 * n.value * page_bytes + 128), C.byref(odd)) == 0
    arr2 = (C.c_void_p * 2)(hs[0].value, odd.value)
    qo2 = (C.c_int32 * 3)(0, 10, 20)
    assert lib.kvc_attend_batch_workspace_size(arr2, 2, qo2, C.byref(sz)) == L.KVC_ERR_INVALID_ARGUMENT
    assert b"whole pages" in lib.kvc_last_error()
    # K and V at different page offsets
    skew = C.c_void_p()
    assert lib.kvc_create(C.byref(cfg), C.c_void_p(base_k + 3 * n.value * page_bytes),
                          C.c_void_p(base_v + 4 * n.value * page_bytes), C.byref(skew)) == 0
    arr3 = (C.c_void_p * 2)(hs[0].value, skew.value)
    assert lib.kvc_attend_batch_workspace_size(arr3, 2, qo2, C.byref(sz)) == L.KVC_ERR_INVALID_ARGUMENT
    # a different head count
    cfg4 = L.KvcConfig(4, d, P, 0, 256, 6, 1, 2, 0, 10, 0)
    other = C.c_void_p()
    assert lib.kvc_create(C.byref(cfg4), C.c_void_p(base_k + 8 * n.value * page_bytes),
                          C.c_void_p(base_v + 8 * n.value * page_bytes), C.byref(other)) == 0
    arr4 = (C.c_void_p * 2)(hs[0].value, other.value)
    assert lib.kvc_attend_batch_workspace_size(arr4, 2, qo2, C.byref(sz)) == L.KVC_ERR_INVALID_ARGUMENT
    # host-only caches cannot attend
    ho = C.c_void_p()
    assert lib.kvc_create(C.byref(cfg), None, None, C.byref(ho)) == 0
    arr5 = (C.c_void_p * 1)(ho.value)
    qo1 = (C.c_int32 * 2)(0, 5)
    assert lib.kvc_attend_batch_workspace_size(arr5, 1, qo1, C.byref(sz)) == L.KVC_ERR_INVALID_ARGUMENT
    for h in hs + [odd, skew, other, ho]:
        assert lib.kvc_destroy(h) == 0
