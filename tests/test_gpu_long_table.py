"""Visible tables longer than the launch arguments hold (more than 640 entries), through kvc_attend.

A LingBot-Map-shaped cache that is never restarted keeps every frame's 6
special tokens ("LingBot-Map Paged KV Cache", section 2: special pages are
append-only), so after about 23,900 frames its visible table passes 640
entries; at 25,000 frames it holds 72 patch pages and 596 special pages.  The
library then stages the table in pinned host memory and copies it into the
workspace on the launch stream.  Two heads keep the oracle's work small; the
table shapes are the full ones.
"""
import numpy as np
import pytest

import synth
from gpu_helpers import check_attention, log, to_dev
from oracle import OracleCache, OracleConfig, attention_f64
from oracle import to_f64 as bits_f64

pytestmark = pytest.mark.gpu


def test_lingbot_cache_25000_frames_668_entries():
    import torch
    from paged_sliding_window_kv_amd import KvCache
    H, P, X, S, W, frames = 2, 256, 6, 8, 64, 25000
    log(f"long table: {frames} frames, H={H}")
    bank = [synth.frame_qkv(41, 0, i, P + X, H, 64, "bf16") for i in range(5)]
    dev_bank = [tuple(to_dev(x, "bf16") for x in f) for f in bank]
    dc = KvCache(num_heads=H, dtype="bf16", patch_tokens=P, special_tokens=X, num_scale_units=S, window_units=W,
                 max_units=frames, device="cuda")
    oc = OracleCache(OracleConfig(num_heads=H, head_dim=64, patch_tokens=P, special_tokens=X, num_scale_units=S,
                                  window_units=W, max_units=frames, store_dtype="bf16"))
    o = torch.empty((P + X, H, 64), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((P + X, H), dtype=torch.float32, device="cuda")
    ws = torch.empty(dc.workspace_bytes(P + X), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    checks = 0
    for t in range(frames):
        b = t % len(bank)
        q, k, v = bank[b]
        dq, dk, dv = dev_bank[b]
        oc.append(k, v)
        dc.append(dk, dv)
        n = S + W + -(-(t + 1) // 42)
        if t % 5000 == 0:
            log(f"  frame {t}")
        if t in (23855, 23856, 24999):  # 640, 641 and 668 entries
            ids, lens = dc.visible_table()
            assert len(ids) == n
            oids, olens = oc.visible_table()
            assert ids.tolist() == oids and lens.tolist() == olens
            dc.attend(dq, o, lse, workspace=ws)
            gk, gv = oc.gather()
            ro, rl = attention_f64(bits_f64(q), bits_f64(gk), bits_f64(gv))
            check_attention(o, lse, ro, rl, "bf16", f"t={t} entries={n} Lk={gk.shape[1]}")
            checks += 1
    assert checks == 3
    assert len(dc.visible_table()[0]) == 668
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    # more calls than the 16 staging slots, back to back: every result must stay the table's
    outs = []
    for i in range(20):
        oi, li = dc.attend(dev_bank[i % len(bank)][0], workspace=ws)
        outs.append((oi, li))
    torch.cuda.synchronize()
    gk, gv = oc.gather()
    for i in (0, 1, 17, 19):
        ro, rl = attention_f64(bits_f64(bank[i % len(bank)][0]), bits_f64(gk), bits_f64(gv))
        check_attention(outs[i][0], outs[i][1], ro, rl, "bf16", f"repeat call {i}")
    for i in range(len(bank), 20):
        j = i % len(bank)
        assert torch.equal(outs[i][0], outs[j][0]) and torch.equal(outs[i][1], outs[j][1]), i
    # the page-subset path over the same long table (keep 1.0 is the whole table)
    os_, ls_ = dc.attend_subset(dev_bank[0][0], 1.0, 5, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(os_, outs[0][0]) and torch.equal(ls_, outs[0][1])
    # and a real subset of it, against the oracle over the same entries
    ids, lens = dc.subset_table(0.97, 9, keep_first=S, keep_last=4)  # 12 + ceil(0.97 * 656) = 649 entries
    assert len(ids) > 640
    os_, ls_ = dc.attend_subset(dev_bank[1][0], 0.97, 9, keep_first=S, keep_last=4, workspace=ws)
    sk, sv = oc.gather(ids.tolist(), lens.tolist())
    ro, rl = attention_f64(bits_f64(bank[1][0]), bits_f64(sk), bits_f64(sv))
    check_attention(os_, ls_, ro, rl, "bf16", f"subset of {len(ids)} entries")


def test_long_table_needs_the_table_region():
    """A workspace without room for the table region is refused, the cache unchanged."""
    import torch
    from paged_sliding_window_kv_amd import KvCache, lib
    from paged_sliding_window_kv_amd import _lib as L
    dc = KvCache(num_heads=1, dtype="bf16", patch_tokens=256, special_tokens=6, num_scale_units=0, window_units=1,
                 max_units=42 * 700, device="cuda")
    k = torch.zeros((262, 1, 64), dtype=torch.bfloat16, device="cuda")
    for _ in range(42 * 660):
        dc.append(k, k)
    assert len(dc.visible_table()[0]) > 640
    st = dc.state()
    q = torch.zeros((262, 1, 64), dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((262, 1), dtype=torch.float32, device="cuda")
    small = torch.empty(256, dtype=torch.uint8, device="cuda")
    s = lib().kvc_attend(dc.handle, q.data_ptr(), 262, 0.0, o.data_ptr(), lse.data_ptr(), small.data_ptr(), 256,
                         torch.cuda.current_stream().cuda_stream)
    assert s == L.KVC_ERR_BUFFER_TOO_SMALL
    assert dc.state() == st
    o, lse = dc.attend(q)  # a workspace of the size the cache asks for
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()
    np.testing.assert_allclose(o.float().cpu().numpy(), 0.0)
