"""Windowed inference on the device: 25,000 frames, attention checked against the oracle, memory flat."""
import pytest

import synth
from gpu_helpers import check_attention, log, to_dev
from oracle import OracleCache, OracleConfig, OracleWindowed, attention_f64, is_keyframe
from oracle import to_f64 as bits_f64

pytestmark = pytest.mark.gpu


def test_windowed_stream_25000_frames():
    import torch
    from paged_sliding_window_kv_amd import KvCache, WindowedStream
    H, P, X, S, W, N = 2, 256, 6, 8, 64, 2
    slots, overlap, frames = 128, 16, 25000
    log(f"windowed stream: {frames} frames, window {slots} slots, overlap {overlap}, keyframe interval {N}")
    bank = [synth.frame_qkv(70, 0, i, P + X, H, 64, "bf16") for i in range(7)]
    dev_bank = [tuple(to_dev(x, "bf16") for x in f) for f in bank]
    oc = OracleWindowed(OracleCache(OracleConfig(num_heads=H, head_dim=64, patch_tokens=P, special_tokens=X,
                                                 num_scale_units=S, window_units=W, max_units=slots + 1,
                                                 store_dtype="bf16")), slots, overlap)
    dc = KvCache(num_heads=H, dtype="bf16", patch_tokens=P, special_tokens=X, num_scale_units=S, window_units=W,
                 max_units=slots + 1, device="cuda")
    ws = WindowedStream(dc, slots, overlap)
    o = torch.empty((P + X, H, 64), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((P + X, H), dtype=torch.float32, device="cuda")
    wsp = torch.empty(max(dc.workspace_bytes(P + X), 256), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    checks = 0
    for t in range(frames):
        b = (t * 3) % len(bank)
        q, k, v = bank[b]
        dq, dk, dv = dev_bank[b]
        r1 = oc.append(k, v)
        r2 = ws.append(dk, dv)
        assert r1 == r2
        if t % 3125 == 0 or t == frames - 1 or (r2 and ws.windows in (1, 2)):
            dc.attend(dq, o, lse, workspace=wsp)
            gk, gv = oc.cache.gather()
            ro, rl = attention_f64(bits_f64(q), bits_f64(gk), bits_f64(gv))
            check_attention(o, lse, ro, rl, "bf16", f"t={t} window {ws.windows} Lk={gk.shape[1]}")
            checks += 1
        if is_keyframe(t, S, N):
            oc.keep()
            ws.keep()
        else:
            oc.drop()
            ws.drop()
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    assert ws.windows == oc.windows and ws.windows > 90
    assert dc.state() == oc.cache.state()
    assert checks >= 10


@pytest.mark.parametrize("dtype", ["bf16", "fp8", "f32"])
def test_windowed_ring_slots_and_restarts(dtype):
    """Every page type: each kept unit's K/V sit bit for bit in its ring slot (written by the append
    itself), and attention right after each restart matches the oracle (the shared units re-appended
    from the ring)."""
    import numpy as np
    import torch
    from paged_sliding_window_kv_amd import KvCache, WindowedStream
    H, P, X, S, W, N = 2, 256, 6, 2, 4, 3
    slots, overlap, frames = 7, 3, 120
    act = "f32" if dtype == "f32" else "bf16"
    log(f"windowed ring: {dtype} pages, {frames} frames, window {slots}, overlap {overlap}, interval {N}")
    bank = [synth.frame_qkv(74, 0, i, P + X, H, 64, act) for i in range(5)]
    dev_bank = [tuple(to_dev(x, act) for x in f) for f in bank]
    oc = OracleWindowed(OracleCache(OracleConfig(num_heads=H, head_dim=64, patch_tokens=P, special_tokens=X,
                                                 num_scale_units=S, window_units=W, max_units=slots + 1,
                                                 store_dtype=dtype)), slots, overlap)
    dc = KvCache(num_heads=H, dtype=dtype, patch_tokens=P, special_tokens=X, num_scale_units=S, window_units=W,
                 max_units=slots + 1, device="cuda")
    ws = WindowedStream(dc, slots, overlap)
    kring, vring = ws._ring
    assert kring.shape[0] == overlap + 1
    keeps = restarts = 0
    for t in range(frames):
        b = (t * 2) % len(bank)
        q, k, v = bank[b]
        dq, dk, dv = dev_bank[b]
        r1 = oc.append(k, v)
        r2 = ws.append(dk, dv)
        assert r1 == r2
        if r2:
            restarts += 1
            o, lse = dc.attend(dq)
            torch.cuda.synchronize()
            gk, gv = oc.cache.gather()
            if dtype == "fp8":  # gather gives the dequantised values
                ro, rl = attention_f64(bits_f64(q), gk, gv)
            else:
                ro, rl = attention_f64(bits_f64(q), bits_f64(gk), bits_f64(gv))
            check_attention(o, lse, ro, rl, act, f"{dtype} t={t} restart {ws.windows} Lk={gk.shape[1]}")
        if is_keyframe(t, S, N):
            oc.keep()
            ws.keep()
            keeps += 1
            slot = (keeps - 1) % (overlap + 1)
            torch.cuda.synchronize()
            assert torch.equal(kring[slot], dk) and torch.equal(vring[slot], dv), (t, slot)
        else:
            oc.drop()
            ws.drop()
    assert restarts == ws.windows == oc.windows >= 3
    assert dc.state() == oc.cache.state()
    assert np.array_equal(dc.visible_table()[0], np.array(oc.cache.visible_table()[0]))


def test_windowed_bench_shape_25000_frames_16_heads():
    """The shape bench.py --workload windowed times: 16 heads, 8 scale frames, a 64-frame window, a restart
    per 128 kept units sharing 16, a keyframe every second frame, 25,000 frames.  All 262 queries x 16 heads
    against the oracle at the fullest window (the frame before the first restart, 19,200 keys), at the first
    two restarts, every 5,000 frames and at the end; the tables and state equal the oracle's throughout."""
    import torch
    from paged_sliding_window_kv_amd import KvCache, WindowedStream
    H, P, X, S, W, N = 16, 256, 6, 8, 64, 2
    slots, overlap, frames = 128, 16, 25000
    log(f"windowed bench shape: {H} heads, {frames} frames")
    bank = [synth.frame_qkv(76, 0, i, P + X, H, 64, "bf16") for i in range(7)]
    dev_bank = [tuple(to_dev(x, "bf16") for x in f) for f in bank]
    oc = OracleWindowed(OracleCache(OracleConfig(num_heads=H, head_dim=64, patch_tokens=P, special_tokens=X,
                                                 num_scale_units=S, window_units=W, max_units=slots + 1,
                                                 store_dtype="bf16")), slots, overlap)
    dc = KvCache(num_heads=H, dtype="bf16", patch_tokens=P, special_tokens=X, num_scale_units=S, window_units=W,
                 max_units=slots + 1, device="cuda")
    ws = WindowedStream(dc, slots, overlap)
    wsp = torch.empty(max(dc.workspace_bytes(P + X), 256), dtype=torch.uint8, device="cuda")
    o = torch.empty((P + X, H, 64), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((P + X, H), dtype=torch.float32, device="cuda")
    # the 128th kept unit is frame 8 + 2 * 119 = 246, so frame 247 restarts; frame 246 sees the
    # fullest window (127 kept units plus its own)
    first = S + N * (slots - S - 1) + 1
    assert first == 247
    checked_lk = []
    for t in range(frames):
        b = (t * 3) % len(bank)
        q, k, v = bank[b]
        r1 = oc.append(k, v)
        r2 = ws.append(dev_bank[b][1], dev_bank[b][2])
        assert r1 == r2, t
        if t == first - 1 or (r2 and ws.windows <= 2) or t % 5000 == 4999:
            dc.attend(dev_bank[b][0], o, lse, workspace=wsp)
            gk, gv = oc.cache.gather()
            ro, rl = attention_f64(bits_f64(q), bits_f64(gk), bits_f64(gv))
            check_attention(o, lse, ro, rl, "bf16", f"t={t} window {ws.windows} Lk={gk.shape[1]}")
            checked_lk.append(gk.shape[1])
        if is_keyframe(t, S, N):
            oc.keep()
            ws.keep()
        else:
            oc.drop()
            ws.drop()
        if t % 2500 == 0:
            assert dc.visible_table()[0].tolist() == oc.cache.visible_table()[0], t
    assert ws.windows == oc.windows == 111
    assert dc.state() == oc.cache.state()
    assert max(checked_lk) == 19200 and len(checked_lk) >= 8
