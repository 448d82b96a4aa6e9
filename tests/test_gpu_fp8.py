"""FP8 (E4M3) KV pages on the device: quantising append bit-exact, attention against the oracle."""
import numpy as np
import pytest

import synth
from gpu_helpers import check_attention, log, to_dev
from oracle import CONTIGUOUS, FRAME_ALIGNED, OracleCache, OracleConfig, attention_f64, is_keyframe
from oracle import to_f64 as bits_f64

pytestmark = pytest.mark.gpu

CASES = [
    # (heads, patch, special, S, W, packing, frames, keyframe interval)
    (4, 256, 6, 2, 4, FRAME_ALIGNED, 40, 1),
    (2, 2 * 1374, 0, 0, 2, FRAME_ALIGNED, 5, 1),     # chunk units: 11 pages, tail 188
    (2, 100, 70, 1, 2, CONTIGUOUS, 20, 2),            # specials straddle pages, keyframe skips
]


def _caches(H, P, X, S, W, packing, frames):
    from paged_sliding_window_kv_amd import KvCache
    oc = OracleCache(OracleConfig(num_heads=H, head_dim=64, patch_tokens=P, special_tokens=X, num_scale_units=S,
                                  window_units=W, special_packing=packing, max_units=frames, store_dtype="fp8"))
    dc = KvCache(num_heads=H, dtype="fp8", patch_tokens=P, special_tokens=X, num_scale_units=S, window_units=W,
                 special_packing="contiguous" if packing == CONTIGUOUS else "frame_aligned", max_units=frames,
                 device="cuda")
    # poison: every code NaN (0xFF), every exponent 127; a slot the append misses, or one the
    # attention reads past a page's length, shows up
    dc.k_pool.fill_(0xFF)
    dc.v_pool.fill_(0xFF)
    dc.k_exps.fill_(127)
    dc.v_exps.fill_(127)
    return oc, dc


@pytest.mark.parametrize("case", CASES)
def test_fp8_append_bit_exact(case):
    import torch
    H, P, X, S, W, packing, frames, interval = case
    log(f"fp8 append case {case}")
    oc, dc = _caches(H, P, X, S, W, packing, frames)
    for t in range(frames):
        k = synth.normal_tokens(8, 0, t, synth.KIND_K, P + X, H, 64, "bf16")
        v = synth.normal_tokens(8, 0, t, synth.KIND_V, P + X, H, 64, "bf16")
        if t == 3:
            k = k.copy()
            k[5] = 0        # an all-zero token: exponent -127, codes 0
        oc.append(k, v)
        dc.append(to_dev(k, "bf16"), to_dev(v, "bf16"))
        if not is_keyframe(t, S, interval):
            oc.rollback()
            dc.rollback()
        if t % 5 == 0 or t == frames - 1:
            torch.cuda.synchronize()
            kc, vc = dc.k_codes.cpu().numpy(), dc.v_codes.cpu().numpy()
            ke, ve = dc.k_exps.cpu().numpy(), dc.v_exps.cpu().numpy()
            ids, lens = oc.visible_table()
            assert dc.visible_table()[0].tolist() == ids
            for p, n in zip(ids, lens):
                assert np.array_equal(kc[p, :, :n], oc.k_pool[p, :, :n]), f"K codes page {p}"
                assert np.array_equal(vc[p, :, :n], oc.v_pool[p, :, :n]), f"V codes page {p}"
                assert np.array_equal(ke[p, :, :n], oc.k_exp[p, :, :n]), f"K exponents page {p}"
                assert np.array_equal(ve[p, :, :n], oc.v_exp[p, :, :n]), f"V exponents page {p}"


@pytest.mark.parametrize("case", CASES)
def test_fp8_attention_against_oracle(case):
    import torch
    H, P, X, S, W, packing, frames, interval = case
    log(f"fp8 attention case {case}")
    oc, dc = _caches(H, P, X, S, W, packing, frames)
    for t in range(frames):
        q, k, v = synth.frame_qkv(9, 0, t, P + X, H, 64, "bf16")
        oc.append(k, v)
        dc.append(to_dev(k, "bf16"), to_dev(v, "bf16"))
        if t % 7 == 0 or t == frames - 1:
            gk, gv = oc.gather()
            ro, rl = attention_f64(bits_f64(q), gk, gv)
            for ns in (0, 3):
                o, lse = dc.attend(to_dev(q, "bf16"), num_splits=ns)
                torch.cuda.synchronize()
                check_attention(o, lse, ro, rl, "bf16", f"t={t} splits={ns or 'auto'} Lk={gk.shape[1]}")
        if not is_keyframe(t, S, interval):
            oc.rollback()
            dc.rollback()


def test_fp8_peaky_queries():
    """Large scores (q scaled by 4): the running-maximum rescale path with FP8 pages."""
    import torch
    H, P, X = 4, 256, 6
    oc, dc = _caches(H, P, X, 2, 4, FRAME_ALIGNED, 12)
    for t in range(12):
        q, k, v = synth.frame_qkv(10, 0, t, P + X, H, 64, "bf16", q_scale=4.0)
        oc.append(k, v)
        dc.append(to_dev(k, "bf16"), to_dev(v, "bf16"))
    gk, gv = oc.gather()
    ro, rl = attention_f64(bits_f64(q), gk, gv)
    o, lse = dc.attend(to_dev(q, "bf16"))
    torch.cuda.synchronize()
    check_attention(o, lse, ro, rl, "bf16", f"peaky Lk={gk.shape[1]}")


def test_fp8_peaky_queries_large_tiles():
    """Large scores (q scaled by 4) with chunk units of 2 x 1374 tokens: FP8 pages on the
    512-row tiles, through the running-maximum rescale path, with and without splits."""
    import torch
    H, P = 2, 2 * 1374
    oc, dc = _caches(H, P, 0, 0, 3, FRAME_ALIGNED, 5)
    for t in range(5):
        q, k, v = synth.frame_qkv(14, 0, t, P, H, 64, "bf16", q_scale=4.0)
        oc.append(k, v)
        dc.append(to_dev(k, "bf16"), to_dev(v, "bf16"))
    gk, gv = oc.gather()
    ro, rl = attention_f64(bits_f64(q), gk, gv)
    for ns in (0, 1, 4):
        o, lse = dc.attend(to_dev(q, "bf16"), num_splits=ns)
        torch.cuda.synchronize()
        check_attention(o, lse, ro, rl, "bf16", f"peaky chunks splits={ns or 'auto'} Lk={gk.shape[1]}")


def test_fp8_lingbot_stream_1000_frames():
    """The 1000-frame LingBot-shaped stream with FP8 pages: last step (24,432 keys) against the oracle."""
    import torch
    from paged_sliding_window_kv_amd import KvCache
    H, P, X, S, W, frames = 16, 256, 6, 8, 64, 1000
    log("fp8 lingbot stream 1000 frames")
    bank = [synth.frame_qkv(11, 0, i, P + X, H, 64, "bf16") for i in range(6)]
    dev_bank = [tuple(to_dev(x, "bf16") for x in f) for f in bank]
    oc = OracleCache(OracleConfig(num_heads=H, head_dim=64, patch_tokens=P, special_tokens=X, num_scale_units=S,
                                  window_units=W, max_units=frames, store_dtype="fp8"))
    dc = KvCache(num_heads=H, dtype="fp8", patch_tokens=P, special_tokens=X, num_scale_units=S, window_units=W,
                 max_units=frames, device="cuda")
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    for t in range(frames):
        _, k, v = bank[t % len(bank)]
        _, dk, dv = dev_bank[t % len(bank)]
        oc.append(k, v)
        dc.append(dk, dv)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    q = bank[(frames - 1) % len(bank)][0]
    o, lse = dc.attend(dev_bank[(frames - 1) % len(bank)][0])
    torch.cuda.synchronize()
    gk, gv = oc.gather()
    assert gk.shape[1] == 24432
    ro, rl = attention_f64(bits_f64(q), gk, gv)
    check_attention(o, lse, ro, rl, "bf16", "fp8 t=999 Lk=24432")
    # half the bytes of the bf16 pools, plus one exponent byte per 64 values
    assert dc.k_pool.numel() == dc.num_pages * H * P * 65
