"""Several caches attending in one launch (kvc_attend_batch), each stream checked against the oracle."""
import numpy as np
import pytest

import synth
from gpu_helpers import check_attention, log, to_dev
from oracle import OracleCache, OracleConfig, attention_f64, is_keyframe
from oracle import to_f64 as bits_f64

pytestmark = pytest.mark.gpu

NAN_BF16 = 0x7FC0


def _streams(caches, oracles, frames, seed, H, P, X, S, interval=1, bank=None):
    """Append frames[i] units to stream i (device and oracle); keyframe skipping with `interval`."""
    for i, (c, oc) in enumerate(zip(caches, oracles)):
        for t in range(frames[i]):
            if bank is None:
                k = synth.normal_tokens(seed + i, 0, t, synth.KIND_K, P + X, H, 64, "bf16")
                v = synth.normal_tokens(seed + i, 0, t, synth.KIND_V, P + X, H, 64, "bf16")
            else:
                _, k, v = bank[(i + t) % len(bank)]
            oc.append(k, v)
            c.append(to_dev(k, "bf16"), to_dev(v, "bf16"))
            if t < frames[i] - 1 and not is_keyframe(t, S, interval):
                oc.rollback()
                c.rollback()


def test_batch_ragged_streams_against_oracle():
    import torch
    from paged_sliding_window_kv_amd import attend_batch, shared_pool_caches
    H, P, X, S, W = 4, 256, 6, 2, 4
    frames = [1, 5, 9, 14, 3]
    qlens = [262, 100, 0, 262, 37]
    log(f"batch of {len(frames)} streams, frames {frames}, queries {qlens}")
    kw = dict(num_heads=H, dtype="bf16", patch_tokens=P, special_tokens=X, num_scale_units=S, window_units=W,
              max_units=20)
    caches = shared_pool_caches(len(frames), "cuda", **kw)
    # every slot not written by an append is NaN: a read of a stale slot or of another stream's page shows
    for c in caches:
        c.k_pool.view(torch.int16).fill_(NAN_BF16)
        c.v_pool.view(torch.int16).fill_(NAN_BF16)
    oracles = [OracleCache(OracleConfig(num_heads=H, head_dim=64, patch_tokens=P, special_tokens=X, num_scale_units=S,
                                        window_units=W, max_units=20, store_dtype="bf16")) for _ in frames]
    _streams(caches, oracles, frames, 30, H, P, X, S, interval=2)
    qs = [synth.normal_tokens(40 + i, 0, 0, synth.KIND_Q, n, H, 64, "bf16") for i, n in enumerate(qlens)]
    qo = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    o, lse = attend_batch(caches, to_dev(np.concatenate(qs), "bf16"), qo)
    torch.cuda.synchronize()
    for i, oc in enumerate(oracles):
        if qlens[i] == 0:
            continue
        gk, gv = oc.gather()
        ro, rl = attention_f64(bits_f64(qs[i]), bits_f64(gk), bits_f64(gv))
        check_attention(o[qo[i]:qo[i + 1]], lse[qo[i]:qo[i + 1]], ro, rl, "bf16", f"stream {i} Lk={gk.shape[1]}")
        # the pages each stream sees are its own
        ids, _ = caches[i].visible_table()
        assert ids.tolist() == oc.visible_table()[0]


def test_batch_of_eight_lingbot_streams():
    """Eight 16-head streams at staggered depths in one launch: rows match each cache's own kvc_attend."""
    import torch
    from paged_sliding_window_kv_amd import attend_batch, shared_pool_caches
    H, P, X, S, W = 16, 256, 6, 8, 64
    frames = [1, 9, 30, 60, 72, 80, 90, 100]
    log(f"batch of 8 LingBot-shaped streams, frames {frames}")
    kw = dict(num_heads=H, dtype="bf16", patch_tokens=P, special_tokens=X, num_scale_units=S, window_units=W,
              max_units=100)
    caches = shared_pool_caches(len(frames), "cuda", **kw)
    bank = [synth.frame_qkv(50, 0, i, P + X, H, 64, "bf16") for i in range(5)]
    oracles = [OracleCache(OracleConfig(num_heads=H, head_dim=64, patch_tokens=P, special_tokens=X, num_scale_units=S,
                                        window_units=W, max_units=100, store_dtype="bf16")) for _ in frames]
    _streams(caches, oracles, frames, 0, H, P, X, S, bank=bank)
    qs = [bank[(i + 3) % len(bank)][0] for i in range(len(frames))]
    qo = np.concatenate([[0], np.cumsum([len(x) for x in qs])]).astype(np.int32)
    o, lse = attend_batch(caches, to_dev(np.concatenate(qs), "bf16"), qo)
    torch.cuda.synchronize()
    for i, c in enumerate(caches):
        o1, l1 = c.attend(to_dev(qs[i], "bf16"))
        torch.cuda.synchronize()
        d = (o[qo[i]:qo[i + 1]].float() - o1.float()).abs().max().item()
        dl = (lse[qo[i]:qo[i + 1]] - l1).abs().max().item()
        log(f"  stream {i}: batch vs own call max|dO|={d:.2e} max|dlse|={dl:.2e}")
        assert d <= 4e-3 and dl <= 1e-4
    for i in (0, 7):
        gk, gv = oracles[i].gather()
        ro, rl = attention_f64(bits_f64(qs[i]), bits_f64(gk), bits_f64(gv))
        check_attention(o[qo[i]:qo[i + 1]], lse[qo[i]:qo[i + 1]], ro, rl, "bf16", f"stream {i} Lk={gk.shape[1]}")
