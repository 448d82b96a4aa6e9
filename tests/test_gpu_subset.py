"""Attention over page-subset tables (kvc_attend_subset) against the oracle on the same subsets."""
import numpy as np
import pytest

import synth
from gpu_helpers import check_attention, log, to_dev
from oracle import OracleCache, OracleConfig, attention_f64, subset_table
from oracle import to_f64 as bits_f64

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("shape", ["lingbot", "chunk"])
def test_subset_attention_against_oracle(shape):
    import torch
    from paged_sliding_window_kv_amd import KvCache
    if shape == "lingbot":
        H, P, X, S, W, frames = 4, 256, 6, 2, 6, 16
    else:
        H, P, X, S, W, frames = 4, 2 * 1374, 0, 0, 3, 6      # 11 pages per unit, tail 188
    log(f"subset attention, {shape}")
    dc = KvCache(num_heads=H, dtype="bf16", patch_tokens=P, special_tokens=X, num_scale_units=S, window_units=W,
                 max_units=frames, device="cuda")
    oc = OracleCache(OracleConfig(num_heads=H, head_dim=64, patch_tokens=P, special_tokens=X, num_scale_units=S,
                                  window_units=W, max_units=frames, store_dtype="bf16"))
    for t in range(frames):
        q, k, v = synth.frame_qkv(60, 0, t, P + X, H, 64, "bf16")
        oc.append(k, v)
        dc.append(to_dev(k, "bf16"), to_dev(v, "bf16"))
        if t in (0, frames // 2, frames - 1):
            ids, lens = oc.visible_table()
            n_special = len(oc.state()["special_pages"])
            for r, seed, kf, kl in ((1.0, 1, 0, 0), (0.5, t, S, n_special), (0.25, 99 + t, 0, 0)):
                si, sl = subset_table(ids, lens, r, seed, kf, kl)
                o, lse = dc.attend_subset(to_dev(q, "bf16"), r, seed, kf, kl)
                torch.cuda.synchronize()
                gk, gv = oc.gather(si, sl)
                ro, rl = attention_f64(bits_f64(q), bits_f64(gk), bits_f64(gv))
                check_attention(o, lse, ro, rl, "bf16", f"t={t} r={r} pages {len(si)}/{len(ids)}")
    # keep_ratio 1 is exactly kvc_attend (same table, same launch)
    o1, l1 = dc.attend_subset(to_dev(q, "bf16"), 1.0, 7)
    o2, l2 = dc.attend(to_dev(q, "bf16"))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
