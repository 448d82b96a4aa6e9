"""KV-append scatter on the GPU: pool bytes against the oracle pool, bit-exact."""
import numpy as np
import pytest

import synth
from gpu_helpers import log, to_dev, to_host_bits, v_pool_natural
from oracle import CONTIGUOUS, FRAME_ALIGNED, OracleCache, OracleConfig, is_keyframe

pytestmark = pytest.mark.gpu


def _compare_pools(dc, oc, dtype):
    kd = to_host_bits(dc.k_pool, dtype)                       # [N, H, P, d]
    vd = v_pool_natural(to_host_bits(dc.v_pool, dtype))      # [N, H, d, P] -> [N, H, P, d]
    ids, lens = oc.visible_table()
    assert dc.visible_table()[0].tolist() == ids
    for p, n in zip(ids, lens):
        assert np.array_equal(kd[p, :, :n], oc.k_pool[p, :, :n]), f"K page {p}"
        assert np.array_equal(vd[p, :, :n], oc.v_pool[p, :, :n]), f"V page {p}"


CASES = [
    # (dtype, heads, patch, special, S, W, packing, frames, keyframe interval)
    ("bf16", 4, 256, 6, 2, 4, FRAME_ALIGNED, 60, 1),
    ("f32", 4, 256, 6, 2, 4, FRAME_ALIGNED, 30, 3),
    ("bf16", 2, 256, 6, 1, 3, CONTIGUOUS, 90, 2),
    ("bf16", 3, 1374, 0, 0, 2, FRAME_ALIGNED, 7, 1),       # VGGT frame: 6 pages, tail 94
    ("bf16", 2, 2 * 1374, 0, 0, 2, FRAME_ALIGNED, 5, 1),   # 2-frame chunk: 11 pages, tail 188
    ("f32", 2, 100, 70, 1, 2, CONTIGUOUS, 20, 1),          # odd sizes, specials straddle pages
]


@pytest.mark.parametrize("case", CASES)
def test_append_bit_exact(case):
    import torch
    from paged_sliding_window_kv_amd import KvCache
    dtype, H, P, X, S, W, packing, frames, interval = case
    log(f"append case {case}")
    ocfg = OracleConfig(num_heads=H, head_dim=64, patch_tokens=P, special_tokens=X, num_scale_units=S,
                        window_units=W, special_packing=packing, max_units=frames, store_dtype=dtype)
    oc = OracleCache(ocfg)
    dc = KvCache(num_heads=H, head_dim=64, dtype=dtype, patch_tokens=P, special_tokens=X, num_scale_units=S,
                 window_units=W, special_packing="contiguous" if packing == CONTIGUOUS else "frame_aligned",
                 max_units=frames, device="cuda")
    # poison the pools: any slot the scatter misses shows up as a mismatch
    dc.k_pool.view(torch.int16).fill_(-1)
    dc.v_pool.view(torch.int16).fill_(-1)
    for t in range(frames):
        k = synth.normal_tokens(4, 0, t, synth.KIND_K, P + X, H, 64, dtype)
        v = synth.normal_tokens(4, 0, t, synth.KIND_V, P + X, H, 64, dtype)
        oc.append(k, v)
        dc.append(to_dev(k, dtype), to_dev(v, dtype))
        if not is_keyframe(t, S, interval):
            oc.rollback()
            dc.rollback()
        if t % 7 == 0 or t == frames - 1:
            torch.cuda.synchronize()
            _compare_pools(dc, oc, dtype)
