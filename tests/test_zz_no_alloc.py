"""kvc_attend_noalloc (the form for callers that cannot allocate) against kvc_attend, through the C ABI.

Two calls in a row on one GPU, the second with a smaller input:
  1. a 10,992-query chunk over a 4-chunk window (43,968 keys): kvc_attend
     takes 5 key splits, whose partials (228 MB) exceed the 32 MiB array, so
     the no-alloc form runs with fewer splits; its output must meet the
     parity bar against kvc_attend's;
  2. a LingBot-shaped frame (262 queries, 24,432 keys, 16 splits, 17.4 MB of
     partials): the same split count, so the outputs must be identical.
A visible table of more than 640 entries is refused without launching.
"""
import ctypes as C

import numpy as np
import pytest

from gpu_helpers import BF16_LSE_ABS, BF16_MAX_ABS, BF16_RMS_REL, log

pytestmark = pytest.mark.gpu


def _bar(o, lse, ro, rl, what):
    o = o.float().cpu().numpy().astype(np.float64)
    ro = ro.float().cpu().numpy().astype(np.float64)
    err = float(np.abs(o - ro).max())
    rel = float(np.sqrt(np.mean((o - ro) ** 2)) / np.sqrt(np.mean(ro ** 2)))
    lerr = float(np.abs(lse.cpu().numpy() - rl.cpu().numpy()).max())
    log(f"  {what}: max_abs={err:.3e} rms_rel={rel:.3e} lse={lerr:.3e}")
    assert np.isfinite(o).all()
    assert err <= BF16_MAX_ABS and rel <= BF16_RMS_REL and lerr <= BF16_LSE_ABS, what


def _both(cache, q):
    """(kvc_attend out, lse), (kvc_attend_noalloc out, lse) for the same cache state and queries."""
    import torch
    from paged_sliding_window_kv_amd import _lib as L
    from paged_sliding_window_kv_amd import lib
    lb = lib()
    n, H, d = q.shape
    sp = torch.cuda.current_stream().cuda_stream
    ref = torch.empty_like(q)
    rlse = torch.empty((n, H), dtype=torch.float32, device=q.device)
    wsb = cache.workspace_bytes(n)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=q.device)
    L.check(lb.kvc_attend(cache.handle, q.data_ptr(), n, 0.0, ref.data_ptr(), rlse.data_ptr(), ws.data_ptr(), wsb, sp),
            "kvc_attend")
    out = torch.full_like(q, float("nan"))
    olse = torch.full((n, H), float("nan"), dtype=torch.float32, device=q.device)
    L.check(lb.kvc_attend_noalloc(cache.handle, q.data_ptr(), n, 0.0, out.data_ptr(), olse.data_ptr(), sp),
            "kvc_attend_noalloc")
    torch.cuda.synchronize()
    return (ref, rlse), (out, olse), wsb


def test_noalloc_two_calls_against_kvc_attend():
    import torch
    from paged_sliding_window_kv_amd import KvCache
    from paged_sliding_window_kv_amd import _lib as L
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    # call 1: the chunked step's shapes
    T, H = 8 * 1374, 16
    log("no-alloc call 1: 10,992 queries over 43,968 keys")
    ch = KvCache(num_heads=H, dtype="bf16", patch_tokens=T, special_tokens=0, num_scale_units=0, window_units=4,
                 max_units=5, device="cuda")
    for _ in range(5):
        kv = torch.randn((2, T, H, 64), generator=g, device="cuda").to(torch.bfloat16)
        ch.append(kv[0], kv[1])
    q = torch.randn((T, H, 64), generator=g, device="cuda").to(torch.bfloat16)
    assert ch.num_splits(T) > 1
    (ro, rl), (o, l), wsb = _both(ch, q)
    assert wsb > L.NOALLOC_SCRATCH_BYTES  # kvc_attend's partials would not fit the array
    _bar(o, l, ro, rl, "chunk, fewer splits than kvc_attend")
    del ch, q, ro, rl, o, l
    # call 2: a LingBot frame, smaller input, same split count as kvc_attend
    log("no-alloc call 2: 262 queries over 24,432 keys")
    fr = KvCache(num_heads=H, dtype="bf16", patch_tokens=256, special_tokens=6, num_scale_units=8, window_units=64,
                 max_units=1000, device="cuda")
    bank = torch.randn((4, 2, 262, H, 64), generator=g, device="cuda").to(torch.bfloat16)
    for t in range(1000):
        fr.append(bank[t % 4, 0], bank[t % 4, 1])
    q = torch.randn((262, H, 64), generator=g, device="cuda").to(torch.bfloat16)
    assert fr.num_splits(262) == 16
    (ro, rl), (o, l), wsb = _both(fr, q)
    assert 0 < wsb <= L.NOALLOC_SCRATCH_BYTES
    _bar(o, l, ro, rl, "frame, same splits as kvc_attend")
    assert torch.equal(o, ro) and torch.equal(l, rl)


def test_noalloc_refuses_long_tables():
    import torch
    from paged_sliding_window_kv_amd import KvCache, lib
    from paged_sliding_window_kv_amd import _lib as L
    c = KvCache(num_heads=1, dtype="bf16", patch_tokens=256, special_tokens=6, num_scale_units=0, window_units=1,
                max_units=42 * 650, device="cuda")
    k = torch.zeros((262, 1, 64), dtype=torch.bfloat16, device="cuda")
    for _ in range(42 * 641):
        c.append(k, k)
    assert len(c.visible_table()[0]) > 640
    q = torch.zeros((262, 1, 64), dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((262, 1), dtype=torch.float32, device="cuda")
    s = lib().kvc_attend_noalloc(c.handle, q.data_ptr(), 262, 0.0, o.data_ptr(), lse.data_ptr(),
                                 torch.cuda.current_stream().cuda_stream)
    assert s == L.KVC_ERR_UNSUPPORTED
    assert b"640" in lib().kvc_last_error()
