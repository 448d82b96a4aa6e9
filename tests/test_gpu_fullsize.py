"""Parity at the full workload sizes, in the launch configurations bench.py times.

Outputs the oracle can afford are compared whole: the last frame of the
1000-frame LingBot-shaped stream, with 24,432 keys.  Larger ones are compared
on sampled query rows: the chunked step (10,992 queries x 43,968 keys) and
global attention over 137,400 tokens.  Inputs cycle through a small bank of
seeded frames (values do not change the launch configuration); the oracle
appends exactly the same bits.
"""
import numpy as np
import pytest

import synth
from gpu_helpers import check_attention, log, to_dev, to_f64
from oracle import OracleCache, OracleConfig, attention_f64, is_keyframe
from oracle import to_f64 as bits_f64

pytestmark = pytest.mark.gpu


def _bank(seed, n, tokens, heads, dtype="bf16"):
    return [synth.frame_qkv(seed, 0, i, tokens, heads, 64, dtype) for i in range(n)]


def test_lingbot_stream_1000_frames_last_step():
    import torch
    from paged_sliding_window_kv_amd import KvCache
    H, P, X, S, W, frames = 16, 256, 6, 8, 64, 1000
    log("lingbot stream 1000 frames (bench launch configuration)")
    bank = _bank(11, 6, P + X, H)
    dc = KvCache(num_heads=H, dtype="bf16", patch_tokens=P, special_tokens=X, num_scale_units=S, window_units=W,
                 max_units=frames, device="cuda")
    oc = OracleCache(OracleConfig(num_heads=H, head_dim=64, patch_tokens=P, special_tokens=X, num_scale_units=S,
                                  window_units=W, max_units=frames, store_dtype="bf16"))
    dev_bank = [(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")) for q, k, v in bank]
    before = torch.cuda.memory_allocated()
    for t in range(frames):
        q, k, v = bank[t % len(bank)]
        dq, dk, dv = dev_bank[t % len(bank)]
        oc.append(k, v)
        dc.append(dk, dv)
        if t in (0, 71, 72, 500):
            o, lse = dc.attend(dq)
            gk, gv = oc.gather()
            ro, rl = attention_f64(bits_f64(q), bits_f64(gk), bits_f64(gv))
            check_attention(o, lse, ro, rl, "bf16", f"t={t} Lk={gk.shape[1]}")
            del o, lse
    torch.cuda.synchronize()
    # constant device memory over the stream: no allocation after create
    assert torch.cuda.memory_allocated() == before
    q = bank[(frames - 1) % len(bank)][0]
    o, lse = dc.attend(dev_bank[(frames - 1) % len(bank)][0])
    gk, gv = oc.gather()
    assert gk.shape[1] == 24432
    ro, rl = attention_f64(bits_f64(q), bits_f64(gk), bits_f64(gv))
    check_attention(o, lse, ro, rl, "bf16", "t=999 Lk=24432")
    ids, lens = dc.visible_table()
    oids, olens = oc.visible_table()
    assert ids.tolist() == oids and lens.tolist() == olens


def test_keyframe_stream_10000_frames_fp32():
    import torch
    from paged_sliding_window_kv_amd import KvCache
    H, P, X, S, W, N, frames = 4, 256, 6, 2, 4, 4, 10000
    log("keyframe stream 10,000 frames fp32 (N=4)")
    bank = _bank(12, 5, P + X, H, "f32")
    dc = KvCache(num_heads=H, dtype="f32", patch_tokens=P, special_tokens=X, num_scale_units=S, window_units=W,
                 max_units=frames, device="cuda")
    oc = OracleCache(OracleConfig(num_heads=H, head_dim=64, patch_tokens=P, special_tokens=X, num_scale_units=S,
                                  window_units=W, max_units=frames, store_dtype="f32"))
    dev_bank = [(to_dev(q, "f32"), to_dev(k, "f32"), to_dev(v, "f32")) for q, k, v in bank]
    o = torch.empty((P + X, H, 64), dtype=torch.float32, device="cuda")
    lse = torch.empty((P + X, H), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(dc.workspace_bytes(P + X), 256), dtype=torch.uint8, device="cuda")
    before = torch.cuda.memory_allocated()
    patch_pages = []
    for t in range(frames):
        q, k, v = bank[t % len(bank)]
        dq, dk, dv = dev_bank[t % len(bank)]
        oc.append(k, v)
        dc.append(dk, dv)
        dc.attend(dq, o, lse, workspace=ws)
        if t % 1999 == 0 or t == frames - 1:
            gk, gv = oc.gather()
            ro, rl = attention_f64(bits_f64(q), bits_f64(gk), bits_f64(gv))
            check_attention(o, lse, ro, rl, "f32", f"t={t} Lk={gk.shape[1]}")
        if not is_keyframe(t, S, N):
            oc.rollback()
            dc.rollback()
        st = dc.state()
        patch_pages.append(len(st["scale_pages"]) + len(st["window_pages"]))
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    st = dc.state()
    assert st == oc.state()
    assert st["num_units"] == 2502 and len(st["special_pages"]) == 60
    assert set(patch_pages[20:]) == {6}          # constant patch-page count after warm-up
    assert dc.visible_table()[1][-1] == 144


def _sampled_rows(o, lse, q_rows, rows, k_all, v_all, what):
    """Compare sampled query rows of a large call with the oracle, computed for those rows only."""
    ro, rl = attention_f64(bits_f64(q_rows), k_all, v_all)
    check_attention(o[rows], lse[rows], ro, rl, "bf16", what)


def test_chunked_full_size_sampled_rows():
    import torch
    from paged_sliding_window_kv_amd import KvCache
    H, tokens, W, chunks = 16, 8 * 1374, 4, 5
    log("chunked: 10,992-token chunks, window 4 (43,968 keys), sampled rows")
    dc = KvCache(num_heads=H, dtype="bf16", patch_tokens=tokens, special_tokens=0, num_scale_units=0,
                 window_units=W, max_units=chunks, device="cuda")
    oc = OracleCache(OracleConfig(num_heads=H, head_dim=64, patch_tokens=tokens, special_tokens=0,
                                  num_scale_units=0, window_units=W, max_units=chunks, store_dtype="bf16"))
    for c in range(chunks):
        q, k, v = synth.frame_qkv(13, 0, c, tokens, H, 64, "bf16")
        oc.append(k, v)
        dc.append(to_dev(k, "bf16"), to_dev(v, "bf16"))
    o, lse = dc.attend(to_dev(q, "bf16"))
    torch.cuda.synchronize()
    gk, gv = oc.gather()
    assert gk.shape[1] == 43968
    rng = np.random.default_rng(3)
    rows = np.sort(np.concatenate([rng.choice(tokens, 60, replace=False), [0, 255, 256, 271, 272, 287, 288, 511, 512, 543, 544, tokens - 1]]))
    rows = np.unique(rows)
    _sampled_rows(o, lse, q[rows], torch.from_numpy(rows).cuda(), bits_f64(gk), bits_f64(gv), "chunk rows")


def test_global_and_frame_attention_full_size_sampled_rows():
    import torch
    from paged_sliding_window_kv_amd import KvCache, paged_attention
    H, F, T = 16, 100, 1374
    log("global: 100 frames x 1374 tokens = 137,400 keys, sampled rows; per-frame attention")
    dc = KvCache(num_heads=H, dtype="bf16", patch_tokens=T, special_tokens=0, num_scale_units=0, window_units=0,
                 max_units=F, device="cuda")
    qs, ks, vs = [], [], []
    for f in range(F):
        q, k, v = synth.frame_qkv(14, 0, f % 7, T, H, 64, "bf16")
        qs.append(q)
        ks.append(k)
        vs.append(v)
        dc.append(to_dev(k, "bf16"), to_dev(v, "bf16"))
    qall = np.concatenate(qs)
    dq = to_dev(qall, "bf16")
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    o, lse = dc.attend(dq)
    torch.cuda.synchronize()
    # no score matrix is materialised ("vLLM-Omni RFC #2727", section 2.3: at 100
    # frames one head's scores alone take about 35 GB): the call allocates its
    # outputs (O 281 MB, lse 8.8 MB) and nothing of the scores' size
    grown = torch.cuda.max_memory_allocated() - base
    scores_one_head = (F * T) ** 2 * 2
    log(f"  attention call peak allocation {grown / 2**20:.1f} MiB (one head's bf16 scores: {scores_one_head / 2**30:.1f} GiB)")
    assert grown < scores_one_head / 100
    k_all = bits_f64(np.concatenate(ks)).transpose(1, 0, 2)
    v_all = bits_f64(np.concatenate(vs)).transpose(1, 0, 2)
    rng = np.random.default_rng(4)
    rows = np.unique(np.concatenate([rng.choice(F * T, 40, replace=False), [0, 255, 256, 271, 272, 287, 288, 511, 512, 543, 544, F * T - 1]]))
    _sampled_rows(o, lse, qall[rows], torch.from_numpy(rows).cuda(), k_all, v_all, "global rows")
    # per-frame attention: 100 sequences, each against its own 6 pages (last one 94 tokens)
    ids, lens = dc.visible_table()
    upp = 6
    qo = torch.arange(0, F * T + 1, T, dtype=torch.int32, device="cuda")
    kv = torch.arange(0, F * upp + 1, upp, dtype=torch.int32, device="cuda")
    of, lf = paged_attention(dq, dc.k_pool, dc.v_pool, torch.from_numpy(ids).cuda(), torch.from_numpy(lens).cuda(),
                             qo, kv, T, upp)
    torch.cuda.synchronize()
    for f in (0, 37, 99):
        sel = np.unique(np.concatenate([rng.choice(T, 24, replace=False), [0, T - 1]]))
        kf = bits_f64(ks[f]).transpose(1, 0, 2)
        vf = bits_f64(vs[f]).transpose(1, 0, 2)
        rows_f = torch.from_numpy(f * T + sel).cuda()
        _sampled_rows(of, lf, qs[f][sel], rows_f, kf, vf, f"frame {f} rows")
