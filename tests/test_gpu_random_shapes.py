"""Seeded random shapes against the fp64 oracle.

Each case draws a batch of sequences whose query counts straddle every tile
shape the library chooses (bf16: 32-row blocks up to 256 queries, the 272-row
tile, 256-row pipelined tiles, 512-row tiles above 1024 queries; fp32: 64-row
tiles of two 32-row blocks), ragged page
tables (lengths 1..P, empty sequences) with NaN-poisoned stale slots, 1 to 3
heads, and forced or automatic key splits.  Page ids are distinct across the
batch; the oracle gathers each sequence's keys from the same pool bits and
computes fp64 attention.
"""
import numpy as np
import pytest

import synth
from gpu_helpers import check_attention, log, to_dev, to_f64, v_pool_device_layout, v_positions
from oracle import attention_f64
from oracle import to_f64 as bits_f64

pytestmark = pytest.mark.gpu

# query counts around each tile-shape boundary
_QN = [1, 31, 32, 200, 256, 257, 262, 272, 273, 300, 511, 512, 513, 1024, 1025, 1300, 1537]


@pytest.mark.parametrize("dtype,case", [("bf16", c) for c in range(8)] + [("f32", c) for c in range(4)])
def test_random_batches_against_oracle(dtype, case):
    import torch
    from paged_sliding_window_kv_amd import paged_attention
    rng = np.random.default_rng((9000 if dtype == "bf16" else 9100) + case)
    H = int(rng.integers(1, 4))
    P, N = 256, 48
    nseq = int(rng.integers(1, 4))
    qlens = [int(rng.choice(_QN)) for _ in range(nseq)]
    counts = [int(rng.integers(0, 6)) for _ in range(nseq)]
    if sum(counts) == 0:
        counts[0] = 1
    ids = rng.choice(N, size=sum(counts), replace=False).astype(np.int32)
    lens = rng.integers(1, P + 1, size=sum(counts)).astype(np.int32)
    full = rng.random(sum(counts)) < 0.5
    lens[full] = P  # half the pages full, as in a stream
    kv = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    qo = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    splits = int(rng.choice([0, 0, 1, 2, 3, 7]))
    log(f"{dtype} case {case}: H={H} qlens={qlens} pages={counts} splits={splits}")
    kpool = synth.normal_tokens(11, case, 0, 1, N * H * P, 1, 64, dtype).reshape(N, H, P, 64)
    vpool = synth.normal_tokens(11, case, 0, 2, N * H * P, 1, 64, dtype).reshape(N, H, P, 64)
    q = synth.normal_tokens(11, case, 0, 0, int(qo[-1]), H, 64, dtype)
    kd = to_dev(kpool, dtype)
    vd = to_dev(v_pool_device_layout(vpool), dtype)
    pos = torch.from_numpy(v_positions(P)).cuda()
    for p_, n in zip(ids, lens):
        kd[p_, :, n:] = float("nan")
        vd[p_][:, :, pos[n:]] = float("nan")
    dev = lambda a: torch.from_numpy(a).cuda()
    o, lse = paged_attention(to_dev(q, dtype), kd, vd, dev(ids), dev(lens), dev(qo), dev(kv),
                             max_qo_len=max(qlens), max_kv_pages=max(counts), num_splits=splits)
    for s_ in range(nseq):
        a, b = qo[s_], qo[s_ + 1]
        sel = list(zip(ids[kv[s_]:kv[s_ + 1]], lens[kv[s_]:kv[s_ + 1]]))
        if sel:
            gk = np.concatenate([kpool[p_, :, :n] for p_, n in sel], axis=1)
            gv = np.concatenate([vpool[p_, :, :n] for p_, n in sel], axis=1)
        else:
            gk = gv = np.zeros((H, 0, 64), kpool.dtype)
        ro, rl = attention_f64(bits_f64(q[a:b]), bits_f64(gk), bits_f64(gv))
        check_attention(o[a:b], lse[a:b], ro, rl, dtype, f"{dtype} case {case} seq={s_} q={b - a} Lk={gk.shape[1]}")
        if not sel:
            assert (to_f64(o[a:b]) == 0).all()


@pytest.mark.parametrize("case", range(6))
def test_random_fp8_batches_against_oracle(case):
    """The same random batches over FP8 pages: E4M3 codes and per-(token, head) row
    exponents from the oracle's quantiser ("vLLM-Omni RFC #2727", section 3.4), stale
    slots past each page's length holding NaN codes (0xFF) with exponent 127.  The
    oracle attends in fp64 over the dequantised keys and values."""
    import torch
    from oracle import dequantize_rows, quantize_rows
    from paged_sliding_window_kv_amd import paged_attention
    rng = np.random.default_rng(9200 + case)
    H = int(rng.integers(1, 4))
    P, N = 256, 48
    nseq = int(rng.integers(1, 4))
    qlens = [int(rng.choice(_QN)) for _ in range(nseq)]
    counts = [int(rng.integers(0, 6)) for _ in range(nseq)]
    if sum(counts) == 0:
        counts[0] = 1
    ids = rng.choice(N, size=sum(counts), replace=False).astype(np.int32)
    lens = rng.integers(1, P + 1, size=sum(counts)).astype(np.int32)
    lens[rng.random(sum(counts)) < 0.5] = P
    kv = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    qo = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    splits = int(rng.choice([0, 0, 1, 2, 3, 7]))
    log(f"fp8 case {case}: H={H} qlens={qlens} pages={counts} splits={splits}")
    kc, ke = quantize_rows(bits_f64(synth.normal_tokens(12, case, 0, 1, N * H * P, 1, 64, "bf16")).reshape(N, H, P, 64))
    vc, ve = quantize_rows(bits_f64(synth.normal_tokens(12, case, 0, 2, N * H * P, 1, 64, "bf16")).reshape(N, H, P, 64))
    for p_, n in zip(ids, lens):
        kc[p_, :, n:] = 0xFF
        vc[p_, :, n:] = 0xFF
        ke[p_, :, n:] = 127
        ve[p_, :, n:] = 127
    # flat pool buffers: codes [N][H][P][d], then exponents [N][H][P]
    kbuf = torch.from_numpy(np.concatenate([kc.reshape(-1), ke.view(np.uint8).reshape(-1)])).cuda()
    vbuf = torch.from_numpy(np.concatenate([vc.reshape(-1), ve.view(np.uint8).reshape(-1)])).cuda()
    q = synth.normal_tokens(12, case, 0, 0, int(qo[-1]), H, 64, "bf16")
    dev = lambda a: torch.from_numpy(a).cuda()
    o, lse = paged_attention(to_dev(q, "bf16"), kbuf, vbuf, dev(ids), dev(lens), dev(qo), dev(kv),
                             max_qo_len=max(qlens), max_kv_pages=max(counts), num_splits=splits, fp8_pages=(N, P))
    for s_ in range(nseq):
        a, b = qo[s_], qo[s_ + 1]
        sel = list(zip(ids[kv[s_]:kv[s_ + 1]], lens[kv[s_]:kv[s_ + 1]]))
        if sel:
            gk = np.concatenate([dequantize_rows(kc[p_, :, :n], ke[p_, :, :n]) for p_, n in sel], axis=1)
            gv = np.concatenate([dequantize_rows(vc[p_, :, :n], ve[p_, :, :n]) for p_, n in sel], axis=1)
        else:
            gk = gv = np.zeros((H, 0, 64))
        ro, rl = attention_f64(bits_f64(q[a:b]), gk, gv)
        check_attention(o[a:b], lse[a:b], ro, rl, "bf16", f"fp8 case {case} seq={s_} q={b - a} Lk={gk.shape[1]}")
        if not sel:
            assert (to_f64(o[a:b]) == 0).all()
