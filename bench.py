#!/usr/bin/env python3
"""Throughput of paged sliding-window KV attention on one MI355X.

Default workload (one JSON line on stdout): VGGT-style chunked global
attention ("vLLM-Omni RFC #2727: Reconstruction Engine", sections 1, 2.2 and
2.3).  24 layer caches, 16 heads x 64 dims, bf16; a unit is a chunk of 8
frames x 1374 tokens = 10,992 query tokens (43 pages of 256), and the window
keeps the last 4 chunks including the current one, so every timed chunk
attends to 43,968 keys.  One step is one chunk through all 24 layers: the
append (scatter of the chunk's K/V into pages) and the attention of its
10,992 queries against the visible table.  `--steps K` times K such steps
after at least 4 untimed ones (the window full); it never changes the
shapes.  Inputs are seeded synthetic N(0,1) tensors, resident in HBM before
timing.

The line also carries, at full size, the LingBot-Map-shaped stream
("LingBot-Map Paged KV Cache", sections 1-2): 24 layer caches, 1,000 frames
of 256 patch + 6 special tokens, 8 scale frames, a 64-frame window, special
pages of 42 frames, each frame's 262 queries attending after its append.

Other workloads (--workload): "stream" (the LingBot stream as the main line;
--steps K times the last K of its 1,000 frames), "global" (full global
attention over 100 frames x 1374 tokens, then per-frame attention),
"stream_batched" (--batch LingBot streams, one attention launch per layer and
frame), "keyframe" (a small fp32 stream over 10,000 frames that keeps every
fourth frame and rolls the others back), "windowed" (the LingBot stream in
windowed mode, section 4: 25,000 frames, a keyframe every second frame, the
24 caches restarted once per window of 128 kept units with the last 16
shared).

Every workload reports `roofline` for its dominant kernel (algorithmic FLOPs
or bytes per launch over the kernel's own duration, taken with HIP events on
the launch stream: the library records events right before and right after
the attention kernel, before the merge of split partials) and `cpu_baseline` (the
oracle timed on the host on a bounded slice of the same workload).
"""
from __future__ import annotations

import argparse
import ctypes as C
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged attention TFLOP/s + streamed frames/s (% of bf16 MFMA peak), 1 MI355X"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix cores (published)
PEAK_F32_TFLOPS = 157.3     # MI355X dense fp32 matrix cores (published)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E (published)

VGGT_TOKENS = 1374
CHUNK = dict(layers=24, heads=16, d=64, page=256, frames_per_chunk=8, window_chunks=4)
STREAM = dict(layers=24, heads=16, d=64, page=256, patch=256, special=6, scale=8, window=64, frames=1000)
KEYFRAME = dict(heads=4, d=64, page=256, patch=256, special=6, scale=2, window=4, interval=4, frames=10000)
WINDOWED = dict(layers=24, heads=16, d=64, page=256, patch=256, special=6, scale=8, window=64, slots=128, overlap=16,
                interval=2, frames=25000)
GLOBAL = dict(layers=24, heads=16, d=64, frames=100)


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def _ok(status: int, where: str) -> None:
    if status != 0:
        from paged_sliding_window_kv_amd import _lib as L
        L.check(status, where)


def attn_flops(lq: int, lk: int, heads: int, d: int = 64) -> float:
    """QK^T and PV: 2 * 2 * Lq * Lk * d per head (softmax not counted)."""
    return 4.0 * lq * lk * d * heads


def attn_bytes(lq: int, lk: int, heads: int, d: int = 64, elem: int = 2, kv_elem: float = 2.0) -> float:
    """Bytes an attention call must move: K and V of the visible tokens, Q in, O out, LSE out.

    kv_elem: bytes per K/V value (2 for bf16 pages, 1 + 1/d for FP8 codes with a row exponent)."""
    return 2.0 * lk * heads * d * kv_elem + 2.0 * lq * heads * d * elem + lq * heads * 4.0


def kv_label(kv_dtype: str) -> str:
    return "bf16" if kv_dtype == "bf16" else "bf16 activations, FP8 (E4M3) KV pages with per-token exponents"


def kv_elem_bytes(kv_dtype: str, d: int = 64) -> float:
    return 2.0 if kv_dtype == "bf16" else 1.0 + 1.0 / d


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def host_info() -> dict:
    """Host cores, CPU model and the BLAS numpy runs on (the oracle's matrix products)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = "unknown"
    try:
        b = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        blas = f"{b.get('name')} {b.get('version')}"
    except Exception:
        pass
    return {"cores": len(os.sched_getaffinity(0)), "blas_threads": blas_threads(), "cpu_model": model,
            "blas": blas, "numpy": np.__version__}


def cpu_baseline(value: float, unit: str, sample: str, sec: float, extra: dict | None = None) -> dict:
    h = host_info()
    out = {"value": value, "unit": unit, "cores": h["blas_threads"], "kind": "oracle", "sample": sample,
           "seconds": sec, "host_cores": h["cores"], "cpu_model": h["cpu_model"], "blas": h["blas"],
           "numpy": h["numpy"]}
    if extra:
        out.update(extra)
    return out


class CallClock:
    """HIP events around attention calls on the launch stream.

    For call i: `before(i)` records a call-start event and hands the library
    a kernel-start and a kernel-done event, which it records right before and
    right after the attention kernel (after its host-side table work, before
    the merge of split partials); `after(i)` records a call-end event.
    kernel-start -> kernel-done is the attention kernel alone; kernel-start ->
    call-end is the kernel plus the merge of its split partials.  The call's
    host-side table work before the launch is left out: while the host is
    slower than the GPU (a 40 us kernel against four event records and a
    ctypes call per layer), it would time the host, not the device.
    """

    def __init__(self, n: int):
        import torch
        from paged_sliding_window_kv_amd import lib
        self.torch, self.lib = torch, lib()
        self.ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n)]
        for trio in self.ev:  # torch creates the HIP events at their first record
            for e in trio:
                e.record()
        torch.cuda.synchronize()
        self.kernel_s = 0.0
        self.call_s = 0.0
        self.calls = 0
        self.kernel_each = []  # seconds, one per call

    def before(self, i: int) -> None:
        self.ev[i][0].record()
        _ok(self.lib.kvc_set_kernel_events(C.c_void_p(self.ev[i][1].cuda_event), C.c_void_p(self.ev[i][2].cuda_event)),
            "kvc_set_kernel_events")

    def after(self, i: int) -> None:
        self.ev[i][3].record()
        _ok(self.lib.kvc_set_kernel_events(None, None), "kvc_set_kernel_events")

    def collect(self, n: int) -> None:
        """Adds calls 0..n-1 (after a synchronize) to the totals."""
        self.torch.cuda.synchronize()
        for i in range(n):
            _, k0, k1, e = self.ev[i]
            k = k0.elapsed_time(k1) * 1e-3
            self.kernel_s += k
            self.kernel_each.append(k)
            self.call_s += k0.elapsed_time(e) * 1e-3
        self.calls += n

    def median_kernel_us(self) -> float:
        return float(np.median(self.kernel_each)) * 1e6 if self.kernel_each else float("nan")


def run_probes() -> dict:
    """Measured denominators (include/kvc_probe.h): dense bf16 matrix-core rate, the 512-row attention kernel's
    per-tile instruction mix on its own (products and softmax from registers and LDS, no global memory or table
    walk), and HBM read/copy bandwidth."""
    import torch
    from paged_sliding_window_kv_amd import lib
    lb = lib()
    dev = torch.device("cuda:0")
    sp = torch.cuda.current_stream(dev).cuda_stream
    scratch = torch.empty(lb.kvc_probe_scratch_bytes(), dtype=torch.uint8, device=dev)
    tf = C.c_double()
    _ok(lb.kvc_probe_mfma_bf16(scratch.data_ptr(), scratch.numel(), sp, C.byref(tf)), "kvc_probe_mfma_bf16")
    mix = C.c_double()
    _ok(lb.kvc_probe_tile_mix(scratch.data_ptr(), scratch.numel(), sp, C.byref(mix)), "kvc_probe_tile_mix")
    nb = 2 << 30
    src = torch.ones(nb, dtype=torch.uint8, device=dev)
    dst = torch.empty(nb, dtype=torch.uint8, device=dev)
    rd, cp = C.c_double(), C.c_double()
    _ok(lb.kvc_probe_hbm(src.data_ptr(), dst.data_ptr(), nb, scratch.data_ptr(), scratch.numel(), sp, C.byref(rd),
                         C.byref(cp)), "kvc_probe_hbm")
    del src, dst, scratch
    torch.cuda.empty_cache()
    out = {"mfma_bf16_tflops": tf.value, "tile_mix_tflops": mix.value, "hbm_read_gbs": rd.value,
           "hbm_copy_gbs": cp.value,
           "mfma_probe": "one 16-wave workgroup per compute unit, 4 chains of v_mfma_f32_32x32x16_bf16 per wave, "
                         "from registers",
           "tile_mix_probe": "attn_wide_kernel's per-tile work without global memory, table walk, masks or rare-path "
                             "checks: 8 waves per compute unit, per wave and 64-key tile one barrier, 16 LDS fragment "
                             "reads, 32 products and two 32-row blocks' softmax in fenced groups",
           "hbm_probe": "2 GiB streaming read (16-byte loads) and 2 GiB copy (read + write bytes)"}
    log(f"[bench] probes: bf16 matrix cores {tf.value:.0f} TFLOP/s, attention tile mix {mix.value:.0f} TFLOP/s, "
        f"HBM read {rd.value:.0f} GB/s, copy {cp.value:.0f} GB/s")
    return out


# ----------------------------------------------------------------------------
# VGGT-style chunked global attention (the default line)
# ----------------------------------------------------------------------------
def chunk_tokens() -> int:
    return CHUNK["frames_per_chunk"] * VGGT_TOKENS


def oracle_chunked_sample(query_rows: int = 1024, seed: int = 0):
    """The oracle on a bounded slice of the chunked workload: one layer, all 16 heads.

    Four chunks fill the window untimed.  Timed: the append of the fifth chunk
    (the oldest is evicted), the gather of the 43,968 visible keys and the fp64
    attention of that chunk's first `query_rows` queries.  Returns (seconds,
    flops of the attention part, visible keys).
    """
    import synth
    from oracle import OracleCache, OracleConfig, attention_f64, to_f64
    c, T, W = CHUNK, chunk_tokens(), CHUNK["window_chunks"]
    oc = OracleCache(OracleConfig(num_heads=c["heads"], head_dim=c["d"], page_size=c["page"], patch_tokens=T,
                                  special_tokens=0, num_scale_units=0, window_units=W, max_units=W + 1,
                                  store_dtype="bf16"))
    bank = [synth.frame_qkv(seed, 0, i, T, c["heads"], c["d"], "bf16") for i in range(2)]
    for i in range(W):
        oc.append(bank[i % 2][1], bank[i % 2][2])
    q, k, v = bank[W % 2]
    t0 = time.perf_counter()
    oc.append(k, v)
    gk, gv = oc.gather()
    attention_f64(to_f64(q[:query_rows]), to_f64(gk), to_f64(gv))
    sec = time.perf_counter() - t0
    return sec, attn_flops(query_rows, gk.shape[1], c["heads"], c["d"]), gk.shape[1]


def run_chunked(args) -> dict:
    """Chunks of 8 frames (10,992 tokens, 43 pages) attend to the last 4 chunks (43,968 keys)."""
    import torch
    from paged_sliding_window_kv_amd import KvCache, lib
    c = CHUNK
    L, H, W, T = c["layers"], c["heads"], c["window_chunks"], chunk_tokens()
    steps, warm = args.steps, max(args.warmup, W)
    log(f"[bench] chunked: {L} layers, chunk {T} tokens, window {W} chunks, {warm} untimed and {steps} timed "
        f"chunk steps, KV {args.kv_dtype}")
    dev = torch.device("cuda:0")
    lb = lib()
    caches = [KvCache(num_heads=H, dtype=args.kv_dtype, patch_tokens=T, special_tokens=0, num_scale_units=0,
                      window_units=W, max_units=warm + steps, device=dev) for _ in range(L)]
    g = torch.Generator(device=dev)
    g.manual_seed(1)
    bank = 2
    shp = (bank, T, H, c["d"])
    qs = [torch.randn(shp, generator=g, device=dev).to(torch.bfloat16) for _ in range(L)]
    ks = [torch.randn(shp, generator=g, device=dev).to(torch.bfloat16) for _ in range(L)]
    vs = [torch.randn(shp, generator=g, device=dev).to(torch.bfloat16) for _ in range(L)]
    out = torch.empty((T, H, c["d"]), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    wsb = max(cc.workspace_bytes(T) for cc in caches)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)
    sp = torch.cuda.current_stream(dev).cuda_stream
    kr = args.keep_ratio
    # events around every attention kernel of the timed steps (a 2 ms kernel:
    # the markers cost 0.1-0.4%), read after the timed region
    clock = CallClock(L * steps)

    def step(i, ci=None):
        """Chunk step i; ci: first clock slot of its 24 attention calls (None: no events)."""
        b = i % bank
        for l in range(L):
            _ok(lb.kvc_append_frame(caches[l].handle, ks[l][b].data_ptr(), vs[l][b].data_ptr(), sp), "append")
            if ci is not None:
                clock.before(ci + l)
            if kr < 1.0:
                # AVGGT-style: each layer its own random page subset (seed = layer)
                _ok(lb.kvc_attend_subset(caches[l].handle, kr, l, 0, 0, qs[l][b].data_ptr(), T, 0.0,
                                         out.data_ptr(), lse.data_ptr(), ws.data_ptr(), wsb, sp), "attend_subset")
            else:
                _ok(lb.kvc_attend(caches[l].handle, qs[l][b].data_ptr(), T, 0.0, out.data_ptr(),
                                  lse.data_ptr(), ws.data_ptr(), wsb, sp), "attend")
            if ci is not None:
                clock.after(ci + l)

    for i in range(warm):
        step(i)
    # one event at each step boundary as well (a 50 ms step: negligible), for the median step
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        marks[i].record()
        step(warm + i, i * L)
    marks[steps].record()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    clock.collect(L * steps)
    step_ms = [marks[i].elapsed_time(marks[i + 1]) for i in range(steps)]
    lk = W * T
    if kr < 1.0:
        # keys each layer attends: the subset keeps the same table positions every steady-state step
        lks = [int(caches[l].subset_table(kr, l)[1].sum()) for l in range(L)]
    else:
        lks = [lk] * L
    flops_step = sum(attn_flops(T, x, H) for x in lks)
    kv_e = kv_elem_bytes(args.kv_dtype)
    bytes_call = sum(attn_bytes(T, x, H, kv_elem=kv_e) for x in lks) / L
    n = clock.calls
    flops_call = flops_step / L
    k_us = clock.kernel_s / n * 1e6
    c_us = clock.call_s / n * 1e6
    ach = flops_call / (k_us * 1e-6) / 1e12
    tf = steps * flops_step / el / 1e12
    splits = caches[0].num_splits(T) if kr >= 1.0 else None
    log(f"[bench] chunked: {el / steps * 1e3:.2f} ms/step, {tf:.1f} TFLOP/s, {steps * 8 / el:.1f} frames/s; "
        f"attention kernel {k_us:.1f} us ({ach:.1f} TFLOP/s, {ach / PEAK_BF16_TFLOPS:.1%} of bf16 peak), "
        f"call with merge {c_us:.1f} us")
    kernel = ("attn_wide_kernel" if args.kv_dtype == "bf16" else "attn_wide_kernel<FP8 pages>")
    res = {
        "value": tf, "unit": "TFLOP/s", "ms_per_step": el / steps * 1e3,
        "frames_per_s": steps * c["frames_per_chunk"] / el,
        "pct_bf16_mfma_peak": 100.0 * tf / PEAK_BF16_TFLOPS,
        "dtype": "bf16",
        "config": {"workload": f"vggt_chunked: 24 layer caches, 16 heads x 64, {kv_label(args.kv_dtype)}, "
                               f"chunks of 8 x 1374 = {T} query tokens (43 pages), window 4 chunks "
                               f"({W * T} visible keys)"
                               + (f", per-layer page subsets keeping {kr} ({sum(lks) / L:.0f} keys attended)"
                                  if kr < 1.0 else "")
                               + f"; step = one chunk through 24 layers (append + attention); {steps} timed steps "
                               f"after {warm} untimed",
                   "layers": L, "heads": H, "head_dim": 64, "chunk_tokens": T, "window_chunks": W,
                   "visible_tokens": W * T, "keep_ratio": kr, "attended_tokens": sum(lks) / L,
                   "kv_dtype": args.kv_dtype, "untimed_chunk_steps": warm, "key_splits": splits},
        "roofline": {"bound": "mfma", "achieved": ach, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": ach / PEAK_BF16_TFLOPS, "traffic": None,
                     "kernel": kernel, "per_launch_flops": flops_call, "per_launch_bytes": bytes_call,
                     "avg_kernel_us": k_us, "median_kernel_us": clock.median_kernel_us(),
                     "avg_call_us_with_merge": c_us, "calls": n,
                     "call_tflops_with_merge": flops_call / (c_us * 1e-6) / 1e12},
        "step_ms": {"median": float(np.median(step_ms)), "min": min(step_ms), "max": max(step_ms), "steps": steps,
                    "source": "HIP events at the step boundaries of the timed region"},
    }
    if not args.no_cpu_baseline:
        rows = args.cpu_rows
        log(f"[bench] oracle: 1 layer, 16 heads, {rows} of the chunk's {T} queries against {W * T} keys")
        sec, fl, olk = oracle_chunked_sample(rows)
        rate = fl / sec / 1e12
        res["cpu_baseline"] = cpu_baseline(
            rate, "TFLOP/s",
            f"1 of 24 layers, all 16 heads, queries 0..{rows - 1} of a 10,992-query chunk against the {olk} "
            f"visible keys (append of the chunk, gather of the window's pages, fp64 attention), {sec:.1f} s; "
            f"extrapolated to a whole chunk step by the FLOP ratio",
            sec, {"extrapolated": True, "frames_per_s": c["frames_per_chunk"] / (flops_step / (rate * 1e12)),
                  "ms_per_step": flops_step / (rate * 1e12) * 1e3})
        log(f"[bench] oracle: {rate * 1e3:.2f} GFLOP/s over {sec:.1f} s")
    del caches, qs, ks, vs, out, lse, ws
    torch.cuda.empty_cache()
    return res


# ----------------------------------------------------------------------------
# LingBot-Map-shaped stream
# ----------------------------------------------------------------------------
def stream_lk(t: int, c=STREAM) -> int:
    """Visible tokens after appending frame t (0-based): scale + window patches + all specials."""
    n = t + 1
    units = min(n, c["scale"]) + min(max(n - c["scale"], 0), c["window"])
    return units * c["patch"] + n * c["special"]


def oracle_stream_sample(frames: int, sample: int, bank: int = 4, seed: int = 0):
    """The oracle on a bounded sample of the LingBot stream: one layer.

    Frames 0 .. frames - sample - 1 are appended untimed; the last `sample`
    frames are timed (append, gather and fp64 attention of the frame's 262
    queries).  The cache holds every frame's special tokens.  Returns
    (seconds, flops of the timed attention, frames timed).
    """
    import synth
    from oracle import OracleCache, OracleConfig, attention_f64, to_f64
    c = STREAM
    sample = max(1, min(sample, frames))
    tok = c["patch"] + c["special"]
    oc = OracleCache(OracleConfig(num_heads=c["heads"], head_dim=c["d"], page_size=c["page"], patch_tokens=c["patch"],
                                  special_tokens=c["special"], num_scale_units=c["scale"], window_units=c["window"],
                                  max_units=frames, store_dtype="bf16"))
    qkv = [synth.frame_qkv(seed, 0, i, tok, c["heads"], c["d"], "bf16") for i in range(bank)]
    for t in range(frames - sample):
        _, k, v = qkv[t % bank]
        oc.append(k, v)
    flops = 0.0
    t0 = time.perf_counter()
    for t in range(frames - sample, frames):
        q, k, v = qkv[t % bank]
        oc.append(k, v)
        gk, gv = oc.gather()
        attention_f64(to_f64(q), to_f64(gk), to_f64(gv))
        flops += attn_flops(tok, gk.shape[1], c["heads"], c["d"])
    return time.perf_counter() - t0, flops, sample


class StreamBench:
    def __init__(self, frames: int, layers: int, bank: int = 4, seed: int = 0, kv_dtype: str = "bf16"):
        import torch
        from paged_sliding_window_kv_amd import KvCache, lib
        c = STREAM
        self.c = c
        self.layers = layers
        self.frames = frames
        self.tokens = c["patch"] + c["special"]
        self.torch = torch
        self.lib = lib()
        dev = torch.device("cuda:0")
        self.dev = dev
        self.kv_elem = kv_elem_bytes(kv_dtype, c["d"])
        self.caches = [KvCache(num_heads=c["heads"], head_dim=c["d"], page_size=c["page"], dtype=kv_dtype,
                               patch_tokens=c["patch"], special_tokens=c["special"], num_scale_units=c["scale"],
                               window_units=c["window"], max_units=max(frames, 64), device=dev)
                       for _ in range(layers)]
        # input bank: `bank` distinct frames per layer, drawn N(0,1) from a seeded generator
        g = torch.Generator(device=dev)
        g.manual_seed(seed)
        shp = (bank, self.tokens, c["heads"], c["d"])
        self.q = [torch.randn(shp, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
                  for _ in range(layers)]
        self.k = [torch.randn(shp, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
                  for _ in range(layers)]
        self.v = [torch.randn(shp, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
                  for _ in range(layers)]
        self.bank = bank
        self.o = [torch.empty((self.tokens, c["heads"], c["d"]), dtype=torch.bfloat16, device=dev)
                  for _ in range(layers)]
        self.lse = [torch.empty((self.tokens, c["heads"]), dtype=torch.float32, device=dev) for _ in range(layers)]
        wsb = max(cc.workspace_bytes(self.tokens) for cc in self.caches)
        self.ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)
        self.wsb = wsb
        # raw pointers for the hot loop
        fb = self.tokens * c["heads"] * c["d"] * 2
        self.qp = [[self.q[l].data_ptr() + i * fb for i in range(bank)] for l in range(layers)]
        self.kp = [[self.k[l].data_ptr() + i * fb for i in range(bank)] for l in range(layers)]
        self.vp = [[self.v[l].data_ptr() + i * fb for i in range(bank)] for l in range(layers)]
        self.op = [x.data_ptr() for x in self.o]
        self.lp = [x.data_ptr() for x in self.lse]
        self.h = [cc.handle for cc in self.caches]
        self.stream = torch.cuda.current_stream(dev)
        self.sp = self.stream.cuda_stream

    def reset(self):
        for cc in self.caches:
            cc.reset()

    def step(self, t: int, clock: CallClock | None = None):
        """One frame: per layer, append the frame's K/V, then attend (the stream's own order)."""
        lib, sp, b = self.lib, self.sp, t % self.bank
        app, att = lib.kvc_append_frame, lib.kvc_attend
        wsp, wsb, nq = self.ws.data_ptr(), self.wsb, self.tokens
        for l in range(self.layers):
            s = app(self.h[l], self.kp[l][b], self.vp[l][b], sp)
            if s:
                _ok(s, "kvc_append_frame")
            if clock is not None:
                clock.before(l)
            s = att(self.h[l], self.qp[l][b], nq, 0.0, self.op[l], self.lp[l], wsp, wsb, sp)
            if s:
                _ok(s, "kvc_attend")
            if clock is not None:
                clock.after(l)
        if clock is not None:
            clock.collect(self.layers)

    def check_tables(self):
        ids, lens = self.caches[0].visible_table()
        return int(lens.sum()), len(ids)


def run_stream(args, timed: int | None = None, cpu_sample: int | None = None) -> dict:
    """The 1,000-frame LingBot stream; the last `timed` frames are timed (all of them by default)."""
    import torch
    c = STREAM
    frames, layers = c["frames"], c["layers"]
    timed = frames if timed is None else max(1, min(timed, frames))
    log(f"[bench] stream: {layers} layers x {frames} frames ({timed} timed), warmup {args.warmup}, "
        f"KV {args.kv_dtype}")
    b = StreamBench(frames, layers, kv_dtype=args.kv_dtype)
    for t in range(args.warmup):
        b.step(t)
    torch.cuda.synchronize()
    b.reset()
    mem0 = torch.cuda.memory_allocated(b.dev)  # pools, inputs, outputs, workspace
    for t in range(frames - timed):
        b.step(t)
        if (t + 1) % 250 == 0:
            log(f"[bench] stream: untimed frame {t + 1}")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for t in range(frames - timed, frames):
        b.step(t)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    mem_growth = torch.cuda.memory_allocated(b.dev) - mem0
    lk_sum, npages = b.check_tables()
    assert lk_sum == stream_lk(frames - 1), (lk_sum, stream_lk(frames - 1))
    heads = c["heads"]
    total_flops = sum(layers * attn_flops(b.tokens, stream_lk(t), heads) for t in range(frames - timed, frames))
    tflops = total_flops / elapsed / 1e12
    fps = timed / elapsed
    log(f"[bench] stream: timed {timed} frames in {elapsed:.3f} s: {tflops:.1f} TFLOP/s, {fps:.1f} frames/s")
    # replay the whole stream with events around every attention call
    b.reset()
    clock = CallClock(layers)
    byt = flo = 0.0
    for t in range(frames):
        b.step(t, clock)
        if (t + 1) % 250 == 0:
            log(f"[bench] stream: event replay frame {t + 1}")
        lk = stream_lk(t)
        byt += layers * attn_bytes(b.tokens, lk, heads, kv_elem=b.kv_elem)
        flo += layers * attn_flops(b.tokens, lk, heads)
    n = clock.calls
    k_us, c_us = clock.kernel_s / n * 1e6, clock.call_s / n * 1e6
    ach_gbs = byt / clock.kernel_s / 1e9
    log(f"[bench] stream attention: kernel {k_us:.2f} us avg ({ach_gbs:.0f} GB/s, "
        f"{flo / clock.kernel_s / 1e12:.1f} TFLOP/s), call with merge {c_us:.2f} us")
    res = {
        "value": tflops,
        "unit": "TFLOP/s",
        "ms_per_step": elapsed / timed * 1e3,
        "frames_per_s": fps,
        "pct_bf16_mfma_peak": 100.0 * tflops / PEAK_BF16_TFLOPS,
        "dtype": "bf16",
        "config": {
            "workload": f"lingbot_stream: 24 layer caches, 16 heads x 64, {kv_label(args.kv_dtype)}, "
                        "256 patch + 6 special tokens/frame, 8 scale frames, 64-frame window, 42 frames/special "
                        f"page, 262 queries/step, {frames} frames streamed, the last {timed} timed; step = one "
                        "frame through 24 layers (append + attention)",
            "layers": layers, "heads": heads, "head_dim": 64, "page_size": 256, "frames": frames,
            "timed_frames": timed, "final_visible_tokens": lk_sum, "final_visible_pages": npages,
            "kv_dtype": args.kv_dtype,
            "kv_pool_mib_per_layer": (b.caches[0].k_pool.numel() * b.caches[0].k_pool.element_size() * 2) / 2**20,
            "device_memory_growth_bytes": mem_growth,
        },
        "roofline": {
            "bound": "hbm", "achieved": ach_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": ach_gbs / PEAK_HBM_GBS, "traffic": None,
            "kernel": "attn_bf16_kernel (272-row tile)" if args.kv_dtype == "bf16" else "attn_bf16_kernel<FP8 pages>",
            "per_launch_bytes": byt / n, "per_launch_flops": flo / n,
            "avg_kernel_us": k_us, "median_kernel_us": clock.median_kernel_us(),
            "avg_call_us_with_merge": c_us, "calls": n,
            "kernel_tflops": flo / clock.kernel_s / 1e12,
            "call_gbs_with_merge": byt / clock.call_s / 1e9,
        },
    }
    sample = args.cpu_sample if cpu_sample is None else cpu_sample
    if not args.no_cpu_baseline and sample > 0:
        log(f"[bench] oracle sample: 1 layer, the last {sample} of {frames} frames")
        sec, fl, nfr = oracle_stream_sample(frames, sample)
        ot = fl / sec / 1e12
        res["cpu_baseline"] = cpu_baseline(
            ot, "TFLOP/s",
            f"1 of 24 layers, frames {frames - nfr}..{frames - 1} of the {frames}-frame stream "
            f"(append + gather + fp64 attention), {sec:.1f} s; frames/s scaled to 24 layers",
            sec, {"frames_per_s": 1.0 / (sec / nfr * layers)})
        log(f"[bench] oracle: {ot * 1e3:.2f} GFLOP/s over {sec:.1f} s")
    del b
    torch.cuda.empty_cache()
    return res


def run_stream_batched(args) -> dict:
    """B LingBot-shaped streams; per layer and frame, B appends then one batched attention launch."""
    import torch
    from paged_sliding_window_kv_amd import attend_batch_workspace_bytes, lib, shared_pool_caches
    c = STREAM
    B, L, frames = args.batch, c["layers"], c["frames"]
    timed = max(1, min(args.steps, frames))
    tok = c["patch"] + c["special"]
    log(f"[bench] stream_batched: {B} streams x {L} layers x {frames} frames ({timed} timed), warmup {args.warmup}")
    dev = torch.device("cuda:0")
    lb = lib()
    kw = dict(num_heads=c["heads"], head_dim=c["d"], page_size=c["page"], dtype="bf16", patch_tokens=c["patch"],
              special_tokens=c["special"], num_scale_units=c["scale"], window_units=c["window"],
              max_units=max(frames, args.warmup, 64))
    layers = [shared_pool_caches(B, dev, **kw) for _ in range(L)]
    g = torch.Generator(device=dev)
    g.manual_seed(3)
    bank = 4
    shp = (bank, B * tok, c["heads"], c["d"])
    qs = [torch.randn(shp, generator=g, device=dev).to(torch.bfloat16) for _ in range(L)]
    ks = [torch.randn(shp, generator=g, device=dev).to(torch.bfloat16) for _ in range(L)]
    vs = [torch.randn(shp, generator=g, device=dev).to(torch.bfloat16) for _ in range(L)]
    out = torch.empty((B * tok, c["heads"], c["d"]), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B * tok, c["heads"]), dtype=torch.float32, device=dev)
    qo = np.arange(0, B * tok + 1, tok, dtype=np.int32)
    qop = qo.ctypes.data_as(C.POINTER(C.c_int32))
    # largest workspace over the stream: the batch at its longest tables
    probe = shared_pool_caches(B, dev, **kw)
    for _ in range(frames):
        for cc in probe:
            cc.append(ks[0][0, :tok], vs[0][0, :tok])
    wsb = attend_batch_workspace_bytes(probe, qo)
    del probe
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)
    sp = torch.cuda.current_stream(dev).cuda_stream
    fb = tok * c["heads"] * c["d"] * 2
    handles = [(C.c_void_p * B)(*[cc.handle.value for cc in layer]) for layer in layers]
    hlist = [[cc.handle for cc in layer] for layer in layers]

    def step(t, clock=None):
        b = t % bank
        for l in range(L):
            kb, vb = ks[l].data_ptr() + b * B * fb, vs[l].data_ptr() + b * B * fb
            for i in range(B):
                _ok(lb.kvc_append_frame(hlist[l][i], kb + i * fb, vb + i * fb, sp), "append")
            if clock is not None:
                clock.before(l)
            _ok(lb.kvc_attend_batch(handles[l], B, qs[l].data_ptr() + b * B * fb, qop, 0.0, out.data_ptr(),
                                    lse.data_ptr(), ws.data_ptr(), wsb, sp), "attend_batch")
            if clock is not None:
                clock.after(l)
        if clock is not None:
            clock.collect(L)

    def reset():
        for layer in layers:
            for cc in layer:
                cc.reset()

    for t in range(args.warmup):
        step(t)
    torch.cuda.synchronize()
    reset()
    for t in range(frames - timed):
        step(t)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for t in range(frames - timed, frames):
        step(t)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    flops = sum(B * L * attn_flops(tok, stream_lk(t), c["heads"]) for t in range(frames - timed, frames))
    reset()
    clock = CallClock(L)
    byt = flo = 0.0
    for t in range(frames):
        step(t, clock)
        byt += B * L * attn_bytes(tok, stream_lk(t), c["heads"])
        flo += B * L * attn_flops(tok, stream_lk(t), c["heads"])
    n = clock.calls
    tf = flops / el / 1e12
    ach = byt / clock.kernel_s / 1e9
    log(f"[bench] stream_batched: {el / timed * 1e3:.2f} ms per frame step, {B * timed / el:.1f} frames/s over "
        f"{B} streams, {tf:.1f} TFLOP/s; batched kernel {clock.kernel_s / n * 1e6:.1f} us avg ({ach:.0f} GB/s), "
        f"call {clock.call_s / n * 1e6:.1f} us")
    res = {
        "value": tf, "unit": "TFLOP/s", "ms_per_step": el / timed * 1e3, "frames_per_s": B * timed / el,
        "pct_bf16_mfma_peak": 100.0 * tf / PEAK_BF16_TFLOPS, "dtype": "bf16",
        "config": {"workload": f"lingbot_stream_batched: {B} streams x 24 layer caches, 16 heads x 64, bf16, "
                               f"262 queries/stream/step, {frames} frames streamed, the last {timed} timed, one "
                               "attention launch per layer and frame",
                   "streams": B, "layers": L, "frames": frames, "timed_frames": timed},
        "roofline": {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": ach / PEAK_HBM_GBS,
                     "traffic": None, "kernel": "attn_bf16_kernel (batched)", "per_launch_bytes": byt / n,
                     "avg_kernel_us": clock.kernel_s / n * 1e6, "median_kernel_us": clock.median_kernel_us(),
                     "avg_call_us_with_merge": clock.call_s / n * 1e6,
                     "calls": n, "kernel_tflops": flo / clock.kernel_s / 1e12},
    }
    if not args.no_cpu_baseline and args.cpu_sample > 0:
        sec, fl, nfr = oracle_stream_sample(frames, args.cpu_sample)
        res["cpu_baseline"] = cpu_baseline(
            fl / sec / 1e12, "TFLOP/s",
            f"one stream, 1 of 24 layers, frames {frames - nfr}..{frames - 1} (append + gather + fp64 attention), "
            f"{sec:.1f} s; the batch's streams are independent, so the rate carries over", sec,
            {"frames_per_s": 1.0 / (sec / nfr * L)})
    return res


# ----------------------------------------------------------------------------
# Full global attention over 100 frames, then per-frame attention
# ----------------------------------------------------------------------------
def oracle_global_sample(query_rows: int = 256, seed: int = 0):
    """The oracle on a slice of the global workload: one layer, all 16 heads.

    100 frames of 1374 tokens are appended untimed (a bank of 2 distinct frames
    cycled; values do not change the cost).  Timed: the gather of all 137,400
    visible keys and the fp64 attention of `query_rows` queries against them,
    plus one frame's 1374 queries against its own 6 pages.  Returns (seconds,
    flops of the timed attention).
    """
    import synth
    from oracle import OracleCache, OracleConfig, attention_f64, to_f64
    H, F = GLOBAL["heads"], GLOBAL["frames"]
    oc = OracleCache(OracleConfig(num_heads=H, head_dim=64, page_size=256, patch_tokens=VGGT_TOKENS,
                                  special_tokens=0, num_scale_units=0, window_units=0, max_units=F,
                                  store_dtype="bf16"))
    bank = [synth.frame_qkv(seed, 0, i, VGGT_TOKENS, H, 64, "bf16") for i in range(2)]
    for f in range(F):
        oc.append(bank[f % 2][1], bank[f % 2][2])
    q = bank[0][0]
    t0 = time.perf_counter()
    gk, gv = oc.gather()
    attention_f64(to_f64(q[:query_rows]), to_f64(gk), to_f64(gv))
    ids, lens = oc.visible_table()
    fk, fv = oc.gather(ids[:6], lens[:6])
    attention_f64(to_f64(q), to_f64(fk), to_f64(fv))
    sec = time.perf_counter() - t0
    return sec, attn_flops(query_rows, gk.shape[1], H) + attn_flops(VGGT_TOKENS, fk.shape[1], H)


def run_global(args) -> dict:
    """100 frames x 1374 tokens: global attention over all 137,400 tokens, then per-frame attention."""
    import torch
    from paged_sliding_window_kv_amd import KvCache, lib, paged_attention
    frames, L, H = GLOBAL["frames"], GLOBAL["layers"], GLOBAL["heads"]
    T = frames * VGGT_TOKENS
    steps = max(1, args.steps)
    log(f"[bench] global: {L} layers, {frames} frames x {VGGT_TOKENS} tokens = {T}, timed {steps} pass(es)")
    dev = torch.device("cuda:0")
    lb = lib()
    caches = [KvCache(num_heads=H, dtype="bf16", patch_tokens=VGGT_TOKENS, special_tokens=0, num_scale_units=0,
                      window_units=0, max_units=frames, device=dev) for _ in range(L)]
    g = torch.Generator(device=dev)
    g.manual_seed(2)
    q = [torch.randn((T, H, 64), generator=g, device=dev).to(torch.bfloat16) for _ in range(L)]
    k = [torch.randn((T, H, 64), generator=g, device=dev).to(torch.bfloat16) for _ in range(L)]
    v = [torch.randn((T, H, 64), generator=g, device=dev).to(torch.bfloat16) for _ in range(L)]
    out_g = torch.empty((T, H, 64), dtype=torch.bfloat16, device=dev)
    out_f = torch.empty((T, H, 64), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    sp = torch.cuda.current_stream(dev).cuda_stream
    fb = VGGT_TOKENS * H * 64 * 2
    # per-frame tables: frame f attends to its own 6 pages (page order of the visible table)
    upp = -(-VGGT_TOKENS // 256)
    qo = torch.arange(0, T + 1, VGGT_TOKENS, dtype=torch.int32, device=dev)
    kv = torch.arange(0, frames * upp + 1, upp, dtype=torch.int32, device=dev)
    wsb = max(cc.workspace_bytes(T) for cc in caches)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)
    # the visible tables of every layer's cache after its 100 appends are the same each pass
    tabs = []
    for l in range(L):
        cc = caches[l]
        for f in range(frames):
            cc.append(k[l][f * VGGT_TOKENS:(f + 1) * VGGT_TOKENS], v[l][f * VGGT_TOKENS:(f + 1) * VGGT_TOKENS])
        ids, lens = cc.visible_table()
        tabs.append((torch.from_numpy(ids).to(dev), torch.from_numpy(lens).to(dev)))
    torch.cuda.synchronize()
    # events around every call of the timed passes (77 ms global calls and 1 ms
    # frame calls: the markers cost well under 1%), read after the timed region
    clock_g = CallClock(L * steps)
    clock_f = CallClock(L * steps)

    def one_pass(ci=None):
        """One pass over the 24 layers; ci: first clock slot of its calls (None: no events)."""
        timed_calls = ci is not None
        for l in range(L):
            cc = caches[l]
            _ok(lb.kvc_reset(cc.handle), "reset")
            for f in range(frames):
                _ok(lb.kvc_append_frame(cc.handle, k[l].data_ptr() + f * fb, v[l].data_ptr() + f * fb, sp), "append")
            if timed_calls:
                clock_g.before(ci + l)
            _ok(lb.kvc_attend(cc.handle, q[l].data_ptr(), T, 0.0, out_g.data_ptr(), lse.data_ptr(), ws.data_ptr(),
                              wsb, sp), "attend")
            if timed_calls:
                clock_g.after(ci + l)
                clock_f.before(ci + l)
            paged_attention(q[l], cc.k_pool, cc.v_pool, tabs[l][0], tabs[l][1], qo, kv, VGGT_TOKENS, upp, out=out_f,
                            lse=None, workspace=ws)
            if timed_calls:
                clock_f.after(ci + l)

    one_pass()
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated(dev)  # inputs, pools, outputs, workspace: all resident
    torch.cuda.reset_peak_memory_stats(dev)
    t0 = time.perf_counter()
    for i in range(steps):
        one_pass(i * L)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    clock_g.collect(L * steps)
    clock_f.collect(L * steps)
    peak = torch.cuda.max_memory_allocated(dev)
    score_bytes = T * T * 2  # the score matrix one head would need if it were stored (bf16)
    log(f"[bench] global: device memory {base / 2**30:.2f} GiB before the pass, peak {peak / 2**30:.2f} GiB during it "
        f"(one head's {T} x {T} bf16 score matrix alone would be {score_bytes / 2**30:.1f} GiB)")
    fl_g = L * attn_flops(T, T, H)
    fl_f = L * frames * attn_flops(VGGT_TOKENS, VGGT_TOKENS, H)
    tf = steps * (fl_g + fl_f) / el / 1e12
    kg = clock_g.kernel_s / clock_g.calls
    ach = fl_g / L / kg / 1e12
    tfr = clock_f.call_s / clock_f.calls
    log(f"[bench] global: {el / steps:.3f} s/pass, {tf:.1f} TFLOP/s overall; global kernel {kg * 1e3:.2f} ms avg "
        f"({ach:.1f} TFLOP/s, {ach / PEAK_BF16_TFLOPS:.1%} of bf16 peak); frame calls {tfr * 1e3:.2f} ms avg "
        f"({fl_f / L / tfr / 1e12:.1f} TFLOP/s)")
    res = {
        "value": tf, "unit": "TFLOP/s", "ms_per_step": el / steps * 1e3, "frames_per_s": steps * frames / el,
        "pct_bf16_mfma_peak": 100.0 * tf / PEAK_BF16_TFLOPS, "dtype": "bf16",
        "config": {"workload": f"vggt_global: 24 layers, 100 frames x 1374 tokens = {T}, 16 heads x 64, bf16, "
                               "global attention (no mask) + per-frame attention per layer, appends included; "
                               "step = one pass over 24 layers",
                   "layers": L, "heads": H, "head_dim": 64, "tokens": T, "global_table_pages": len(tabs[0][0]),
                   "device_memory_gib": base / 2**30, "peak_device_memory_gib": peak / 2**30,
                   "score_matrix_one_head_gib": score_bytes / 2**30},
        "roofline": {"bound": "mfma", "achieved": ach, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": ach / PEAK_BF16_TFLOPS, "traffic": None, "kernel": "attn_wide_kernel (global)",
                     "per_launch_flops": fl_g / L, "avg_kernel_us": kg * 1e6,
                     "median_kernel_us": clock_g.median_kernel_us(),
                     "avg_call_us_with_merge": clock_g.call_s / clock_g.calls * 1e6, "calls": clock_g.calls,
                     "frame_attn_tflops": fl_f / L / tfr / 1e12},
    }
    if not args.no_cpu_baseline:
        rows = max(1, args.cpu_rows // 4)
        sec, fl = oracle_global_sample(rows)
        rate = fl / sec / 1e12
        res["cpu_baseline"] = cpu_baseline(
            rate, "TFLOP/s",
            f"1 of 24 layers, all 16 heads: {rows} queries against all {T} keys plus one frame's 1374 queries "
            f"against its own pages (gather + fp64 attention), {sec:.1f} s; extrapolated to a pass by the FLOP ratio",
            sec, {"extrapolated": True, "frames_per_s": frames / ((fl_g + fl_f) / (rate * 1e12))})
    return res


# ----------------------------------------------------------------------------
# Keyframe stream (fp32)
# ----------------------------------------------------------------------------
def keyframe_kept(t: int, c=KEYFRAME) -> bool:
    """Frame t's unit stays in the cache: the scale frames, then every interval-th frame."""
    return t < c["scale"] or (t - c["scale"]) % c["interval"] == 0


def keyframe_lk(units: int, c=KEYFRAME) -> int:
    """Visible tokens with `units` units in the cache: scale + window patches, and the
    special tokens of every unit (special pages are never evicted)."""
    return (min(units, c["scale"]) + min(max(units - c["scale"], 0), c["window"])) * c["patch"] + units * c["special"]


def oracle_keyframe_sample(frames: int, seed: int = 0):
    """The oracle on the first `frames` frames of the keyframe stream (append, fp64 attention, rollback)."""
    import synth
    from oracle import OracleCache, OracleConfig, attention_f64, to_f64
    c = KEYFRAME
    tok = c["patch"] + c["special"]
    oc = OracleCache(OracleConfig(num_heads=c["heads"], head_dim=c["d"], page_size=c["page"],
                                  patch_tokens=c["patch"], special_tokens=c["special"], num_scale_units=c["scale"],
                                  window_units=c["window"], max_units=frames, store_dtype="f32"))
    bank = [synth.frame_qkv(seed, 0, i, tok, c["heads"], c["d"], "f32") for i in range(4)]
    fl = 0.0
    t0 = time.perf_counter()
    for t in range(frames):
        q, k, v = bank[t % 4]
        oc.append(k, v)
        gk, gv = oc.gather()
        attention_f64(to_f64(q), to_f64(gk), to_f64(gv))
        fl += attn_flops(tok, gk.shape[1], c["heads"], c["d"])
        if not keyframe_kept(t):
            oc.rollback()
    return time.perf_counter() - t0, fl


def run_keyframe(args) -> dict:
    """Keyframe stream: 1 layer, 4 heads x 64, fp32 pages, 2 scale + 4 window frames, keyframe interval 4.

    Each frame appends its unit, attends its 262 queries and, unless it is a
    keyframe, rolls the append back (10,000 frames, 7,500 rollbacks).  The step
    is the whole frame: host page bookkeeping, append kernel, attention.
    """
    import torch
    from paged_sliding_window_kv_amd import KvCache, lib
    c = KEYFRAME
    frames = args.steps
    tok, H, d = c["patch"] + c["special"], c["heads"], c["d"]
    log(f"[bench] keyframe: 1 layer, {frames} frames, interval {c['interval']}, warmup {args.warmup}")
    dev = torch.device("cuda:0")
    cache = KvCache(num_heads=H, head_dim=d, page_size=c["page"], dtype="f32", patch_tokens=c["patch"],
                    special_tokens=c["special"], num_scale_units=c["scale"], window_units=c["window"],
                    max_units=max(frames, args.warmup, 1), device=dev)
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    bank = 4
    q, k, v = (torch.randn((bank, tok, H, d), generator=g, device=dev, dtype=torch.float32) for _ in range(3))
    o = torch.empty((tok, H, d), dtype=torch.float32, device=dev)
    lse = torch.empty((tok, H), dtype=torch.float32, device=dev)
    wsb = cache.workspace_bytes(tok)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)
    L = lib()
    h, sp = cache.handle, torch.cuda.current_stream(dev).cuda_stream
    fb = tok * H * d * 4
    qp = [q.data_ptr() + i * fb for i in range(bank)]
    kp = [k.data_ptr() + i * fb for i in range(bank)]
    vp = [v.data_ptr() + i * fb for i in range(bank)]
    op, lp, wsp = o.data_ptr(), lse.data_ptr(), ws.data_ptr()

    def frame(t, clock=None, slot=0):
        b = t % bank
        _ok(L.kvc_append_frame(h, kp[b], vp[b], sp), "kvc_append_frame")
        if clock is not None:
            clock.before(slot)
        _ok(L.kvc_attend(h, qp[b], tok, 0.0, op, lp, wsp, wsb, sp), "kvc_attend")
        if clock is not None:
            clock.after(slot)
        if not keyframe_kept(t):
            _ok(L.kvc_rollback_last_frame(h), "kvc_rollback_last_frame")

    for t in range(args.warmup):
        frame(t)
    torch.cuda.synchronize()
    cache.reset()
    torch.cuda.synchronize()
    mem0 = torch.cuda.memory_allocated(dev)
    t0 = time.perf_counter()
    for t in range(frames):
        frame(t)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    mem1 = torch.cuda.memory_allocated(dev)
    st = cache.state()
    # visible tokens when frame t attends: its own unit plus the units kept before it
    total_flops, lks, kept = 0.0, [], 0
    for t in range(frames):
        lk = keyframe_lk(kept + 1)
        lks.append(lk)
        total_flops += attn_flops(tok, lk, H, d)
        kept += keyframe_kept(t)
    assert st["num_units"] == kept, (st["num_units"], kept)
    assert len(st["scale_pages"]) + len(st["window_pages"]) == min(kept, c["scale"] + c["window"])
    assert mem1 == mem0, (mem0, mem1)
    fps = frames / elapsed
    log(f"[bench] keyframe: {frames} frames in {elapsed:.3f} s, {fps:.0f} frames/s, "
        f"{total_flops / elapsed / 1e12:.2f} TFLOP/s; {kept} units kept, device memory unchanged")
    # attention calls alone, replayed with events around each call
    cache.reset()
    chunk = 64
    clock = CallClock(chunk)
    for t0_ in range(0, frames, chunk):
        n = min(chunk, frames - t0_)
        for i in range(n):
            frame(t0_ + i, clock, i)
        clock.collect(n)
    ach = total_flops / clock.kernel_s / 1e12
    log(f"[bench] keyframe attention: kernel {clock.kernel_s / frames * 1e6:.2f} us avg, {ach:.2f} TFLOP/s "
        f"(fp32 matrix cores)")
    res = {
        "value": fps, "unit": "frames/s", "ms_per_step": elapsed / frames * 1e3, "frames_per_s": fps,
        "dtype": "f32",
        "pct_bf16_mfma_peak": None,
        "config": {"workload": f"keyframe_stream: 1 layer cache, {H} heads x {d}, fp32, 256 patch + 6 special "
                               f"tokens/frame, {c['scale']} scale frames, {c['window']}-frame window, keyframe "
                               f"every {c['interval']} frames (others rolled back), 262 queries/step, {frames} "
                               "frames; step = one frame (append, attention, rollback)",
                   "layers": 1, "heads": H, "head_dim": d, "page_size": c["page"], "frames": frames,
                   "units_kept": kept, "rollbacks": frames - kept, "max_visible_tokens": max(lks),
                   "tflops_whole_step": total_flops / elapsed / 1e12,
                   "device_memory_growth_bytes": mem1 - mem0},
        "roofline": {"bound": "mfma", "achieved": ach, "peak": PEAK_F32_TFLOPS, "unit": "TFLOP/s",
                     "frac": ach / PEAK_F32_TFLOPS, "traffic": None, "kernel": "attn_f32_kernel",
                     "avg_kernel_us": clock.kernel_s / frames * 1e6, "median_kernel_us": clock.median_kernel_us(),
                     "avg_call_us_with_merge": clock.call_s / frames * 1e6, "calls": frames},
    }
    if not args.no_cpu_baseline:
        n = min(frames, 2000)
        sec, fl = oracle_keyframe_sample(n)
        res["cpu_baseline"] = cpu_baseline(n / sec, "frames/s",
                                           f"frames 0..{n - 1} of the keyframe stream (append, fp64 attention, "
                                           f"rollback), {sec:.1f} s", sec, {"tflops": fl / sec / 1e12})
    return res


# ----------------------------------------------------------------------------
# Windowed stream (bf16)
# ----------------------------------------------------------------------------
def windowed_schedule(frames: int, c=WINDOWED):
    """Per frame t: (units in the cache when frame t attends, whether its append restarted the window).

    A window holds c["slots"] kept units; the append after the window is full
    resets the cache and re-appends the last c["overlap"] kept units (fewer if
    fewer were ever kept); a frame that is not a keyframe is rolled back and
    takes no slot.
    """
    units = slots = kept = 0
    out = []
    for t in range(frames):
        restart = slots >= c["slots"]
        if restart:
            units = slots = min(kept, c["overlap"])
        units += 1
        out.append((units, restart))
        if keyframe_kept(t, c):
            slots += 1
            kept += 1
        else:
            units -= 1
    return out


def oracle_windowed_sample(sample: int, seed: int = 0):
    """The oracle on `sample` frames of one layer of the windowed stream, centred on the first restart.

    Frames before the sample are appended, kept or dropped untimed; each
    timed frame is appended (with the restart when it falls there), gathered,
    attended in fp64 and kept or dropped.  Returns (seconds, flops, first
    timed frame).
    """
    import synth
    from oracle import OracleCache, OracleConfig, OracleWindowed, attention_f64, to_f64
    c = WINDOWED
    tok = c["patch"] + c["special"]
    first = next(t for t, (_, r) in enumerate(windowed_schedule(4 * c["slots"] * c["interval"])) if r)
    t0_ = max(0, first - sample // 2)
    ow = OracleWindowed(OracleCache(OracleConfig(num_heads=c["heads"], head_dim=c["d"], page_size=c["page"],
                                                 patch_tokens=c["patch"], special_tokens=c["special"],
                                                 num_scale_units=c["scale"], window_units=c["window"],
                                                 max_units=c["slots"] + 1, store_dtype="bf16")),
                        c["slots"], c["overlap"])
    bank = [synth.frame_qkv(seed, 0, i, tok, c["heads"], c["d"], "bf16") for i in range(4)]

    def finish(t):
        if keyframe_kept(t, c):
            ow.keep()
        else:
            ow.drop()

    for t in range(t0_):
        _, k, v = bank[t % 4]
        ow.append(k, v)
        finish(t)
    fl = 0.0
    start = time.perf_counter()
    for t in range(t0_, t0_ + sample):
        q, k, v = bank[t % 4]
        ow.append(k, v)
        gk, gv = ow.cache.gather()
        attention_f64(to_f64(q), to_f64(gk), to_f64(gv))
        fl += attn_flops(tok, gk.shape[1], c["heads"], c["d"])
        finish(t)
    return time.perf_counter() - start, fl, t0_


def run_windowed(args) -> dict:
    """Windowed LingBot stream: 24 layer caches restarted once per window of 128 kept units, 16 units shared.

    Per frame and layer: kvc_windowed_append (the restart, when the window is
    full, inside it), the frame's attention, then kvc_windowed_keep (keyframes:
    the unit takes a slot and is copied into the overlap ring) or
    kvc_windowed_drop (rollback).  The step is one frame through 24 layers.
    """
    import torch
    from paged_sliding_window_kv_amd import KvCache, lib
    from paged_sliding_window_kv_amd._lib import KvcWindowedState
    c = WINDOWED
    frames, layers, H, d = args.steps, c["layers"], c["heads"], c["d"]
    tok = c["patch"] + c["special"]
    log(f"[bench] windowed: {layers} layers x {frames} frames, window {c['slots']} slots, overlap {c['overlap']}, "
        f"keyframe every {c['interval']} frames, warmup {args.warmup}")
    dev = torch.device("cuda:0")
    L = lib()
    caches = [KvCache(num_heads=H, head_dim=d, page_size=c["page"], dtype="bf16", patch_tokens=c["patch"],
                      special_tokens=c["special"], num_scale_units=c["scale"], window_units=c["window"],
                      max_units=c["slots"] + 1, device=dev) for _ in range(layers)]
    nb = C.c_size_t()
    _ok(L.kvc_windowed_ring_bytes(caches[0].handle, c["overlap"], C.byref(nb)), "kvc_windowed_ring_bytes")
    rings = [[torch.empty(nb.value, dtype=torch.uint8, device=dev) for _ in range(2)] for _ in range(layers)]
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    bank = 4
    shp = (bank, tok, H, d)
    q, k, v = ([torch.randn(shp, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
                for _ in range(layers)] for _ in range(3))
    o = [torch.empty((tok, H, d), dtype=torch.bfloat16, device=dev) for _ in range(layers)]
    lse = [torch.empty((tok, H), dtype=torch.float32, device=dev) for _ in range(layers)]
    wsb = caches[0].workspace_bytes(tok)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)
    fb = tok * H * d * 2
    qp = [[q[l].data_ptr() + i * fb for i in range(bank)] for l in range(layers)]
    kp = [[k[l].data_ptr() + i * fb for i in range(bank)] for l in range(layers)]
    vp = [[v[l].data_ptr() + i * fb for i in range(bank)] for l in range(layers)]
    op, lp, wsp = [x.data_ptr() for x in o], [x.data_ptr() for x in lse], ws.data_ptr()
    sp = torch.cuda.current_stream(dev).cuda_stream
    handles = []

    def start():
        """Fresh windowed handles over emptied caches (the rings are reused)."""
        torch.cuda.synchronize()
        for h in handles:
            _ok(L.kvc_windowed_destroy(h), "kvc_windowed_destroy")
        handles.clear()
        for l, cc in enumerate(caches):
            cc.reset()
            h = C.c_void_p()
            _ok(L.kvc_windowed_create(cc.handle, c["slots"], c["overlap"], rings[l][0].data_ptr(),
                                      rings[l][1].data_ptr(), C.byref(h)), "kvc_windowed_create")
            handles.append(h)
        torch.cuda.synchronize()

    restarted = C.c_int32()
    rp = C.byref(restarted)
    app, att, keep, drop = L.kvc_windowed_append, L.kvc_attend, L.kvc_windowed_keep, L.kvc_windowed_drop

    def frame(t, clock=None):
        b = t % bank
        kf = keyframe_kept(t, c)
        for l in range(layers):
            s = app(handles[l], kp[l][b], vp[l][b], sp, rp)
            if s:
                _ok(s, "kvc_windowed_append")
            if clock is not None:
                clock.before(l)
            s = att(caches[l].handle, qp[l][b], tok, 0.0, op[l], lp[l], wsp, wsb, sp)
            if s:
                _ok(s, "kvc_attend")
            if clock is not None:
                clock.after(l)
            s = keep(handles[l], sp) if kf else drop(handles[l])
            if s:
                _ok(s, "kvc_windowed_keep/drop")
        if clock is not None:
            clock.collect(layers)

    try:
        start()
        for t in range(args.warmup):
            frame(t)
        start()
        mem0 = torch.cuda.memory_allocated(dev)
        t0 = time.perf_counter()
        for t in range(frames):
            frame(t)
            if (t + 1) % 5000 == 0:
                log(f"[bench] windowed: frame {t + 1}")
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        mem1 = torch.cuda.memory_allocated(dev)
        sched = windowed_schedule(frames)
        st = KvcWindowedState()
        _ok(L.kvc_windowed_get_state(handles[0], C.byref(st)), "kvc_windowed_get_state")
        restarts = sum(r for _, r in sched)
        kept = sum(keyframe_kept(t, c) for t in range(frames))
        assert st.windows == restarts, (st.windows, restarts)
        assert caches[0].state()["num_units"] == sched[-1][0] - (0 if keyframe_kept(frames - 1, c) else 1)
        assert mem1 == mem0, (mem0, mem1)
        lks = [keyframe_lk(u, c) for u, _ in sched]
        total_flops = layers * sum(attn_flops(tok, lk, H, d) for lk in lks)
        tflops = total_flops / elapsed / 1e12
        fps = frames / elapsed
        log(f"[bench] windowed: {frames} frames in {elapsed:.3f} s: {fps:.1f} frames/s, {tflops:.1f} TFLOP/s; "
            f"{restarts} restarts, {kept} units kept, device memory unchanged")
        # attention calls alone: the first `replay` frames again, events around every call
        replay = min(frames, args.replay_frames)
        start()
        clock = CallClock(layers)
        for t in range(replay):
            frame(t, clock)
        byt = layers * sum(attn_bytes(tok, lk, H) for lk in lks[:replay])
        flo = layers * sum(attn_flops(tok, lk, H, d) for lk in lks[:replay])
        n = clock.calls
        k_us, c_us = clock.kernel_s / n * 1e6, clock.call_s / n * 1e6
        ach_gbs = byt / clock.kernel_s / 1e9
        log(f"[bench] windowed attention over frames 0..{replay - 1}: kernel {k_us:.2f} us avg "
            f"({ach_gbs:.0f} GB/s), call with merge {c_us:.2f} us")
    finally:
        torch.cuda.synchronize()
        for h in handles:
            L.kvc_windowed_destroy(h)
        handles.clear()
    res = {
        "value": tflops, "unit": "TFLOP/s", "ms_per_step": elapsed / frames * 1e3, "frames_per_s": fps,
        "pct_bf16_mfma_peak": 100.0 * tflops / PEAK_BF16_TFLOPS, "dtype": "bf16",
        "config": {"workload": f"windowed_stream: {layers} layer caches, {H} heads x {d}, bf16, 256 patch + 6 "
                               f"special tokens/frame, {c['scale']} scale frames, {c['window']}-frame window, "
                               f"restart every {c['slots']} kept units sharing the last {c['overlap']}, keyframe "
                               f"every {c['interval']} frames (others rolled back), 262 queries/step, {frames} "
                               "frames; step = one frame through 24 layers (windowed append, attention, keep or "
                               "drop)",
                   "layers": layers, "heads": H, "head_dim": d, "page_size": c["page"], "frames": frames,
                   "window_slots": c["slots"], "overlap": c["overlap"], "keyframe_interval": c["interval"],
                   "restarts": restarts, "units_kept": kept, "max_visible_tokens": max(lks),
                   "mean_visible_tokens": sum(lks) / len(lks),
                   "kv_pool_mib_per_layer": caches[0].k_pool.numel() * caches[0].k_pool.element_size() * 2 / 2**20,
                   "ring_mib_per_layer": 2 * nb.value / 2**20,
                   "device_memory_growth_bytes": mem1 - mem0},
        "roofline": {"bound": "hbm", "achieved": ach_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": ach_gbs / PEAK_HBM_GBS, "traffic": None, "kernel": "attn_bf16_kernel (272-row tile)",
                     "per_launch_bytes": byt / n, "per_launch_flops": flo / n, "avg_kernel_us": k_us,
                     "median_kernel_us": clock.median_kernel_us(),
                     "avg_call_us_with_merge": c_us, "calls": n, "replayed_frames": replay,
                     "kernel_tflops": flo / clock.kernel_s / 1e12},
    }
    if not args.no_cpu_baseline and args.cpu_sample > 0:
        sample = args.cpu_sample
        log(f"[bench] oracle sample: 1 layer, {sample} frames around the first restart")
        sec, fl, first = oracle_windowed_sample(sample)
        ot = fl / sec / 1e12
        res["cpu_baseline"] = cpu_baseline(
            ot, "TFLOP/s",
            f"1 of 24 layers, frames {first}..{first + sample - 1} of the windowed stream (windowed append with "
            f"the first restart, gather, fp64 attention, keep or drop), {sec:.1f} s; frames/s scaled to 24 layers",
            sec, {"frames_per_s": 1.0 / (sec / sample * layers)})
    return res


# ----------------------------------------------------------------------------
# counter calibration and profile bookkeeping
# ----------------------------------------------------------------------------
def copy_probe(nbytes: int = 1 << 30, reps: int = 5) -> None:
    """A plain device-to-device copy of known size (reference for the FETCH_SIZE/WRITE_SIZE counters)."""
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes, "reps": reps}))


def code_text(text: str, line_comment: str) -> str:
    """The text without comments, trailing blanks or empty lines: what the compiler sees of it (string literals
    are kept whole)."""
    out = []
    for line in text.splitlines():
        quote = None
        cut = len(line)
        i = 0
        while i < len(line):
            ch = line[i]
            if quote:
                if ch == "\\":
                    i += 1
                elif ch == quote:
                    quote = None
            elif ch in "\"'":
                quote = ch
            elif line.startswith(line_comment, i):
                cut = i
                break
            i += 1
        code = line[:cut].rstrip()
        if code:
            out.append(code)
    return "\n".join(out)


def attn_source_hash() -> str:
    """Hash of the attention kernels' code and of the build script (whose flags shape the generated code),
    comments left out: a change to a comment leaves the generated code, and so the profiles taken on it, valid."""
    import hashlib
    h = hashlib.sha256()
    for rel, mark in ((("csrc", "attn_bf16.hip"), "//"), (("csrc", "kernels.hpp"), "//"), (("build.py",), "#")):
        with open(os.path.join(ROOT, "paged_sliding_window_kv_amd", *rel), encoding="utf-8") as f:
            h.update(code_text(f.read(), mark).encode())
    return h.hexdigest()[:16]


def measured_traffic_ratio(name: str):
    """HBM bytes over algorithmic bytes per launch, from a committed counter summary.

    The summary holds lines `kernel_source_sha256_16: <hash>` and
    `traffic_ratio: <ratio>`.  None if the kernel source changed since the
    counters were taken (different hash) or the summary is missing.
    """
    path = os.path.join(ROOT, "profiles", name)
    try:
        kv = {}
        with open(path) as f:
            for line in f:
                if ":" in line:
                    a, b = line.split(":", 1)
                    kv[a.strip()] = b.strip()
        if kv.get("kernel_source_sha256_16") != attn_source_hash():
            return None
        return float(kv["traffic_ratio"])
    except (OSError, KeyError, ValueError):
        return None


def add_traffic(res: dict, summary: str) -> None:
    ratio = measured_traffic_ratio(summary)
    rf = res["roofline"]
    if ratio is not None and "per_launch_bytes" in rf:
        rf["traffic"] = ratio * rf["per_launch_bytes"]
        rf["traffic_ratio"] = ratio
        rf["traffic_source"] = f"profiles/{summary}"


DEFAULT_STEPS = {"chunked": 20, "stream": STREAM["frames"], "global": 1, "stream_batched": STREAM["frames"],
                 "keyframe": KEYFRAME["frames"], "windowed": WINDOWED["frames"]}


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps: chunk steps at the full window (chunked, default 20), the last K frames of "
                         "the 1,000-frame stream (stream, stream_batched), passes (global, default 1), frames "
                         "(keyframe, default 10,000; windowed, default 25,000)")
    ap.add_argument("--warmup", type=int, default=5, help="untimed steps before timing (chunked: at least 4)")
    ap.add_argument("--workload", default="chunked",
                    choices=["chunked", "stream", "global", "stream_batched", "keyframe", "windowed"])
    ap.add_argument("--batch", type=int, default=6, help="streams of the stream_batched workload (at most 6 keep "
                    "the 1000-frame tables within one launch)")
    ap.add_argument("--kv-dtype", default="bf16", choices=["bf16", "fp8"],
                    help="stream and chunked: KV page type (fp8 = E4M3 codes with per-token exponents, "
                         "RFC section 3.4)")
    ap.add_argument("--keep-ratio", type=float, default=1.0,
                    help="chunked: attend to a per-layer random page subset keeping this fraction (AVGGT-style)")
    ap.add_argument("--no-extras", action="store_true", help="chunked: skip the LingBot stream and the probes")
    ap.add_argument("--copy-probe", action="store_true", help="run a 1 GiB device copy and exit (counter calibration)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=8192,
                    help="chunked/global oracle slice: query rows of one layer (all heads)")
    ap.add_argument("--cpu-sample", type=int, default=24,
                    help="stream / windowed oracle sample: frames of one layer (the last ones; windowed: around "
                         "the first restart)")
    ap.add_argument("--replay-frames", type=int, default=2000,
                    help="windowed: frames replayed with events around every attention call")
    args = ap.parse_args(argv)
    if args.steps is None:
        args.steps = DEFAULT_STEPS[args.workload]
    if args.steps < 1:
        ap.error("--steps must be at least 1")
    if args.warmup < 0:
        ap.error("--warmup must be non-negative")
    if args.replay_frames < 1:
        ap.error("--replay-frames must be at least 1")
    return args


def main(argv=None):
    args = parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (this path has no multi-GPU "
              "mode: the cache and kernels run on one device)", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_probe:
        copy_probe()
        return
    extras = {}
    if args.workload == "chunked":
        res = run_chunked(args)
        if args.keep_ratio >= 1.0 and args.kv_dtype == "bf16":
            add_traffic(res, "attn_wide_vggt_chunked.md")
        if not args.no_extras:
            st = run_stream(args, cpu_sample=args.cpu_sample)
            if args.kv_dtype == "bf16":
                add_traffic(st, "attn_bf16_lingbot_stream_traffic.md")
            extras["lingbot_stream"] = {k: st[k] for k in ("value", "unit", "ms_per_step", "frames_per_s",
                                                           "pct_bf16_mfma_peak", "config", "roofline")}
            if "cpu_baseline" in st:
                extras["lingbot_stream"]["cpu_baseline"] = st["cpu_baseline"]
    elif args.workload == "stream":
        res = run_stream(args, timed=args.steps)
        if args.kv_dtype == "bf16":
            add_traffic(res, "attn_bf16_lingbot_stream_traffic.md")
    elif args.workload == "stream_batched":
        res = run_stream_batched(args)
    elif args.workload == "keyframe":
        res = run_keyframe(args)
    elif args.workload == "windowed":
        res = run_windowed(args)
    else:
        res = run_global(args)
    probes = None
    if not args.no_extras:
        probes = run_probes()
        rf = res["roofline"]
        meas = probes["mfma_bf16_tflops"] if rf["unit"] == "TFLOP/s" and rf["peak"] == PEAK_BF16_TFLOPS else (
            probes["hbm_read_gbs"] if rf["unit"] == "GB/s" else None)
        if meas:
            rf["peak_measured"] = meas
            rf["frac_of_measured"] = rf["achieved"] / meas
        if rf.get("kernel") in ("attn_wide_kernel", "attn_wide_kernel (global)"):
            rf["tile_mix_tflops"] = probes["tile_mix_tflops"]
            rf["frac_of_tile_mix"] = rf["achieved"] / probes["tile_mix_tflops"]
    out = {
        "metric": METRIC,
        "value": res["value"],
        "unit": res["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": res.get("dtype", "bf16"),
        "data": "synthetic (seeded N(0,1) Q/K/V drawn on the device)",
        "config": res["config"],
        "frames_per_s": res["frames_per_s"],
        "pct_bf16_mfma_peak": res["pct_bf16_mfma_peak"],
        "roofline": res["roofline"],
    }
    if "cpu_baseline" in res:
        out["cpu_baseline"] = res["cpu_baseline"]
    if "step_ms" in res:
        out["step_ms"] = res["step_ms"]
    if extras:
        out["extras"] = extras
    if probes:
        out["probes"] = probes
    out["kernel_source_sha256_16"] = attn_source_hash()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
