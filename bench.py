#!/usr/bin/env python3
"""Throughput of paged sliding-window KV attention on one MI355X.

Default workload (one JSON line on stdout): a LingBot-Map-shaped stream.
24 independent layer caches, 16 heads x 64 dims, bf16.  Each frame carries
256 patch and 6 special tokens.  There are 8 scale frames, a 64-frame window
and 42 frames per special page.  1000 frames are streamed.  One step is one
frame through all 24 layers: the append (scatter of K/V into pages), the
visible table and the attention of the frame's 262 query tokens against it.
Inputs are seeded synthetic N(0,1) tensors, resident in HBM before timing.

Other workloads (--workload): "chunked" is VGGT-style chunked global attention
(8-frame chunks of 1374 tokens, window of 4 chunks).  "global" is full global
attention over 100 frames x 1374 tokens followed by per-frame attention.
"""
from __future__ import annotations

import argparse
import ctypes as C
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged attention TFLOP/s + streamed frames/s (% of bf16 MFMA peak), 1 MI355X"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------
# shared pieces
# ----------------------------------------------------------------------------
def _ok(status: int, where: str) -> None:
    if status != 0:
        from paged_sliding_window_kv_amd import _lib as L
        L.check(status, where)


def attn_flops(lq: int, lk: int, heads: int, d: int = 64) -> float:
    """QK^T and PV: 2 * 2 * Lq * Lk * d per head (softmax not counted)."""
    return 4.0 * lq * lk * d * heads


def attn_bytes(lq: int, lk: int, heads: int, d: int = 64, elem: int = 2) -> float:
    """Bytes an attention call must move: K and V of the visible tokens, Q in, O out, LSE out."""
    return 2.0 * lk * heads * d * elem + 2.0 * lq * heads * d * elem + lq * heads * 4.0


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


# ----------------------------------------------------------------------------
# LingBot-Map-shaped stream
# ----------------------------------------------------------------------------
STREAM = dict(layers=24, heads=16, d=64, page=256, patch=256, special=6, scale=8, window=64, frames=1000)


def stream_lk(t: int, c=STREAM) -> int:
    """Visible tokens after appending frame t (0-based): scale + window patches + all specials."""
    n = t + 1
    units = min(n, c["scale"]) + min(max(n - c["scale"], 0), c["window"])
    return units * c["patch"] + n * c["special"]


class StreamBench:
    def __init__(self, frames: int, layers: int, bank: int = 4, seed: int = 0):
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
        self.caches = [KvCache(num_heads=c["heads"], head_dim=c["d"], page_size=c["page"], dtype="bf16",
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

    def step(self, t: int, events=None):
        lib, sp, b = self.lib, self.sp, t % self.bank
        app, att = lib.kvc_append_frame, lib.kvc_attend
        wsp, wsb, nq = self.ws.data_ptr(), self.wsb, self.tokens
        for l in range(self.layers):
            s = app(self.h[l], self.kp[l][b], self.vp[l][b], sp)
            if s:
                _ok(s, "kvc_append_frame")
            if events is not None:
                events[2 * l].record(self.stream)
            s = att(self.h[l], self.qp[l][b], nq, 0.0, self.op[l], self.lp[l], wsp, wsb, sp)
            if s:
                _ok(s, "kvc_attend")
            if events is not None:
                events[2 * l + 1].record(self.stream)

    def run(self, frames: int):
        for t in range(frames):
            self.step(t)

    def timed(self, frames: int) -> float:
        torch = self.torch
        self.reset()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        self.run(frames)
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    def attention_kernel_time(self, frames: int):
        """Replay the stream with HIP events around every attention call (same stream).

        Returns (seconds inside attention calls, algorithmic bytes, flops) summed over the replay.
        """
        torch = self.torch
        self.reset()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * self.layers)]
        tot = 0.0
        byt = 0.0
        flo = 0.0
        c = self.c
        for t in range(frames):
            self.step(t, ev)
            ev[-1].synchronize()
            lk = stream_lk(t, c)
            for l in range(self.layers):
                tot += ev[2 * l].elapsed_time(ev[2 * l + 1]) * 1e-3
            byt += self.layers * attn_bytes(self.tokens, lk, c["heads"], c["d"])
            flo += self.layers * attn_flops(self.tokens, lk, c["heads"], c["d"])
        return tot, byt, flo

    def check_tables(self):
        ids, lens = self.caches[0].visible_table()
        return int(lens.sum()), len(ids)


def oracle_stream_sample(frames: int, sample: int, bank: int = 4, seed: int = 0):
    """The CPU oracle on a bounded sample of the same stream: one layer.

    Units are appended up to frame frames - sample - 1 untimed.  The last
    `sample` frames are then timed: append, gather and fp64 attention.
    Returns (seconds, flops of the timed part, frames timed).
    """
    import synth
    from oracle import OracleCache, OracleConfig, attention_f64, to_f64
    c = STREAM
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


def run_stream(args) -> dict:
    import torch
    frames, layers = args.steps, STREAM["layers"]
    log(f"[bench] stream: {layers} layers x {frames} frames, warmup {args.warmup}")
    b = StreamBench(max(frames, args.warmup), layers)
    if args.warmup:
        b.run(args.warmup)
        torch.cuda.synchronize()
    elapsed = b.timed(frames)
    lk_sum, npages = b.check_tables()
    assert lk_sum == stream_lk(frames - 1), (lk_sum, stream_lk(frames - 1))
    total_flops = sum(layers * attn_flops(b.tokens, stream_lk(t), STREAM["heads"]) for t in range(frames))
    tflops = total_flops / elapsed / 1e12
    fps = frames / elapsed
    log(f"[bench] timed {frames} frames in {elapsed:.3f} s: {tflops:.1f} TFLOP/s, {fps:.1f} frames/s")
    att_s, att_b, att_f = b.attention_kernel_time(frames)
    n_launch = frames * layers
    avg_us = att_s / n_launch * 1e6
    ach_gbs = att_b / att_s / 1e9
    log(f"[bench] attention calls: {avg_us:.2f} us avg, {ach_gbs:.0f} GB/s, {att_f / att_s / 1e12:.1f} TFLOP/s")
    res = {
        "value": tflops,
        "unit": "TFLOP/s",
        "ms_per_step": elapsed / frames * 1e3,
        "frames_per_s": fps,
        "pct_bf16_mfma_peak": 100.0 * tflops / PEAK_BF16_TFLOPS,
        "config": {
            "workload": "lingbot_stream: 24 layer caches, 16 heads x 64, bf16, 256 patch + 6 special tokens/frame, "
                        "8 scale frames, 64-frame window, 42 frames/special page, 262 queries/step, "
                        f"{frames} frames",
            "layers": layers, "heads": 16, "head_dim": 64, "page_size": 256, "frames": frames,
            "final_visible_tokens": lk_sum, "final_visible_pages": npages,
        },
        "roofline": {
            "bound": "hbm", "achieved": ach_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": ach_gbs / PEAK_HBM_GBS, "traffic": None,
            "kernel": "paged attention call (attn_bf16_kernel + attn_merge_kernel)",
            "avg_call_us": avg_us, "calls": n_launch,
            "bytes_per_call_avg": att_b / n_launch,
            "attn_tflops": att_f / att_s / 1e12,
            "attn_frac_bf16_peak": att_f / att_s / 1e12 / PEAK_BF16_TFLOPS,
        },
    }
    if not args.no_cpu_baseline:
        sample = args.cpu_sample
        log(f"[bench] oracle sample: 1 layer, last {sample} of {frames} frames")
        sec, fl, nfr = oracle_stream_sample(frames, sample)
        ot = fl / sec / 1e12
        res["cpu_baseline"] = {
            "value": ot, "unit": "TFLOP/s", "cores": blas_threads(), "kind": "oracle",
            "sample": f"1 of 24 layers, frames {frames - sample}..{frames - 1} of the {frames}-frame stream "
                      f"(append + gather + fp64 attention), {sec:.1f} s",
            "frames_per_s": 1.0 / (sec / nfr * layers),
        }
        log(f"[bench] oracle: {ot * 1e3:.2f} GFLOP/s over {sec:.1f} s")
    return res


# ----------------------------------------------------------------------------
def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000, help="frames streamed in the timed region")
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--workload", default="stream", choices=["stream"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=4, help="frames of one layer the oracle times")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (this path has no multi-GPU "
              "mode: the cache and kernels run on one device)", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    res = run_stream(args)
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
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q/K/V, 4-frame bank per layer)",
        "config": res["config"],
        "frames_per_s": res["frames_per_s"],
        "pct_bf16_mfma_peak": res["pct_bf16_mfma_peak"],
        "roofline": res["roofline"],
    }
    if "cpu_baseline" in res:
        out["cpu_baseline"] = res["cpu_baseline"]
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
