"""Shared helpers of the GPU parity tests: host<->device bit moves and tolerance checks."""
import math
import sys

import numpy as np

import synth

# Tolerances.  bf16 inputs with fp32 accumulation: the stated bar is a max-abs
# error of 2e-2 against the fp64 oracle.  Outputs of N(0,1) data are small
# (|O| ~ sqrt(e / Lk)), so the RMS error relative to the reference's RMS and
# the log-sum-exp are checked as well.  The bf16 kernel rounds P and O to bf16
# (relative 2^-9 each), so 1e-2 relative RMS leaves ample room; lse carries
# only fp32 rounding.  fp32 path: fp32 products and sums over <= 2e4 terms.
BF16_MAX_ABS = 2e-2
BF16_RMS_REL = 1e-2
BF16_LSE_ABS = 1e-3
F32_MAX_ABS = 1e-4
F32_LSE_ABS = 1e-4


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(x: np.ndarray, dtype: str, device="cuda"):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)


def to_host_bits(t, dtype: str) -> np.ndarray:
    import torch
    if dtype == "bf16":
        return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)
    return t.detach().cpu().numpy()


def to_f64(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def check_attention(o_dev, lse_dev, o_ref, lse_ref, dtype: str, what: str = ""):
    o = to_f64(o_dev)
    lse = to_f64(lse_dev) if lse_dev is not None else None
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    err = float(np.abs(o - o_ref).max()) if o.size else 0.0
    if dtype == "bf16":
        rms_ref = math.sqrt(float(np.mean(o_ref ** 2))) if o.size else 1.0
        rms_err = math.sqrt(float(np.mean((o - o_ref) ** 2))) if o.size else 0.0
        rel = rms_err / max(rms_ref, 1e-30)
        log(f"  {what}: max_abs={err:.3e} rms_rel={rel:.3e}")
        assert err <= BF16_MAX_ABS, f"{what}: max abs error {err}"
        assert rel <= BF16_RMS_REL or rms_ref < 1e-12, f"{what}: rms rel error {rel}"
        lse_tol = BF16_LSE_ABS
    else:
        log(f"  {what}: max_abs={err:.3e}")
        assert err <= F32_MAX_ABS, f"{what}: max abs error {err}"
        lse_tol = F32_LSE_ABS
    if lse is not None:
        fin = np.isfinite(lse_ref)
        assert (np.isneginf(lse[~fin])).all(), f"{what}: lse of empty rows must be -inf"
        if fin.any():
            le = float(np.abs(lse[fin] - lse_ref[fin]).max())
            assert le <= lse_tol, f"{what}: lse error {le}"


def v_slot_pos(s: int) -> int:
    """Element of a V pool row that holds slot s (the layout include/kvc.h documents)."""
    return (s & ~15) | (s & 3) | ((s & 4) << 1) | ((s & 8) >> 1)


def v_positions(page_size: int) -> np.ndarray:
    return np.array([v_slot_pos(s) for s in range(page_size)], np.int64)


def v_pool_device_layout(v_nat: np.ndarray) -> np.ndarray:
    """[N, H, P, d] natural V pages -> [N, H, d, P] device layout (rows in pool slot order)."""
    vt = np.ascontiguousarray(v_nat.transpose(0, 1, 3, 2))
    return np.ascontiguousarray(vt[..., v_positions(vt.shape[-1])])  # map is its own inverse


def v_pool_natural(v_dev: np.ndarray) -> np.ndarray:
    """[N, H, d, P] device layout -> [N, H, P, d] natural V pages."""
    return np.ascontiguousarray(v_dev[..., v_positions(v_dev.shape[-1])].transpose(0, 1, 3, 2))


def unit_qkv(seed, layer, t, tokens, heads, head_dim, dtype, q_scale=1.0):
    return synth.frame_qkv(seed, layer, t, tokens, heads, head_dim, dtype, q_scale)
