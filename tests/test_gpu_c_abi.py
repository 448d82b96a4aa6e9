"""The C ABI from C on the GPU: tests/c/abi_device.c, a C99 program linked
against libkvc.so and HIP's C API (no Python or PyTorch in its process),
drives a bf16 cache through appends, keyframe rollbacks ("LingBot-Map Paged
KV Cache", sections 2-3) and one attention call; its visible table must equal
the oracle's and its O and lse must match the oracle's attention."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import synth
from gpu_helpers import BF16_LSE_ABS, BF16_MAX_ABS, BF16_RMS_REL, log
from oracle import OracleCache, OracleConfig, attention_f64, is_keyframe
from oracle import to_f64 as bits_f64
from paged_sliding_window_kv_amd import _lib as L

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _build(tmp_path):
    L.lib()  # raises if libkvc.so is missing
    libdir = os.path.dirname(os.path.abspath(L.LIB_PATH))
    exe = str(tmp_path / "abi_device")
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{ROCM}/include", os.path.join(ROOT, "tests", "c", "abi_device.c"),
           "-o", exe, f"-L{libdir}", "-lkvc", f"-Wl,-rpath,{libdir}", f"-L{ROCM}/lib", "-lamdhip64",
           f"-Wl,-rpath,{ROCM}/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("H,X,S,W,units,interval", [(2, 6, 2, 4, 40, 3), (16, 6, 8, 64, 100, 1)])
def test_c_program_drives_the_device_path(tmp_path, H, X, S, W, units, interval):
    exe = _build(tmp_path)
    P, T = 256, 256 + X
    log(f"C ABI on the device: H={H}, S={S}, W={W}, {units} units, keyframe interval {interval}")
    bank = [synth.frame_qkv(77, 0, i, T, H, 64, "bf16") for i in range(5)]
    oc = OracleCache(OracleConfig(num_heads=H, head_dim=64, patch_tokens=P, special_tokens=X, num_scale_units=S,
                                  window_units=W, max_units=units, store_dtype="bf16"))
    inp = tmp_path / "in.bin"
    with open(inp, "wb") as f:
        f.write(np.array([H, P, X, S, W, units, interval], dtype="<i4").tobytes())
        for t in range(units):
            _, k, v = bank[t % 5]
            f.write(np.ascontiguousarray(k).astype("<u2").tobytes())
            f.write(np.ascontiguousarray(v).astype("<u2").tobytes())
            oc.append(k, v)
            if t < units - 1 and not is_keyframe(t, S, interval):
                oc.rollback()
        q = bank[(units + 2) % 5][0]
        f.write(np.ascontiguousarray(q).astype("<u2").tobytes())
    out = tmp_path / "out.bin"
    r = subprocess.run([exe, str(inp), str(out)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.startswith("OK"), r.stdout + r.stderr
    raw = out.read_bytes()
    n = int(np.frombuffer(raw[:4], "<i4")[0])
    ids = np.frombuffer(raw[4:4 + 4 * n], "<i4").tolist()
    lens = np.frombuffer(raw[4 + 4 * n:4 + 8 * n], "<i4").tolist()
    off = 4 + 8 * n
    o_bits = np.frombuffer(raw[off:off + T * H * 64 * 2], "<u2").reshape(T, H, 64)
    lse = np.frombuffer(raw[off + T * H * 64 * 2:], "<f4").reshape(T, H).astype(np.float64)
    oids, olens = oc.visible_table()
    assert ids == oids and lens == olens
    gk, gv = oc.gather()
    ro, rl = attention_f64(bits_f64(q), bits_f64(gk), bits_f64(gv))
    o = bits_f64(o_bits)
    err = float(np.abs(o - ro).max())
    rel = float(np.sqrt(np.mean((o - ro) ** 2)) / np.sqrt(np.mean(ro ** 2)))
    lerr = float(np.abs(lse - rl).max())
    log(f"  Lk={gk.shape[1]}, {n} pages: max_abs={err:.3e} rms_rel={rel:.3e} lse={lerr:.3e}")
    assert err <= BF16_MAX_ABS and rel <= BF16_RMS_REL and lerr <= BF16_LSE_ABS
