"""The roofline probes (include/kvc_probe.h) on the GPU: each runs, returns a
rate in range, and refuses a short scratch buffer.  The tile-mix probe issues
a subset of the matrix-core probe's load per product (plus the softmax), so it
cannot beat the matrix-core rate, and the chip's published bf16 peak bounds
both; the read probe cannot beat the published HBM bandwidth by much."""
import ctypes as C

import pytest

from gpu_helpers import log

pytestmark = pytest.mark.gpu


def test_probes_rates_in_range():
    import torch
    from paged_sliding_window_kv_amd import lib
    from paged_sliding_window_kv_amd import _lib as L
    lb = lib()
    sp = torch.cuda.current_stream().cuda_stream
    n = lb.kvc_probe_scratch_bytes()
    scratch = torch.empty(n, dtype=torch.uint8, device="cuda")
    mfma, mix = C.c_double(), C.c_double()
    assert lb.kvc_probe_mfma_bf16(scratch.data_ptr(), n, sp, C.byref(mfma)) == 0
    assert lb.kvc_probe_tile_mix(scratch.data_ptr(), n, sp, C.byref(mix)) == 0
    log(f"probes: matrix cores {mfma.value:.0f} TFLOP/s, tile mix {mix.value:.0f} TFLOP/s")
    assert 500.0 < mfma.value < 2600.0
    assert 300.0 < mix.value <= mfma.value * 1.02
    nb = 1 << 30
    src = torch.ones(nb, dtype=torch.uint8, device="cuda")
    dst = torch.empty(nb, dtype=torch.uint8, device="cuda")
    rd, cp = C.c_double(), C.c_double()
    assert lb.kvc_probe_hbm(src.data_ptr(), dst.data_ptr(), nb, scratch.data_ptr(), n, sp, C.byref(rd), C.byref(cp)) == 0
    log(f"probes: HBM read {rd.value:.0f} GB/s, copy {cp.value:.0f} GB/s")
    assert 1000.0 < rd.value < 8800.0 and 500.0 < cp.value < 8800.0
    torch.cuda.synchronize()
    assert torch.equal(dst[:4096], src[:4096])
    # a short scratch buffer is refused before anything is launched
    assert lb.kvc_probe_tile_mix(scratch.data_ptr(), n - 1, sp, C.byref(mix)) == L.KVC_ERR_BUFFER_TOO_SMALL
    assert lb.kvc_probe_mfma_bf16(scratch.data_ptr(), n - 1, sp, C.byref(mfma)) == L.KVC_ERR_BUFFER_TOO_SMALL
