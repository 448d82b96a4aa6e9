"""The FP8 (E4M3) quantiser of the oracle pinned against torch's float8_e4m3fn and the format's definition."""
import math

import numpy as np
import pytest

import synth
from oracle import (E4M3_MAX, OracleCache, OracleConfig, bf16_bits_to_f64, dequantize_rows, e4m3_decode,
                    e4m3_encode, quantize_rows, row_exponent)
from oracle.fp8 import e4m3_encode_array, row_exponents


def _torch_codes(values):
    import torch
    return torch.tensor(np.asarray(values, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_matches_torch_on_every_code():
    import torch
    codes = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    mine = np.array([e4m3_decode(c) for c in range(256)])
    nan = np.isnan(codes)
    assert (nan == np.isnan(mine)).all() and nan.sum() == 2          # S.1111.111 only
    assert (codes[~nan] == mine[~nan]).all()
    assert max(mine[~nan]) == E4M3_MAX == 448.0
    assert e4m3_decode(0x01) == 2.0 ** -9 and e4m3_decode(0x08) == 2.0 ** -6   # subnormal step, smallest normal


def test_encode_matches_torch_round_to_nearest_even():
    finite = sorted({abs(e4m3_decode(c)) for c in range(256) if not math.isnan(e4m3_decode(c))})
    mids = [(a + b) / 2 for a, b in zip(finite, finite[1:])]          # every tie, both signs
    rng = np.random.default_rng(1)
    rand = np.concatenate([rng.uniform(-448, 448, 20000), rng.uniform(-0.03, 0.03, 20000)])
    for vals in (finite + [-x for x in finite], mids + [-x for x in mids], rand.astype(np.float32)):
        mine = np.array([e4m3_encode(float(v)) for v in vals], np.uint8)
        assert (mine == _torch_codes(vals)).all()
    with pytest.raises(ValueError):
        e4m3_encode(449.0)


def test_row_exponent_is_the_smallest_that_fits():
    rng = np.random.default_rng(2)
    for amax in list(rng.uniform(1e-6, 1e6, 2000)) + [448.0, 448.0 * 2 ** 5, 448.0 * 2 ** -5, 1.0, 2.0 ** -120]:
        e = row_exponent(float(amax))
        assert amax <= 448.0 * 2.0 ** e
        assert e == -127 or amax > 448.0 * 2.0 ** (e - 1)
    assert row_exponent(448.0) == 0 and row_exponent(448.0 * 8) == 3 and row_exponent(449.0) == 1
    assert row_exponent(0.0) == -127


def test_quantised_rows_round_trip_within_half_a_step():
    x = bf16_bits_to_f64(synth.normal_tokens(3, 0, 0, synth.KIND_K, 64, 4, 64, "bf16")) * 3.0
    codes, exps = quantize_rows(x)
    y = dequantize_rows(codes, exps)
    # relative error of a normal E4M3 value is at most 2^-4; absolute error at most 2^-10 * 2^e below 2^-6
    scale = np.ldexp(1.0, exps.astype(np.int64))[..., None]
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * scale)
    assert (np.abs(y - x) <= bound).all()
    # every row uses its range: the largest magnitude lands in the top binade
    assert (np.abs(y).max(axis=-1) / scale[..., 0] >= 224).all()
    # values already on the grid come back exactly
    assert (dequantize_rows(*quantize_rows(y)) == y).all()


def test_fp8_cache_gathers_the_quantised_history():
    """Gathered K/V of an FP8 cache equal the per-token quantisation of the tokens the table selects."""
    H, P, X, S, W = 2, 256, 6, 1, 2
    oc = OracleCache(OracleConfig(num_heads=H, head_dim=64, patch_tokens=P, special_tokens=X, num_scale_units=S,
                                  window_units=W, max_units=6, store_dtype="fp8"))
    hist_k = []
    for t in range(6):
        k = synth.normal_tokens(5, 0, t, synth.KIND_K, P + X, H, 64, "bf16")
        v = synth.normal_tokens(5, 0, t, synth.KIND_V, P + X, H, 64, "bf16")
        oc.append(k, v)
        hist_k.append(k)
    gk, _ = oc.gather()
    # scale unit 0, window units 4, 5, then the special tokens of all six frames
    sel = [hist_k[0][:P], hist_k[4][:P], hist_k[5][:P]] + [h[P:] for h in hist_k]
    ref = dequantize_rows(*quantize_rows(bf16_bits_to_f64(np.concatenate(sel))))
    assert (gk == ref.transpose(1, 0, 2)).all()


def test_vectorised_forms_agree_with_the_scalar_steps():
    rng = np.random.default_rng(3)
    finite = sorted({abs(e4m3_decode(c)) for c in range(256) if not math.isnan(e4m3_decode(c))})
    mids = [(a + b) / 2 for a, b in zip(finite, finite[1:])]
    y = np.concatenate([rng.uniform(-448, 448, 5000), rng.uniform(-0.02, 0.02, 5000), finite, mids,
                        [-x for x in mids], [0.0, -0.0]])
    assert (e4m3_encode_array(y) == np.array([e4m3_encode(float(v)) for v in y], np.uint8)).all()
    amax = np.concatenate([rng.uniform(1e-8, 1e8, 3000), [0.0, 448.0, 449.0, 448.0 * 2 ** 7]])
    assert (row_exponents(amax) == np.array([row_exponent(float(a)) for a in amax])).all()
