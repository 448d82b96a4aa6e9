"""FP8 KV pages (test infrastructure: the oracle of the quantised cache).

"vLLM-Omni RFC #2727: Reconstruction Engine", section 3.4, item 5, lists KV
Cache FP8/INT8 for about half the memory; the large-scale configuration of
the same section combines it with the chunked cache ("KV-FP8").  The pages fix
neither the FP8 format nor the scaling.  Reading used here:

* Format: OCP 8-bit floating point E4M3 (1 sign, 4 exponent bits with bias
  7, 3 mantissa bits; exponent field 0 gives subnormals m * 2^-9; the all-ones
  pattern S.1111.111 is NaN; the largest finite value is 448).
* Scale: one power of two per (token, head) row of K and of V, 2^e with e the
  smallest integer in [-127, 127] such that max|x| <= 448 * 2^e (e = -127
  for an all-zero row).  Rows are quantised when they are appended, so a
  page that fills over many appends (the special stream) never needs
  rescaling, and a dequantised value (code value * 2^e) is exactly a bf16
  number (3 mantissa bits).
* Rounding: x / 2^e (exact) to the nearest E4M3 value, ties to the even
  code.  |x / 2^e| <= 448 by the choice of e, so nothing saturates.
"""
from __future__ import annotations

import math

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode(code: int) -> float:
    """Value of an E4M3 code (OCP definition above)."""
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 15
    m = code & 7
    if e == 15 and m == 7:
        return math.nan
    if e == 0:
        return s * m * 2.0 ** -9
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3_VALUES = np.array([e4m3_decode(c) for c in range(256)])


def e4m3_encode(y: float) -> int:
    """Nearest E4M3 code to y (|y| <= 448), ties to the even code."""
    if not abs(y) <= E4M3_MAX:
        raise ValueError("value outside the E4M3 range")
    sign = 0x80 if math.copysign(1.0, y) < 0 else 0
    a = abs(y)
    if a < 2.0 ** -6:                    # subnormal range: steps of 2^-9
        m = round(a * 512.0)             # exact product; round() is half-to-even
        return sign | m                  # m == 8 is the smallest normal, code 0x08
    fm, fe = math.frexp(a)               # a = fm * 2^fe, fm in [0.5, 1)
    E = fe - 1                           # a in [2^E, 2^(E+1))
    m = round((a / 2.0 ** E - 1.0) * 8.0)  # exact; 0..8
    if m == 8:
        E, m = E + 1, 0
    return sign | ((E + 7) << 3) | m


def e4m3_encode_array(y: np.ndarray) -> np.ndarray:
    """e4m3_encode over an array (same steps, vectorised; |y| <= 448)."""
    y = np.asarray(y, np.float64)
    if not (np.abs(y) <= E4M3_MAX).all():
        raise ValueError("value outside the E4M3 range")
    sign = np.where(np.signbit(y), 0x80, 0).astype(np.int64)
    a = np.abs(y)
    sub = a < 2.0 ** -6
    m_sub = np.round(a * 512.0).astype(np.int64)           # numpy rounds half to even
    fm, fe = np.frexp(np.where(sub, 1.0, a))
    E = fe.astype(np.int64) - 1
    m = np.round((np.where(sub, 1.0, a) / np.ldexp(1.0, E) - 1.0) * 8.0).astype(np.int64)
    carry = m == 8
    E = np.where(carry, E + 1, E)
    m = np.where(carry, 0, m)
    code = np.where(sub, m_sub, ((E + 7) << 3) | m)
    return (sign | code).astype(np.uint8)


def row_exponent(amax: float) -> int:
    """Smallest e in [-127, 127] with amax <= 448 * 2^e."""
    if amax == 0.0:
        return -127
    fm, fe = math.frexp(amax)            # amax = fm * 2^fe
    E = fe - 1
    e = E - 8 if 2.0 * fm <= 1.75 else E - 7
    return max(-127, min(127, e))


def row_exponents(amax: np.ndarray) -> np.ndarray:
    """row_exponent over an array."""
    amax = np.asarray(amax, np.float64)
    fm, fe = np.frexp(amax)
    E = fe.astype(np.int64) - 1
    e = np.where(2.0 * fm <= 1.75, E - 8, E - 7)
    e = np.where(amax == 0.0, -127, e)
    return np.clip(e, -127, 127)


def quantize_rows(x: np.ndarray):
    """x: float64 array [..., d] of exact bf16 values -> (codes uint8 [..., d], exponents int8 [...])."""
    e = row_exponents(np.abs(x).max(axis=-1))
    codes = e4m3_encode_array(x * np.ldexp(1.0, -e)[..., None])   # exact: power-of-two scaling
    return codes, e.astype(np.int8)


def dequantize_rows(codes: np.ndarray, exps: np.ndarray) -> np.ndarray:
    """codes uint8 [..., d], exponents int8 [...] -> float64 values code * 2^e."""
    return E4M3_VALUES[codes] * np.ldexp(1.0, exps.astype(np.int64))[..., None]
