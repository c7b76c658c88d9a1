"""FP8 E4M3 codec written from the format's definition (oracle side).

The V3 FP8 framework stores every quantised tensor in E4M3 ("DeepSeek_V3_Report:
Annotation", section "Mantissa over Exponents"). The variant used here is the
OCP E4M3FN layout, the one gfx950's fp8 matrix instructions read:

* bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0 mantissa;
* exponent field 0 encodes subnormals m/8 * 2^-6 (smallest 2^-9);
* exponent field 1..15 encodes (1 + m/8) * 2^(e-7);
* S.1111.111 is NaN; there are no infinities, so the largest finite value is
  1.75 * 2^8 = 448.

Encoding saturates to +-448 and rounds to nearest, ties to the even code.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def _decode_fields(codes) -> np.ndarray:
    """Decode from the bit fields (the definition)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    sub = m / 8.0 * 2.0 ** -6
    nrm = (1.0 + m / 8.0) * np.ldexp(1.0, (e - 7).astype(np.int64))
    v = np.where(e == 0, sub, nrm) * sign
    return np.where((c & 0x7F) == 0x7F, np.nan, v)


_TABLE = _decode_fields(np.arange(256, dtype=np.uint8))       # value of every code
_GRID = _TABLE[:0x7F]                                         # non-negative finite values, code order
assert np.all(np.diff(_GRID) > 0)


def e4m3_decode(codes) -> np.ndarray:
    """Decode uint8 codes to float64 (NaN for the two NaN codes)."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(x) -> np.ndarray:
    """Round float values to E4M3 codes: saturate to 448, nearest, ties to even.

    Within a binade [2^E, 2^(E+1)) (E >= -6) the representable values are the
    multiples of the quantum 2^(E-3); below 2^-6 the quantum is 2^-9. Rounding
    to the nearest multiple with ties to the even multiple is exactly rounding
    to the nearest code with ties to the even mantissa, and a carry into the
    next binade lands on its first value. Division and multiplication by the
    power-of-two quantum are exact.
    """
    x = np.asarray(x, dtype=np.float64)
    neg = np.signbit(x)
    a = np.minimum(np.abs(x), E4M3_MAX)
    _, ex = np.frexp(a)                     # a = m * 2^ex, m in [0.5, 1)  =>  binade E = ex - 1
    q = np.ldexp(1.0, np.maximum(ex - 1, -6) - 3)
    v = np.minimum(np.rint(a / q) * q, E4M3_MAX)
    # code of the grid value v: exponent field E + 7 and mantissa v / 2^(E-3) - 8 in
    # the normal range, v / 2^-9 below 2^-6
    _, ev = np.frexp(v)
    ev = ev - 1
    normal = v >= 2.0 ** -6
    code = np.where(normal, (ev + 7) * 8 + (np.ldexp(v, 3 - ev) - 8), np.ldexp(v, 9)).astype(np.uint8)
    code |= np.where(neg, 0x80, 0).astype(np.uint8)
    return np.where(np.isnan(x), np.uint8(0x7F), code).astype(np.uint8)


def e4m3_encode_nearest(x) -> np.ndarray:
    """Reference encoder by exhaustive nearest-value search (slow; used to cross-check)."""
    x = np.asarray(x, dtype=np.float64)
    neg = np.signbit(x)
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.clip(np.searchsorted(_GRID, a, side="left"), 0, len(_GRID) - 1)
    lo = np.clip(hi - 1, 0, len(_GRID) - 1)
    d_lo, d_hi = a - _GRID[lo], _GRID[hi] - a
    code = np.where((d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0)), hi, lo)
    code = np.where(a == _GRID[hi], hi, code).astype(np.uint8)
    code |= np.where(neg, 0x80, 0).astype(np.uint8)
    return np.where(np.isnan(x), np.uint8(0x7F), code).astype(np.uint8)
