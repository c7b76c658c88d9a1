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


def e4m3_decode(codes) -> np.ndarray:
    """Decode uint8 codes to float64 (NaN for the two NaN codes)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    sub = m / 8.0 * 2.0 ** -6
    nrm = (1.0 + m / 8.0) * np.ldexp(1.0, (e - 7).astype(np.int64))
    v = np.where(e == 0, sub, nrm) * sign
    v = np.where((c & 0x7F) == 0x7F, np.nan, v)
    return v


# Non-negative finite values in code order 0x00..0x7E; the order of codes is
# also the order of values, which the encoder's search relies on.
_GRID = e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
assert np.all(np.diff(_GRID) > 0)


def e4m3_encode(x) -> np.ndarray:
    """Round float values to E4M3 codes: saturate to 448, nearest, ties to even."""
    x = np.asarray(x, dtype=np.float64)
    neg = np.signbit(x)
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_GRID, a, side="left")          # _GRID[hi-1] < a <= _GRID[hi]
    hi = np.clip(hi, 0, len(_GRID) - 1)
    lo = np.clip(hi - 1, 0, len(_GRID) - 1)
    d_lo = a - _GRID[lo]
    d_hi = _GRID[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a == _GRID[hi], hi, code)
    code = code.astype(np.uint8) | np.where(neg, 0x80, 0).astype(np.uint8)
    code = np.where(np.isnan(x), np.uint8(0x7F), code)
    return code.astype(np.uint8)
