"""MXFP4 expert weights (oracle side, TEST INFRASTRUCTURE).

"DeepSeek V3 / V4 Infra", section on V4 post-training: the MoE expert weights
are trained quantisation-aware in FP4 (MXFP4), and the FP4 -> FP8 (E4M3)
dequantisation is lossless as long as, inside every 128x128 FP8 block, the
ratio of the largest to the smallest 1x32 FP4 sub-block scale stays below a
bound, because E4M3 has two exponent bits more than E2M1.

MXFP4 is the OCP Microscaling format: blocks of 32 consecutive values share
one E8M0 scale (a bare power of two 2^(code - 127)); each value is an E2M1
code:

* bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa;
* exponent field 0: subnormal 0 or 0.5; fields 1..3: (1 + m/2) * 2^(e-1);
* magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; no infinities or NaN.

Readings taken here (the pages name the format, not its conversion rule):

* shared scale of a block = 2^(floor(log2(amax)) - 2), 2 being the exponent
  of E2M1's largest value (the OCP rule), at least 2^-127; an all-zero block
  takes 2^0;
* elements = E2M1 of x / scale, round to nearest with ties to the even code,
  saturating at +-6 (so a block maximum in [6, 8) * scale clips to 6); the
  sign bit is the sign of x, so a negative value that rounds to 0 keeps it;
* blocks run along K (the contraction axis of the expert GEMMs), as the
  1x32 sub-block of the pages.

The bound of the lossless claim, derived: a value is e * 2^k (e an E2M1
magnitude, k the sub-block exponent). With the FP8 block scale S = 2^(kmax-6)
it becomes e * 2^j, j = k - kmax + 6 <= 6, so 6 * 2^j <= 384 < 448; it is an
exact E4M3 value while 0.5 * 2^j >= 2^-9 (E4M3's smallest subnormal, on whose
grid 1.5 * 2^j then also lies), i.e. j >= -8. Hence lossless iff
kmax - kmin <= 14 over the sub-blocks that hold a nonzero value.
"""
from __future__ import annotations

import numpy as np

from .e4m3 import E4M3_MAX, e4m3_encode

E2M1_MAX = 6.0
E2M1_EMAX = 2              # exponent of the largest E2M1 value
MX_BLOCK = 32
LOSSLESS_SPAN = 14         # kmax - kmin bound of the FP4 -> FP8 conversion


def _decode_fields(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x8, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = (c & 0x1).astype(np.float64)
    sub = m * 0.5
    nrm = (1.0 + m / 2.0) * np.ldexp(1.0, (e - 1).astype(np.int64))
    return np.where(e == 0, sub, nrm) * sign


_TABLE = _decode_fields(np.arange(16, dtype=np.uint8))
_GRID = _TABLE[:8]                        # non-negative magnitudes, code order
assert np.all(np.diff(_GRID) > 0)


def e2m1_decode(codes) -> np.ndarray:
    """Decode E2M1 codes (0..15) to float64."""
    return _TABLE[np.asarray(codes, dtype=np.uint8) & 0xF]


def e2m1_encode(x) -> np.ndarray:
    """Nearest E2M1 code, ties to the even code (mantissa bit 0), saturating at +-6.

    Magnitudes are compared with the midpoints of neighbouring grid values; at
    an exact midpoint the neighbour with the even code wins.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E2M1_MAX)
    hi = np.searchsorted(_GRID, a, side="left").clip(0, 7)     # first grid value >= a
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _GRID[lo]
    d_hi = _GRID[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    mag = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(np.signbit(x), mag | 0x8, mag).astype(np.uint8)


def mx_block_exponent(amax) -> np.ndarray:
    """E8M0 exponent k of a block: floor(log2(amax)) - 2 (0 for an all-zero block), at least -127
    (E8M0's smallest; only blocks with amax below 2^-125 meet the bound)."""
    amax = np.asarray(amax, dtype=np.float64)
    _, e = np.frexp(np.where(amax > 0, amax, 1.0))      # amax = m 2^e, 0.5 <= m < 1
    return np.where(amax > 0, np.maximum(e - 1 - E2M1_EMAX, -127), 0).astype(np.int64)


def quantize_mxfp4(w):
    """w [..., R, K] (bf16 / fp32 values) -> (codes [..., R, K] uint8 (one E2M1 code per value),
    scales [..., R, K/32] uint8 E8M0 codes = k + 127)."""
    w = np.asarray(w.float().cpu().numpy() if hasattr(w, "float") else w, dtype=np.float64)
    K = w.shape[-1]
    assert K % MX_BLOCK == 0
    blk = w.reshape(*w.shape[:-1], K // MX_BLOCK, MX_BLOCK)
    k = mx_block_exponent(np.max(np.abs(blk), axis=-1))
    assert np.all((k >= -127) & (k <= 127))
    codes = e2m1_encode(blk / np.ldexp(1.0, k)[..., None])   # exact: division by a power of two
    return codes.reshape(w.shape), (k + 127).astype(np.uint8)


def dequantize_mxfp4(codes, scales) -> np.ndarray:
    """Exact values (float64) of E2M1 codes [..., R, K] with E8M0 scales [..., R, K/32]."""
    v = e2m1_decode(codes)
    K = v.shape[-1]
    k = np.asarray(scales, dtype=np.int64) - 127
    blk = v.reshape(*v.shape[:-1], K // MX_BLOCK, MX_BLOCK) * np.ldexp(1.0, k)[..., None]
    return blk.reshape(v.shape)


def pack_e2m1(codes) -> np.ndarray:
    """Two codes per byte along the last axis, the even index in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_e2m1(packed) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def mxfp4_to_e4m3_blocks(codes, scales):
    """FP4 -> FP8 conversion of one matrix [R, K] (R, K multiples of 128): E4M3 codes and one fp32
    scale per 128x128 block, S = 2^(kmax - 6) with kmax over the block's sub-blocks that hold a nonzero
    value. Returns (e4m3 codes, block scales [R/128, K/128], lossless [R/128, K/128] bool: kmax - kmin
    <= 14). Where lossless holds the dequantised values equal the FP4 ones exactly."""
    v = dequantize_mxfp4(codes, scales)
    R, K = v.shape
    k = np.asarray(scales, dtype=np.int64) - 127                       # [R, K/32]
    nz = np.abs(e2m1_decode(codes)).reshape(R, K // 32, 32).max(axis=2) > 0
    kb = np.where(nz, k, -10 ** 6).reshape(R // 128, 128, K // 128, 4)
    kmax = kb.max(axis=(1, 3))
    kmin = np.where(nz, k, 10 ** 6).reshape(R // 128, 128, K // 128, 4).min(axis=(1, 3))
    empty = kmax < -10 ** 5
    kmax = np.where(empty, 6, kmax)
    S = np.ldexp(1.0, kmax - 6)
    lossless = empty | (kmax - kmin <= LOSSLESS_SPAN)
    scaled = v / np.repeat(np.repeat(S, 128, axis=0), 128, axis=1)
    assert np.all(np.abs(scaled) <= E4M3_MAX)
    return e4m3_encode(scaled), S.astype(np.float32), lossless
