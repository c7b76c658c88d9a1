"""Pins of the MXFP4 oracle (oracle/mxfp4.py) against the format's published table, brute force,
closed-form bounds and an independent conversion path."""
import numpy as np
import pytest

import oracle

# The OCP Microscaling E2M1 magnitudes, codes 0..7 (sign in bit 3).
E2M1_SPEC = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_decode_matches_spec_table():
    v = oracle.e2m1_decode(np.arange(16))
    assert np.array_equal(v[:8], E2M1_SPEC)
    assert np.array_equal(v[8:], -np.array(E2M1_SPEC))
    assert np.all(np.signbit(v[8:]))


def test_e2m1_encode_brute_force():
    """Nearest value by exhaustive comparison with the 8 magnitudes; exact ties go to the even code;
    beyond 6 saturate; the sign follows the input."""
    rng = np.random.default_rng(0)
    mids = [(a + b) / 2 for a, b in zip(E2M1_SPEC, E2M1_SPEC[1:])]
    x = np.concatenate([rng.uniform(-8, 8, 20000), np.array(E2M1_SPEC), mids, -np.array(mids),
                        [7.0, 100.0, -6.5, 1e-30, -1e-30]])
    codes = oracle.e2m1_encode(x)
    grid = np.array(E2M1_SPEC)
    for xv, c in zip(x, codes):
        a = min(abs(xv), 6.0)
        d = np.abs(grid - a)
        best = np.flatnonzero(d == d.min())
        want = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
        assert (c & 7) == want, (xv, c)
        assert bool(c & 8) == bool(np.signbit(xv)), (xv, c)
    # round trip of every code
    assert np.array_equal(oracle.e2m1_encode(oracle.e2m1_decode(np.arange(16))), np.arange(16))


def test_pack_nibble_order():
    assert np.array_equal(oracle.pack_e2m1(np.array([1, 2, 15, 0], dtype=np.uint8)), [0x21, 0x0F])
    c = np.random.default_rng(1).integers(0, 16, (5, 64)).astype(np.uint8)
    assert np.array_equal(oracle.unpack_e2m1(oracle.pack_e2m1(c)), c)


def test_mx_scale_rule_and_error_bounds():
    """Scale = 2^(floor(log2 amax) - 2): every block max lands in [4, 8) before saturation; the
    dequantised values are within half an E2M1 step of the input (steps 0.5 / 1 / 2 in the binades
    below 2 / 2..4 / 4..8, times the scale), saturating at 6 * scale."""
    rng = np.random.default_rng(2)
    w = (rng.standard_normal((64, 256)) * 10.0 ** rng.integers(-6, 3, (64, 1))).astype(np.float32)
    w[5, 32:64] = 0.0                                   # an all-zero block: scale 2^0, zero codes
    codes, scales = oracle.quantize_mxfp4(w)
    k = scales.astype(np.int64) - 127
    blk = np.abs(w.astype(np.float64)).reshape(64, 8, 32)
    amax = blk.max(axis=2)
    nz = amax > 0
    r = amax[nz] / np.ldexp(1.0, k[nz])
    assert np.all((r >= 4) & (r < 8))
    assert k[5, 1] == 0 and np.all(codes[5, 32:64] == 0)
    deq = oracle.dequantize_mxfp4(codes, scales)
    s = np.repeat(np.ldexp(1.0, k), 32, axis=1)
    a = np.abs(w.astype(np.float64)) / s
    step = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))
    err = np.abs(deq - w) / s
    assert np.all(err <= np.where(a > 6, a - 6, step / 2) + 1e-12)


def _lossless_matrix(rng, span):
    """128x256 weights whose 1x32 sub-block exponents span at most `span` inside each 128x128 block."""
    w = rng.standard_normal((128, 256))
    e = rng.integers(0, span + 1, (128, 8))
    e[0, :] = 0
    e[1, :] = span
    return (w * np.ldexp(1.0, np.repeat(e, 32, axis=1) - 20)).astype(np.float32)


def test_fp4_to_fp8_conversion_is_lossless_within_the_span():
    """Random codes (every E2M1 value, the smallest included) with sub-block exponents spanning exactly
    0, 7 or 14 inside each 128x128 block convert exactly."""
    rng = np.random.default_rng(3)
    for span in (0, 7, 14):
        codes = rng.integers(0, 16, (256, 256)).astype(np.uint8)
        k = rng.integers(-30, -30 + span + 1, (256, 8))
        k[::128, :] = -30            # each block holds both extremes
        k[1::128, :] = -30 + span
        codes[::128, :] = 1          # 0.5 * 2^kmin present
        q8, S, ok = oracle.mxfp4_to_e4m3_blocks(codes, (k + 127).astype(np.uint8))
        assert np.all(ok)
        assert np.array_equal(oracle.dequantize_blocks(q8, S), oracle.dequantize_mxfp4(codes, (k + 127).astype(np.uint8)))
    # quantised Gaussian weights have narrow spans
    codes, scales = oracle.quantize_mxfp4(_lossless_matrix(rng, 8))
    q8, S, ok = oracle.mxfp4_to_e4m3_blocks(codes, scales)
    assert np.all(ok) and np.array_equal(oracle.dequantize_blocks(q8, S), oracle.dequantize_mxfp4(codes, scales))


def test_fp4_to_fp8_conversion_loses_beyond_the_span():
    """Span 15: the smallest sub-block's 0.5 * 2^kmin falls below E4M3's smallest subnormal after the
    block scale and is lost."""
    codes = np.zeros((128, 128), dtype=np.uint8)
    scales = np.full((128, 4), 127, dtype=np.uint8)
    codes[0, 0] = 7                       # 6 * 2^0 in sub-block (0, 0)
    codes[1, 32] = 1                      # 0.5 * 2^-15 in sub-block (1, 1)
    scales[1, 1] = 127 - 15
    q8, S, ok = oracle.mxfp4_to_e4m3_blocks(codes, scales)
    assert not ok[0, 0]
    assert oracle.dequantize_blocks(q8, S)[1, 32] != oracle.dequantize_mxfp4(codes, scales)[1, 32]
    scales[1, 1] = 127 - 14
    q8, S, ok = oracle.mxfp4_to_e4m3_blocks(codes, scales)
    assert ok[0, 0] and oracle.dequantize_blocks(q8, S)[1, 32] == 0.5 * 2.0 ** -14


def test_ffn_mxfp4_equals_fp8_ffn_on_converted_weights():
    """Two independent dequantisation paths: the MXFP4 FFN equals the fp8 FFN fed with the losslessly
    converted E4M3 blocks, bit for bit (both sum exact products in fp64)."""
    rng = np.random.default_rng(4)
    d, I = 256, 128
    wgu = (rng.standard_normal((2 * I, d)) * 0.02).astype(np.float32)
    wd = (rng.standard_normal((d, I)) * 0.02).astype(np.float32)
    gq, gs = oracle.quantize_mxfp4(wgu)
    dq, ds = oracle.quantize_mxfp4(wd)
    g8, gS, gok = oracle.mxfp4_to_e4m3_blocks(gq, gs)
    d8, dS, dok = oracle.mxfp4_to_e4m3_blocks(dq, ds)
    assert np.all(gok) and np.all(dok)
    a = rng.standard_normal((40, d)).astype(np.float32)
    y4 = oracle.ffn_mxfp4(a, gq, gs, dq, ds)
    y8 = oracle.ffn_fp8(a, g8, gS, d8, dS)
    assert np.array_equal(y4, y8)
    # and near the unquantised FFN (E2M1 weights: about 10% per weight)
    ref = oracle.swiglu_ffn(a, wgu, wd)
    rel = np.linalg.norm(y4 - ref) / np.linalg.norm(ref)
    assert 0.05 < rel < 0.3


@pytest.mark.parametrize("shape", [(3, 128, 256), (2, 256, 128)])
def test_quantize_mxfp4_batched_matches_per_matrix(shape):
    w = np.random.default_rng(5).standard_normal(shape).astype(np.float32)
    codes, scales = oracle.quantize_mxfp4(w)
    assert codes.shape == shape and scales.shape == shape[:-1] + (shape[-1] // 32,)
    for i in range(shape[0]):
        c, s = oracle.quantize_mxfp4(w[i])
        assert np.array_equal(c, codes[i]) and np.array_equal(s, scales[i])
