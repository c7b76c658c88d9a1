"""Pin P11 (CPU): the limited-precision accumulator of the oracle.

"DeepSeek_V3_Report: Annotation", FP8 framework, section "Increasing
Accumulation Precision": with about 14 bits kept during FP8 accumulation, a
GEMM of two random K = 4096 matrices shows a maximum relative error near 2%;
promoting the partial sums to FP32 every N_C = 128 elements removes most of
it. Checked here: the bit-keeping step against closed forms, the accumulator
against an exact GEMM when no bits are dropped, the printed ~2% and its
removal by promotion.
"""
import numpy as np

import oracle


def test_keep_bits_closed_forms():
    x = np.array([1.0 + 2.0 ** -20, -(1.0 + 2.0 ** -20), 3.0, 2.0 ** -30 * (1 + 2.0 ** -13), 0.0, 1.5 * 2.0 ** 40])
    got = oracle.keep_bits(x, 14)
    assert np.array_equal(got, [1.0, -1.0, 3.0, 2.0 ** -30 * (1 + 2.0 ** -13), 0.0, 1.5 * 2.0 ** 40])
    rng = np.random.default_rng(1)
    v = rng.standard_normal(10000) * 10.0 ** rng.integers(-5, 6, 10000)
    k = oracle.keep_bits(v, 14)
    m, _ = np.frexp(k)
    assert np.all(m * 2 ** 14 == np.trunc(m * 2 ** 14))          # at most 14 significant bits
    assert np.all(np.abs(k) <= np.abs(v)) and np.all(np.sign(k) == np.sign(v))   # toward zero
    assert np.all(np.abs(v - k) < 2.0 ** -13 * np.abs(v))
    assert np.array_equal(oracle.keep_bits(v, 53), v)


def test_accumulator_without_loss_is_the_exact_gemm():
    rng = np.random.default_rng(2)
    a = rng.integers(-8, 9, (16, 256)).astype(np.float64)
    b = rng.integers(-8, 9, (8, 256)).astype(np.float64)
    assert np.array_equal(oracle.limited_precision_gemm(a, b, bits=53), a @ b.T)
    assert np.array_equal(oracle.limited_precision_gemm(a, b, bits=53, promote_every=128), a @ b.T)


def _e4m3_random(rng, shape):
    return oracle.e4m3_decode(oracle.e4m3_encode(rng.standard_normal(shape).astype(np.float32)))


def test_k4096_error_near_two_percent_and_promotion_removes_it():
    rng = np.random.default_rng(3)
    a, b = _e4m3_random(rng, (48, 4096)), _e4m3_random(rng, (48, 4096))
    exact = a @ b.T
    rel = lambda x: np.abs(x - exact).max() / np.abs(exact).max()
    limited = rel(oracle.limited_precision_gemm(a, b))
    promoted = rel(oracle.limited_precision_gemm(a, b, promote_every=128))
    print(f"K=4096: limited accumulation {limited:.3e}, promoted every 128 {promoted:.3e}")
    assert 0.01 < limited < 0.03                       # "near 2%"
    assert promoted < 0.001                            # well below once promoted every 128
    # the error grows with K: a 512-long product loses less
    ex512 = a[:, :512] @ b[:, :512].T
    l512 = np.abs(oracle.limited_precision_gemm(a[:, :512], b[:, :512]) - ex512).max() / np.abs(ex512).max()
    assert l512 < limited
