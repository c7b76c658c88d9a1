"""Limited-precision accumulation of fp8 GEMMs -- TEST INFRASTRUCTURE ONLY.

"DeepSeek_V3_Report: Annotation", FP8 framework, section "Increasing
Accumulation Precision" (and the matching paragraph of "DeepSeek V3 / V4
Infra", V3 FP8 section, figure 7b): the H800 tensor core keeps only about 14
bits while accumulating FP8 products; a GEMM of two random K = 4096 matrices
then shows a maximum relative error near 2%; copying the partial sums to FP32
registers every N_C = 128 elements removes most of it.

The pages give the bit count and the outcome, not the adder's design. The
reading taken here: the exact products enter the accumulator in groups of
`group` = 4 (one MMA step), and after each addition the running sum keeps
`bits` = 14 significant bits, the rest dropped (truncation toward zero, as
bits shifted out by alignment are lost). This reading reproduces the printed
~2% for random inputs; single-product steps give ~6% and rounding instead of
truncation ~0.2%. With promotion, each 128-element chunk is accumulated that
way from zero and then added into an fp32 accumulator.
"""
from __future__ import annotations

import numpy as np


def keep_bits(x: np.ndarray, bits: int) -> np.ndarray:
    """x with only its `bits` leading significant bits, truncated toward zero."""
    m, e = np.frexp(x)                                    # x = m * 2**e, 0.5 <= |m| < 1
    return np.ldexp(np.trunc(m * 2.0 ** bits) / 2.0 ** bits, e)


def limited_precision_gemm(a: np.ndarray, b: np.ndarray, bits: int = 14, group: int = 4,
                           promote_every: int | None = None) -> np.ndarray:
    """a [M, K] . b [N, K]^T with the accumulator above; promote_every = N_C adds the
    chunk sums into fp32 registers (and restarts the limited accumulator) every N_C
    elements. a and b hold exactly representable values (e.g. decoded E4M3 codes)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    K = a.shape[1]
    assert b.shape[1] == K and K % group == 0
    assert promote_every is None or promote_every % group == 0
    fp32_acc = np.zeros((a.shape[0], b.shape[0]), dtype=np.float32)
    s = np.zeros((a.shape[0], b.shape[0]))
    for k0 in range(0, K, group):
        s = keep_bits(s + a[:, k0:k0 + group] @ b[:, k0:k0 + group].T, bits)
        if promote_every and (k0 + group) % promote_every == 0:
            fp32_acc = fp32_acc + s.astype(np.float32)
            s = np.zeros_like(s)
    return fp32_acc.astype(np.float64) + s
