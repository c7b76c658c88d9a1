"""Comparison helpers for the GPU-vs-oracle parity tests.

Tolerances (relative L2 per output tensor): 1e-4 for the fp32 workload, 2e-2
for bf16, 1e-2 against the quantisation-emulating oracle for fp8 and for MXFP4
weights (the same E4M3 activations; the oracle sums exact products). Expert
indices, permutation and loads must match exactly, except that a token's
selection may differ where the oracle's K-th and (K+1)-th biased scores (or
M-th and (M+1)-th group scores) are closer than 1e-6; such tokens are counted
and reported.
"""
from __future__ import annotations

import numpy as np
import torch

TOL = {"f32": 1e-4, "bf16": 2e-2, "fp8": 1e-2, "mxfp4": 1e-2}
NEAR_TIE = 1e-6


def np64(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu", torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def npi(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu").numpy().astype(np.int64)
    return np.asarray(t, dtype=np.int64)


def rel_l2(x, ref) -> float:
    x, ref = np64(x), np64(ref)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / (den if den > 0 else 1.0))


def routing_mismatches(gpu_idx, oracle_route) -> np.ndarray:
    """Tokens whose selected set differs; asserts every one is an exempt near-tie."""
    g = npi(gpu_idx)
    o = oracle_route["idx"]
    bad = np.where(np.any(g != o, axis=1))[0]
    near = (oracle_route["k_gap"] < NEAR_TIE) | (oracle_route["m_gap"] < NEAR_TIE)
    not_exempt = bad[~near[bad]]
    assert not_exempt.size == 0, (
        f"{not_exempt.size} tokens select different experts without a near-tie, e.g. token {not_exempt[:5]}: "
        f"gpu {g[not_exempt[:2]]} oracle {o[not_exempt[:2]]} k_gap {oracle_route['k_gap'][not_exempt[:2]]}")
    if bad.size:
        print(f"[parity] {bad.size} near-tie selection flips (exempt) at tokens {bad[:10]}")
    return bad


def report(name: str, value: float, tol: float):
    print(f"[parity] {name}: rel_l2 = {value:.3e} (tol {tol:.0e})")
    assert value <= tol, f"{name}: rel_l2 {value:.3e} > {tol:.0e}"
