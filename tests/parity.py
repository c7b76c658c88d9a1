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


# ---------------------------------------------------------------- tiled weight layouts
# The libraries' E4M3 and MXFP4 weight codes come in tiled layouts (documented with moe_quantize_weights
# and moe_quantize_weights_mxfp4 in include/moe.h). These NumPy transforms rebuild them from plain
# row-major codes, so tests can feed oracle-quantised weights to the kernels and compare the quantisers.

def tile_rows(R: int, gate_up: bool) -> np.ndarray:
    """[ntiles, 256] matrix row held by each tile row (>= R: padding)."""
    nt = -(-R // 256)
    rw = np.arange(256)
    rows = np.empty((nt, 256), dtype=np.int64)
    for t in range(nt):
        if gate_up:
            j = (rw >> 5) & 3
            hc = 128 * t + 64 * (rw >> 7) + 32 * (j & 1) + (rw & 31)
            rows[t] = np.where(j >= 2, R // 2 + hc, hc)
        else:
            rows[t] = 256 * t + rw
    return rows


def _gather_tiles(x, R, gate_up, fill):
    rows = tile_rows(R, gate_up)
    out = np.full(rows.shape + x.shape[1:], fill, dtype=x.dtype)
    valid = rows < R
    out[valid] = x[rows[valid]]
    return out


def tile_e4m3(codes, gate_up: bool) -> np.ndarray:
    """E4M3 codes [R, K] -> flat tiled codes: per tile and 64-wide K step a 16 KB block, row rw at 64 rw,
    16-byte quarter c at 16 (c ^ ((rw >> 2) & 3))."""
    R, K = codes.shape
    c = _gather_tiles(np.asarray(codes, dtype=np.uint8), R, gate_up, 0)           # [nt, 256, K]
    nt = c.shape[0]
    src = c.reshape(nt, 256, K // 64, 4, 16)
    out = np.zeros((nt, K // 64, 256, 4, 16), dtype=np.uint8)
    rw = np.arange(256)
    swz = (rw >> 2) & 3
    for q in range(4):
        out[:, :, rw, q ^ swz, :] = src[:, :, :, q, :].transpose(0, 2, 1, 3)
    return out.reshape(-1)


def tile_mxfp4(codes, scales, gate_up: bool, pack):
    """MXFP4 codes [R, K] (one per value) and E8M0 scales [R, K/32] -> flat tiled codes (per tile and 64-wide
    K step an 8 KB block, row rw at 32 rw, 16-byte half k at 16 (k ^ ((rw >> 3) & 1)), two codes per byte)
    and flat tiled scales ([tile][K/128][4][256]). pack: the two-per-byte packing of the codes."""
    R, K = codes.shape
    c = _gather_tiles(np.asarray(codes, dtype=np.uint8), R, gate_up, 0)
    sc = _gather_tiles(np.asarray(scales, dtype=np.uint8), R, gate_up, 127)
    nt = c.shape[0]
    packed = pack(c).reshape(nt, 256, K // 64, 2, 16)
    out = np.zeros((nt, K // 64, 256, 2, 16), dtype=np.uint8)
    rw = np.arange(256)
    swz = (rw >> 3) & 1
    for k16 in (0, 1):
        out[:, :, rw, k16 ^ swz, :] = packed[:, :, :, k16, :].transpose(0, 2, 1, 3)
    return out.reshape(-1), np.ascontiguousarray(sc.reshape(nt, 256, K // 128, 4).transpose(0, 2, 3, 1)).reshape(-1)
