"""Backward of the DeepSeekMoE layer, written out plainly in NumPy fp64 (TEST INFRASTRUCTURE).

Sources: "DeepSeek_V3_Report: Annotation", eq. (12)-(16) (the layer the
gradients run through) and the FP8 framework's sections on the mixed precision
framework and low-precision activations: the three GEMMs of a linear layer
(forward, input gradient, weight gradient), weight gradients kept in high
precision, the gating module in its original precision, and the SwiGLU inputs
cached in the forward with the SwiGLU output recomputed in the backward.

Readings (the pages give the recipe, not the derivatives):

* the expert selection is a fixed, non-differentiable choice: the gradient of
  the loss reaches the affinities only through the gates of the selected
  experts, g_k = s_k / sum_j s_j (eq. (13)-(14)); the bias b_i, used for the
  selection only, gets no gradient;
* s_i = Sigmoid(u . e_i) (eq. (15)) passes it on to u and to the centroids e_i;
* every expert FFN is y = (SiLU(a W_g^T) * (a W_u^T)) W_d^T with
  SiLU'(x) = sigma(x) (1 + x (1 - sigma(x)));
* the layer output is u + sum_s FFN_s(u) + sum_k g_k FFN_k(u) (eq. (12)), so
  the residual passes d_out through unchanged.

The FP8 form (``ffn_backward_fp8``, ``layer_backward`` with gemm "fp8") follows
the FP8 framework's recipe for the three GEMMs of each linear layer: Dgrad
takes its activation gradient quantised per 1x128 tile along its K and the
forward's 128x128 weight blocks; the SwiGLU inputs are cached as 1x128 E4M3
tiles and the SwiGLU output recomputed from them; Wgrad contracts over the
tokens, so its operands are re-tiled to 128x1 (one scale per 128 consecutive
rows of a column, the "transposed re-quantisation"). Readings: the 128-row
blocks start at each expert's first row (the last one is shorter); the re-tiled
operands take power-of-two scales (the pages' rule for activations converted
from 1x128 to 128x1 tiles, so the conversion adds no scale rounding); the
re-tiled token operand of dW_gate_up is the forward's dequantised 1x128 input;
the combine backward's output dy is rounded to bf16 (the pages keep the combine
in BF16 in both passes), the other GEMM outputs and SwiGLU backward values stay
unrounded (the GEMMs output FP32).
"""
from __future__ import annotations

import numpy as np

from .e4m3 import e4m3_decode
from .moe import (_f64, _quantize_groups_pow2, dequantize_blocks, dequantize_tiles, expert_ffn, permute,
                  quantize_blocks, quantize_tiles, route)


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def ffn_backward(a, w_gate_up, w_down, dy):
    """One expert: a [n, d], w_gate_up [2I, d], w_down [d, I], dy [n, d] -> (da [n, d], dW_gate_up [2I, d],
    dW_down [d, I]), all fp64, from the forward's SwiGLU inputs G = a W_g^T, U = a W_u^T (recomputed here as
    the cache holds them)."""
    a, wgu, wd, dy = _f64(a), _f64(w_gate_up), _f64(w_down), _f64(dy)
    I = wgu.shape[0] // 2
    G = a @ wgu[:I].T
    U = a @ wgu[I:].T
    sg = _sigmoid(G)
    silu = G * sg
    h = silu * U
    dh = dy @ wd                                       # dL/dh = dL/dy . W_d
    d_wd = dy.T @ h                                    # dL/dW_d
    dG = dh * U * sg * (1.0 + G * (1.0 - sg))          # SiLU' = sigma (1 + x (1 - sigma))
    dU = dh * silu
    d_wgu = np.concatenate([dG.T @ a, dU.T @ a])       # dL/dW_g, dL/dW_u
    da = dG @ wgu[:I] + dU @ wgu[I:]
    return da, d_wgu, d_wd


def requant_cols_pow2(x, offsets):
    """The 1x128 -> 128x1 re-tiling of a Wgrad operand: x [n, C] -> the dequantised values of x quantised
    to E4M3 with one power-of-two scale per (128 consecutive rows of a segment, column), fp64. Segments are
    [offsets[e], offsets[e + 1]); blocks start at each segment's first row."""
    x = _f64(x)
    out = np.zeros_like(x)
    for e in range(len(offsets) - 1):
        for b0 in range(int(offsets[e]), int(offsets[e + 1]), 128):
            b1 = min(b0 + 128, int(offsets[e + 1]))
            codes, scale = _quantize_groups_pow2(x[b0:b1].T)        # one group per column
            out[b0:b1] = (e4m3_decode(codes) * scale.astype(np.float64)[:, None]).T
    return out


def round_bf16(x):
    """Round to the nearest bf16 value (ties to even), via fp32 (exact for the fp32 products that feed it)."""
    b = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32)).view(np.uint32).astype(np.uint64)
    b = ((b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)
    return b.view(np.float32).astype(np.float64)


def _q1x128(x):
    """Dequantised values of x quantised per 1x128 tile along its rows (fp32 scales)."""
    return dequantize_tiles(*quantize_tiles(x))


def ffn_backward_fp8(a, wgu_codes, wgu_scale, wd_codes, wd_scale, dy, pow2_input=False):
    """One expert with the FP8 recipe: a [n, d] (the forward input, quantised per 1x128 tile), weights as
    128x128-block E4M3 codes and scales, dy [n, d] -> (da, dW_gate_up, dW_down), fp64 over the quantised
    values (each sum of E4M3 products is exact in fp64, as in the forward oracle).

    Forward recomputed: G, U over the quantised operands, cached as 1x128 E4M3 tiles of [G, U].
    Dgrad: dh = Q(dy) W_d and da = Q([dG, dU]) W_gate_up (Q: 1x128 tiles along K = d and 2I).
    SwiGLU backward from the cached (dequantised) G, U; h recomputed from them.
    Wgrad: dW_d = R(dy)^T R(h), dW_gate_up = R([dG, dU])^T R(a_q) (R: 128x1 re-tiling, requant_cols_pow2).
    """
    wgu, wd = dequantize_blocks(wgu_codes, wgu_scale), dequantize_blocks(wd_codes, wd_scale)
    a_q = dequantize_tiles(*quantize_tiles(a, pow2=pow2_input))
    I = wgu.shape[0] // 2
    gu = _q1x128(np.concatenate([a_q @ wgu[:I].T, a_q @ wgu[I:].T], axis=1))   # the FP8 SwiGLU-input cache
    G, U = gu[:, :I], gu[:, I:]
    sg = _sigmoid(G)
    h = G * sg * U                                     # recomputed SwiGLU output
    dy = _f64(dy)
    dh = _q1x128(dy) @ wd
    dgu = np.concatenate([dh * U * sg * (1.0 + G * (1.0 - sg)), dh * G * sg], axis=1)
    da = _q1x128(dgu) @ wgu
    rows = [0, a_q.shape[0]]
    d_wd = requant_cols_pow2(dy, rows).T @ requant_cols_pow2(h, rows)
    d_wgu = requant_cols_pow2(dgu, rows).T @ requant_cols_pow2(a_q, rows)
    return da, d_wgu, d_wd


def gate_backward(scores, idx, d_gate):
    """Gates g_k = s_k / S (S = sum of the selected s) -> dL/ds on the selected experts: [T, K] fp64,
    ds_k = (dg_k - sum_j g_j dg_j) / S."""
    s = np.take_along_axis(_f64(scores), np.asarray(idx, dtype=np.int64), axis=1)
    S = s.sum(axis=1, keepdims=True)
    g = s / S
    dg = _f64(d_gate)
    return (dg - (g * dg).sum(axis=1, keepdims=True)) / S


def layer_backward(cfg, inputs, d_out, pow2_input: bool = False):
    """Gradients of the layer output w.r.t. u, the centroids and the expert weights, for the selection the
    forward makes (bf16 / fp32 GEMM recipe: exact fp64 over the stored values; cfg.gemm "fp8": the FP8
    recipe of ffn_backward_fp8, the forward outputs from the fp8 forward oracle).

    Returns dict(du [T, d], d_centroids [N_r, d], d_w_gate_up [N_r, 2I, d], d_w_down [N_r, d, I],
    d_s_gate_up [N_s, 2I, d], d_s_down [N_s, d, I], d_gate [T, K], dz [T, K]) plus the forward's route.
    """
    fp8 = cfg.gemm == "fp8"
    u = _f64(inputs["u"])
    cent = _f64(inputs["centroids"])
    dO = _f64(d_out)
    T, d = u.shape
    K, N, Ns = cfg.topk, cfg.n_routed, cfg.n_shared
    r = route(inputs["u"], inputs["centroids"], inputs["bias"], cfg.n_groups, cfg.topk_groups, cfg.group_topn, K)
    idx, gate = r["idx"], r["gate"]
    offsets, perm_token, row_of = permute(idx, N)
    du = dO.copy()                                     # residual
    d_gate = np.zeros((T, K))
    d_wgu = np.zeros((N,) + tuple(inputs["w_gate_up"].shape[1:]))
    d_wd = np.zeros((N,) + tuple(inputs["w_down"].shape[1:]))
    for e in range(N):
        lo, hi = offsets[e], offsets[e + 1]
        if hi == lo:
            continue
        toks = perm_token[lo:hi]
        slot = np.array([int(np.flatnonzero(idx[t] == e)[0]) for t in toks])
        a = u[toks]
        dy = gate[toks, slot][:, None] * dO[toks]
        if fp8:
            dy = round_bf16(dy)                                    # the combine backward's bf16 output
            wq = quantize_blocks(inputs["w_gate_up"][e]) + quantize_blocks(inputs["w_down"][e])
            y = expert_ffn(a, None, None, "fp8", wq, pow2_input)
            da, dg_w, dd_w = ffn_backward_fp8(a, *wq, dy, pow2_input)
        else:
            wgu, wd = _f64(inputs["w_gate_up"][e]), _f64(inputs["w_down"][e])
            I = wgu.shape[0] // 2
            h = (a @ wgu[:I].T) * _sigmoid(a @ wgu[:I].T) * (a @ wgu[I:].T)
            y = h @ wd.T
            da, dg_w, dd_w = ffn_backward(a, wgu, wd, dy)
        d_gate[toks, slot] = (dO[toks] * y).sum(axis=1)           # d out / d g_k = y_k
        d_wgu[e] = dg_w
        d_wd[e] = dd_w
        np.add.at(du, toks, da)
    d_sgu = np.zeros((Ns,) + tuple(inputs["s_gate_up"].shape[1:])) if Ns else None
    d_sd = np.zeros((Ns,) + tuple(inputs["s_down"].shape[1:])) if Ns else None
    for s_ in range(Ns):
        if fp8:
            wq = quantize_blocks(inputs["s_gate_up"][s_]) + quantize_blocks(inputs["s_down"][s_])
            da, dg_w, dd_w = ffn_backward_fp8(u, *wq, dO, pow2_input)
        else:
            da, dg_w, dd_w = ffn_backward(u, inputs["s_gate_up"][s_], inputs["s_down"][s_], dO)
        d_sgu[s_], d_sd[s_] = dg_w, dd_w
        du += da
    ds = gate_backward(r["s"], idx, d_gate)                        # [T, K] on the selected experts
    s_sel = np.take_along_axis(r["s"], idx, axis=1)
    dz = ds * s_sel * (1.0 - s_sel)                                 # through s = Sigmoid(z)
    d_cent = np.zeros_like(cent)
    for k in range(K):
        du += dz[:, k:k + 1] * cent[idx[:, k]]
        np.add.at(d_cent, idx[:, k], dz[:, k:k + 1] * u)
    return dict(du=du, d_centroids=d_cent, d_w_gate_up=d_wgu, d_w_down=d_wd, d_s_gate_up=d_sgu, d_s_down=d_sd,
                d_gate=d_gate, dz=dz, route=r, offsets=offsets, perm_token=perm_token, row_of=row_of)
