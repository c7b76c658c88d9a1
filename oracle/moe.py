"""DeepSeekMoE layer forward, written out plainly in NumPy (TEST INFRASTRUCTURE).

Source of every step: "DeepSeek_V3_Report: Annotation" (the translated V3
report), section "DeepSeekMoE with Auxiliary-Loss-Free Load Balancing":

* eq. (15): affinity s_{i,t} = Sigmoid(u_t^T e_i);
* eq. (16): selection uses s_{i,t} + b_i, the bias never enters a gate value;
* eq. (14), (13): g'_{i,t} = s_{i,t} for the selected experts, and the gate is
  g'_{i,t} divided by the sum of the selected g';
* eq. (12): h'_t = u_t + sum of the shared FFNs + sum_i g_{i,t} FFN_i(u_t);
* the step-end rule of the same section: an overloaded expert's bias drops
  by gamma, an underloaded one's rises by gamma;
* section "Node-Limited Routing": a token reaches at most M groups, chosen by
  the sum of the highest affinities of the experts in each group;
* section "No Token-Dropping": every token keeps all K selected experts.

The FFN is SwiGLU (SwiGLU paragraph of the same page, beta = 1), followed by
the down projection. The fp8 variant follows the sections "Fine-Grained
Quantization", "Increasing Accumulation Precision" and "Online Quantization":
1x128 activation tiles, 128x128 weight blocks, one fp32 scale each, computed
from the current max-abs.

Readings taken where the pages leave a step open are listed where they apply
(selection precision, tie order, group score size, bias-update equality case,
quantisation scale form).
"""
from __future__ import annotations

import numpy as np

from .e4m3 import E4M3_MAX, e4m3_decode, e4m3_encode

F32 = np.float32


def _f64(x) -> np.ndarray:
    """Widen an array or tensor (fp32 / bf16 / fp64) exactly to fp64."""
    if hasattr(x, "detach"):  # torch tensor (bf16 has no numpy dtype)
        import torch
        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _f32(x) -> np.ndarray:
    if hasattr(x, "detach"):
        import torch
        return x.detach().to("cpu", torch.float32).numpy()
    return np.asarray(x, dtype=F32)


# --------------------------------------------------------------------------
# Routing: eq. (13)-(16) and node-limited routing
# --------------------------------------------------------------------------

def affinity(u, centroids) -> np.ndarray:
    """eq. (15): s[t, i] = 1 / (1 + exp(-u_t . e_i)), in fp64."""
    z = _f64(u) @ _f64(centroids).T
    return 1.0 / (1.0 + np.exp(-z))


def route(u, centroids, bias, n_groups: int, topk_groups: int, group_topn: int, topk: int,
          scores=None):
    """Biased, group-limited top-K selection with gates from the raw affinities.

    Reading of the selection precision: the pages keep the gating module in
    its original precision (FP8 framework, "Mixed Precision Framework"), so
    the selection compares fp32 values: s32 = fl32(s), s'32 = fl32(s32 + b).
    The gates use the fp64 affinities.

    Group score (node-limited routing): sum of the ``group_topn`` largest s'
    of the group, added in fp32 from the largest down. The M groups with the
    highest scores are kept; then the K experts with the highest s' inside
    them are selected. Ties go to the lower group / expert index.

    Returns a dict with ``idx`` [T,K] (ascending expert id), ``gate`` [T,K]
    fp64, ``load`` [N_r] int64, and diagnostics: ``s`` (fp64), ``sb32``,
    ``kept_groups`` [T,M], ``k_gap`` (fp64 gap between the K-th and (K+1)-th
    biased scores among the allowed experts) and ``m_gap`` (gap between the
    M-th and (M+1)-th group scores; +inf when every group is kept).
    """
    s = affinity(u, centroids) if scores is None else _f64(scores)
    T, N = s.shape
    G, M, K = n_groups, topk_groups, topk
    S = N // G
    b32 = _f32(bias)
    s32 = s.astype(F32)
    sb32 = (s32 + b32).astype(F32)                      # one fp32 rounding
    sb64 = s + b32.astype(np.float64)

    allowed = np.ones((T, N), dtype=bool)
    kept = np.tile(np.arange(G), (T, 1))
    m_gap = np.full(T, np.inf)
    if G > 1 and M < G:
        grp = sb32.reshape(T, G, S)
        top = -np.sort(-grp, axis=2)[:, :, :group_topn]   # descending
        gs = top[:, :, 0].astype(F32)
        for j in range(1, group_topn):
            gs = (gs + top[:, :, j]).astype(F32)
        order = np.argsort(-gs, axis=1, kind="stable")      # ties: lower group first
        kept = np.sort(order[:, :M], axis=1)
        gsd = np.take_along_axis(gs, order, axis=1).astype(np.float64)
        m_gap = gsd[:, M - 1] - gsd[:, M]
        allowed = np.zeros((T, G), dtype=bool)
        np.put_along_axis(allowed, kept, True, axis=1)
        allowed = np.repeat(allowed, S, axis=1)

    masked = np.where(allowed, sb32, -np.inf)
    order = np.argsort(-masked, axis=1, kind="stable")      # ties: lower expert first
    sel = order[:, :K]
    idx = np.sort(sel, axis=1)
    sb64m = np.where(allowed, sb64, -np.inf)
    srt = -np.sort(-sb64m, axis=1)
    k_gap = srt[:, K - 1] - srt[:, K] if N > K else np.full(T, np.inf)

    s_sel = np.take_along_axis(s, idx, axis=1)
    gate = s_sel / s_sel.sum(axis=1, keepdims=True)          # eq. (13) over raw s
    load = np.bincount(idx.ravel(), minlength=N).astype(np.int64)
    return dict(idx=idx.astype(np.int64), gate=gate, load=load, s=s, sb32=sb32,
                kept_groups=kept, k_gap=k_gap, m_gap=m_gap)


# --------------------------------------------------------------------------
# Permutation (the one-GPU form of the dispatch)
# --------------------------------------------------------------------------

def permute(idx, n_routed: int):
    """Stable counting sort of the (token, slot) pairs by expert.

    Rows are ordered by expert, then by token ("No Token-Dropping": all T*K
    pairs get a row). Returns ``offsets`` [N_r+1], ``perm_token`` [T*K]
    (token of each row) and ``row_of`` [T*K] (row of pair t*K + k).
    """
    idx = np.asarray(idx, dtype=np.int64)
    T, K = idx.shape
    load = np.bincount(idx.ravel(), minlength=n_routed)
    offsets = np.zeros(n_routed + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(load)
    perm_token = np.empty(T * K, dtype=np.int64)
    row_of = np.empty(T * K, dtype=np.int64)
    fill = offsets[:-1].copy()
    for t in range(T):                    # ascending token order keeps it stable
        for k in range(K):
            e = idx[t, k]
            r = fill[e]
            fill[e] += 1
            perm_token[r] = t
            row_of[t * K + k] = r
    return offsets, perm_token, row_of


# --------------------------------------------------------------------------
# Expert FFN: SwiGLU then the down projection
# --------------------------------------------------------------------------

def silu(x):
    """Swish with beta = 1: x * sigmoid(x)."""
    return x / (1.0 + np.exp(-x))


def swiglu_ffn(a, w_gate_up, w_down) -> np.ndarray:
    """y = (SiLU(a W_g^T) * (a W_u^T)) W_d^T in fp64.

    w_gate_up [2I, d] holds the gate rows then the up rows; w_down [d, I].
    """
    a = _f64(a)
    wgu = _f64(w_gate_up)
    I = wgu.shape[0] // 2
    gate = a @ wgu[:I].T
    up = a @ wgu[I:].T
    h = silu(gate) * up
    return h @ _f64(w_down).T


# --------------------------------------------------------------------------
# fp8: online 1x128 / 128x128 quantisation and the quantised FFN
# --------------------------------------------------------------------------

def _quantize_groups(x32: np.ndarray):
    """Quantise each row of x32 [n, g] (one scaling group per row).

    Reading of the scale form (the pages give only "from the current
    max-abs"; the 1x128 tile gets one fp32 scale): amax = max |x|; if amax is
    0 the scale is 1 and every code 0; otherwise inv = fl32(448 / amax),
    code = E4M3(fl32(x * inv)) and scale = fl32(amax / 448). Dequantised value
    = decode(code) * scale.
    """
    x32 = np.asarray(x32, dtype=F32)
    amax = np.max(np.abs(x32), axis=1)
    zero = amax == 0
    safe = np.where(zero, F32(1), amax).astype(F32)
    inv = (F32(E4M3_MAX) / safe).astype(F32)
    scaled = (x32 * inv[:, None]).astype(F32)
    codes = e4m3_encode(scaled)
    codes[zero] = 0
    scale = np.where(zero, F32(1), (safe / F32(E4M3_MAX)).astype(F32)).astype(F32)
    return codes, scale


def _quantize_groups_pow2(x32: np.ndarray):
    """Quantise each row of x32 [n, g] with a power-of-two scale.

    "DeepSeek_V3_Report: Annotation", FP8 framework, "Low-Precision
    Communication": the activations quantised before the MoE up-projection
    (and dispatched) take scaling factors that are integral powers of 2.
    Reading: the scale is the smallest power of two s with fl32(amax / 448)
    <= s, so no element exceeds 448 after scaling; s = 1 and codes 0 when
    amax = 0. x / s is exact, code = E4M3(x / s).
    """
    x32 = np.asarray(x32, dtype=F32)
    amax = np.max(np.abs(x32), axis=1)
    zero = amax == 0
    v = (np.where(zero, F32(1), amax).astype(F32) / F32(E4M3_MAX)).astype(F32).astype(np.float64)
    m, e = np.frexp(v)                                   # v = m * 2**e, 0.5 <= m < 1
    scale = np.ldexp(1.0, np.where(m == 0.5, e - 1, e))  # 2**ceil(log2 v)
    scale = np.where(zero, 1.0, scale)
    codes = e4m3_encode((x32.astype(np.float64) / scale[:, None]).astype(F32))
    codes[zero] = 0
    return codes, scale.astype(F32)


def quantize_tiles(x, pow2: bool = False) -> tuple:
    """1x128 tiles along the last axis: x [R, C] -> codes [R, C] uint8, scales [R, C/128] fp32
    (pow2: power-of-two scales, see _quantize_groups_pow2)."""
    x32 = _f32(x)
    R, C = x32.shape
    assert C % 128 == 0
    q = _quantize_groups_pow2 if pow2 else _quantize_groups
    codes, scale = q(x32.reshape(R * (C // 128), 128))
    return codes.reshape(R, C), scale.reshape(R, C // 128)


def dequantize_tiles(codes, scale) -> np.ndarray:
    R, C = codes.shape
    v = e4m3_decode(codes).reshape(R, C // 128, 128) * np.asarray(scale, np.float64)[:, :, None]
    return v.reshape(R, C)


def quantize_blocks(w) -> tuple:
    """128x128 blocks: w [R, C] -> codes [R, C] uint8, scales [R/128, C/128] fp32."""
    w32 = _f32(w)
    R, C = w32.shape
    assert R % 128 == 0 and C % 128 == 0
    blocks = w32.reshape(R // 128, 128, C // 128, 128).transpose(0, 2, 1, 3).reshape(-1, 128 * 128)
    codes, scale = _quantize_groups(blocks)
    codes = codes.reshape(R // 128, C // 128, 128, 128).transpose(0, 2, 1, 3).reshape(R, C)
    return codes, scale.reshape(R // 128, C // 128)


def dequantize_blocks(codes, scale) -> np.ndarray:
    R, C = codes.shape
    v = e4m3_decode(codes).reshape(R // 128, 128, C // 128, 128)
    v = v * np.asarray(scale, np.float64)[:, None, :, None]
    return v.reshape(R, C)


def ffn_fp8(a, wgu_codes, wgu_scale, wd_codes, wd_scale, return_h=False, pow2_input=False):
    """The SwiGLU FFN with the V3 fp8 recipe, in fp64 over the quantised values.

    a [n, d] (fp32/bf16 values) is quantised per 1x128 tile; the weights come
    already quantised per 128x128 block. The product over dequantised values
    in fp64 equals the pages' per-128-chunk promotion sum_c s_a,c s_w,c
    sum_{k in c} q_a q_w exactly: each chunk sum is a sum of at most 128
    products of two E4M3 values, exactly representable in fp64. The SwiGLU
    output is rounded to fp32 and quantised per 1x128 tile along I before the
    down projection (the activations of every fp8 GEMM are quantised online).
    pow2_input: the up-projection input takes power-of-two scales (the
    dispatched-activation variant); H keeps fp32 scales.
    """
    return ffn_quantised_acts(a, dequantize_blocks(wgu_codes, wgu_scale), dequantize_blocks(wd_codes, wd_scale),
                               return_h, pow2_input)


def ffn_quantised_acts(a, wgu, wd, return_h=False, pow2_input=False):
    """SwiGLU FFN over exact weight values wgu [2I, d], wd [d, I] (float64), with the activations of both
    GEMMs quantised online per 1x128 tile (E4M3, fp32 scales; the input optionally with power-of-two
    scales) and the products summed exactly in fp64."""
    a_codes, a_scale = quantize_tiles(a, pow2=pow2_input)
    a_dq = dequantize_tiles(a_codes, a_scale)
    I = wgu.shape[0] // 2
    gate = a_dq @ wgu[:I].T
    up = a_dq @ wgu[I:].T
    h32 = (silu(gate) * up).astype(F32)
    h_codes, h_scale = quantize_tiles(h32)
    y = dequantize_tiles(h_codes, h_scale) @ wd.T
    if return_h:
        return y, dict(h32=h32, h_codes=h_codes, h_scale=h_scale, a_codes=a_codes, a_scale=a_scale)
    return y


def ffn_mxfp4(a, wgu_codes, wgu_scales, wd_codes, wd_scales, return_h=False, pow2_input=False):
    """The SwiGLU FFN with MXFP4 expert weights ("DeepSeek V3 / V4 Infra", V4 post-training FP4 QAT
    section): weights given as E2M1 codes [2I, d] / [d, I] (one per value) with E8M0 scales per 32
    consecutive K values ([2I, d/32] / [d, I/32]); activations quantised to E4M3 per 1x128 tile as in the
    fp8 recipe. Products of an E2M1 and an E4M3 value and their sums are exact in fp64."""
    from .mxfp4 import dequantize_mxfp4
    return ffn_quantised_acts(a, dequantize_mxfp4(wgu_codes, wgu_scales), dequantize_mxfp4(wd_codes, wd_scales),
                               return_h, pow2_input)


def expert_ffn(a, w_gate_up, w_down, gemm: str = "bf16", wq=None, pow2_input: bool = False):
    """FFN of one expert on rows a, in the precision recipe of ``gemm``.

    ``gemm`` "f32" / "bf16": exact fp64 arithmetic on the stored values.
    ``gemm`` "fp8": the weights are quantised per 128x128 block (unless
    ``wq`` = (gu_codes, gu_scale, d_codes, d_scale) is given) and the FFN runs
    through :func:`ffn_fp8` (``pow2_input``: power-of-two scales on its input);
    ``gemm`` "mxfp4": MXFP4 weights (``wq`` as from quantize_mxfp4) through
    :func:`ffn_mxfp4`.
    """
    if gemm == "mxfp4":
        from .mxfp4 import quantize_mxfp4
        if wq is None:
            wq = (*quantize_mxfp4(w_gate_up), *quantize_mxfp4(w_down))
        return ffn_mxfp4(a, *wq, pow2_input=pow2_input)
    if gemm != "fp8":
        return swiglu_ffn(a, w_gate_up, w_down)
    if wq is None:
        gq, gs = quantize_blocks(w_gate_up)
        dq, ds = quantize_blocks(w_down)
    else:
        gq, gs, dq, ds = wq
    return ffn_fp8(a, gq, gs, dq, ds, pow2_input=pow2_input)


# --------------------------------------------------------------------------
# Combine (eq. 12) and the step-end bias update
# --------------------------------------------------------------------------

def combine(u, y_routed, row_of, gate, y_shared=None) -> np.ndarray:
    """eq. (12): out[t] = u[t] + sum_s y_shared[s, t] + sum_k gate[t,k] * y_routed[row_of[t,k]].

    y_shared is [N_s, T, d] (or None). Everything in fp64.
    """
    u = _f64(u)
    T, d = u.shape
    gate = np.asarray(gate, np.float64)
    K = gate.shape[1]
    y = _f64(y_routed)
    out = u.copy()
    if y_shared is not None:
        out += _f64(y_shared).reshape(-1, T, d).sum(axis=0)
    rows = np.asarray(row_of, np.int64).reshape(T, K)
    for k in range(K):
        out += gate[:, k:k + 1] * y[rows[:, k]]
    return out


def bias_update(bias, load, T: int, K: int, gamma: float = 0.001) -> np.ndarray:
    """Step-end update: b_i - gamma if expert i is overloaded, b_i + gamma if underloaded.

    Reading: "overloaded" means more than the batch mean T*K/N_r token-expert
    pairs (the V3 essay's "more than the average"), "underloaded" fewer; an
    expert exactly at the mean keeps its bias. The comparison is done on
    integers (load * N_r against T * K), the update in fp32 with gamma as fp32.
    """
    b = _f32(bias).copy()
    load = np.asarray(load, np.int64)
    N = b.shape[0]
    g = F32(gamma)
    over = load * N > T * K
    under = load * N < T * K
    b[over] = (b[over] - g).astype(F32)
    b[under] = (b[under] + g).astype(F32)
    return b


def balance_stats(scores, topk_idx, seq_len: int, alpha: float = 1e-4):
    """Complementary sequence-wise balance statistics, eq. (17)-(20) of
    "DeepSeek_V3_Report: Annotation", section "Complementary Sequence-Wise
    Auxiliary Loss", for each run of seq_len consecutive tokens (the last run
    may be shorter, T_s tokens):

        f_i = N_r / (K_r T_s) * #{t in the run : expert i selected for t}
        s'_{i,t} = s_{i,t} / sum_j s_{j,t}
        P_i = (1 / T_s) * sum_t s'_{i,t}
        L_Bal = alpha * sum_i f_i P_i

    Reading: the selection indicator of eq. (18) is the routing's own choice
    (topk_idx, after the bias and the group limit) rather than a plain top-K
    of the raw s. scores [T, N_r] are the affinities s (any dtype, widened to
    fp64). Returns f [n_seq, N_r], P [n_seq, N_r], loss [n_seq] in fp64.
    """
    s = np.asarray(scores, np.float64)
    idx = np.asarray(topk_idx, np.int64)
    T, N = s.shape
    K = idx.shape[1]
    n_seq = -(-T // seq_len)
    f = np.zeros((n_seq, N))
    P = np.zeros((n_seq, N))
    loss = np.zeros(n_seq)
    for q in range(n_seq):
        lo, hi = q * seq_len, min(T, (q + 1) * seq_len)
        Ts = hi - lo
        cnt = np.bincount(idx[lo:hi].ravel(), minlength=N)[:N]
        f[q] = N * cnt / (K * Ts)
        P[q] = (s[lo:hi] / s[lo:hi].sum(axis=1, keepdims=True)).sum(axis=0) / Ts
        loss[q] = alpha * np.sum(f[q] * P[q])
    return f, P, loss


# --------------------------------------------------------------------------
# Whole layer (small configs; large ones are checked per expert / per token)
# --------------------------------------------------------------------------

def layer_forward(cfg, inputs, shared_fp8: bool = True, pow2_input: bool = False):
    """One layer forward plus the step-end bias update, for a config object.

    ``inputs``: u, centroids, bias, w_gate_up [N_r,2I,d], w_down [N_r,d,I],
    s_gate_up [N_s,2I,d], s_down [N_s,d,I]. For fp8 configs the shared
    expert also runs in fp8 (``shared_fp8``); its output and the combine stay
    in high precision. ``pow2_input``: the fp8 up-projection inputs take
    power-of-two tile scales (see _quantize_groups_pow2).
    """
    r = route(inputs["u"], inputs["centroids"], inputs["bias"], cfg.n_groups, cfg.topk_groups,
              cfg.group_topn, cfg.topk)
    offsets, perm_token, row_of = permute(r["idx"], cfg.n_routed)
    u64 = _f64(inputs["u"])
    y = np.zeros((cfg.T * cfg.topk, cfg.d))
    for e in range(cfg.n_routed):
        lo, hi = offsets[e], offsets[e + 1]
        if hi > lo:
            y[lo:hi] = expert_ffn(u64[perm_token[lo:hi]], inputs["w_gate_up"][e], inputs["w_down"][e], cfg.gemm,
                                  pow2_input=pow2_input)
    sgemm = cfg.gemm if (cfg.gemm != "fp8" or shared_fp8) else "bf16"
    ysh = np.stack([expert_ffn(u64, inputs["s_gate_up"][s], inputs["s_down"][s], sgemm, pow2_input=pow2_input)
                    for s in range(cfg.n_shared)]) if cfg.n_shared else None
    out = combine(u64, y, row_of, r["gate"], ysh)
    new_bias = bias_update(inputs["bias"], r["load"], cfg.T, cfg.topk, cfg.gamma)
    return dict(route=r, offsets=offsets, perm_token=perm_token, row_of=row_of,
                y=y, y_shared=ysh, out=out, bias=new_bias)
