"""Pins of the backward oracle (oracle/backward.py): central finite differences of the forward oracle on a
small layer, a full cross-check against torch autograd over an independent torch forward, and the gate
Jacobian's invariants."""
import numpy as np
import pytest
import torch

import oracle
from moe_inputs import get_config


def _inputs(cfg, seed=0):
    rng = np.random.default_rng(seed)
    f = lambda *s, sc=1.0: rng.standard_normal(s) * sc
    N, Ns, d, I, T = cfg.n_routed, cfg.n_shared, cfg.d, cfg.inter, cfg.T
    return dict(u=f(T, d), centroids=f(N, d, sc=0.05), bias=rng.uniform(-0.01, 0.01, N),
                w_gate_up=f(N, 2 * I, d, sc=0.05), w_down=f(N, d, I, sc=0.05),
                s_gate_up=f(Ns, 2 * I, d, sc=0.05), s_down=f(Ns, d, I, sc=0.05))


CFG = dict(T=6, gemm="f32")


def _loss(cfg, inp, R):
    return float((oracle.layer_forward(cfg, inp)["out"] * R).sum())


def test_finite_differences():
    """dL/dp for L = sum(out * R) at sampled entries of every parameter and of u, against central
    differences of the forward oracle (selection unchanged by the perturbation)."""
    cfg = get_config("c1", **CFG)
    inp = _inputs(cfg, 1)
    R = np.random.default_rng(2).standard_normal((cfg.T, cfg.d))
    g = oracle.layer_backward(cfg, inp, R)
    idx0 = g["route"]["idx"]
    grads = dict(u=g["du"], centroids=g["d_centroids"], w_gate_up=g["d_w_gate_up"], w_down=g["d_w_down"],
                 s_gate_up=g["d_s_gate_up"], s_down=g["d_s_down"])
    rng = np.random.default_rng(3)
    for name, gr in grads.items():
        x = inp[name]
        picks = [tuple(rng.integers(0, n) for n in x.shape) for _ in range(5)]
        if name in ("w_gate_up", "w_down", "centroids"):    # an expert some token selected
            picks = [(int(idx0[0, 0]),) + p[1:] for p in picks]
        for p in picks:
            eps = 1e-5
            old = x[p]
            x[p] = old + eps
            lp, ip = _loss(cfg, inp, R), oracle.route(inp["u"], inp["centroids"], inp["bias"], cfg.n_groups,
                                                       cfg.topk_groups, cfg.group_topn, cfg.topk)["idx"]
            x[p] = old - eps
            lm, im = _loss(cfg, inp, R), oracle.route(inp["u"], inp["centroids"], inp["bias"], cfg.n_groups,
                                                       cfg.topk_groups, cfg.group_topn, cfg.topk)["idx"]
            x[p] = old
            assert np.array_equal(ip, idx0) and np.array_equal(im, idx0), (name, p)
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - gr[p]) <= 1e-6 * max(1.0, abs(fd)), (name, p, fd, gr[p])


def _torch_forward(cfg, inp, idx):
    """An independent torch forward of eq. (12)-(15) for a fixed selection idx, in fp64."""
    t = {k: torch.tensor(v, dtype=torch.float64, requires_grad=k != "bias") for k, v in inp.items()}
    u, cent = t["u"], t["centroids"]
    s = torch.sigmoid(u @ cent.T)
    sel = torch.gather(s, 1, torch.as_tensor(idx))
    gate = sel / sel.sum(dim=1, keepdim=True)
    out = u.clone()
    I = cfg.inter

    def ffn(a, wgu, wd):
        return torch.nn.functional.silu(a @ wgu[:I].T) * (a @ wgu[I:].T) @ wd.T

    for s_ in range(cfg.n_shared):
        out = out + ffn(u, t["s_gate_up"][s_], t["s_down"][s_])
    for k in range(cfg.topk):
        rows = []
        for tok in range(cfg.T):
            e = int(idx[tok, k])
            rows.append(ffn(u[tok:tok + 1], t["w_gate_up"][e], t["w_down"][e]))
        out = out + gate[:, k:k + 1] * torch.cat(rows)
    return out, t


@pytest.mark.parametrize("seed", [0, 1])
def test_against_torch_autograd(seed):
    cfg = get_config("c1", T=16, gemm="f32")
    inp = _inputs(cfg, seed)
    R = np.random.default_rng(seed + 10).standard_normal((cfg.T, cfg.d))
    g = oracle.layer_backward(cfg, inp, R)
    out, t = _torch_forward(cfg, inp, g["route"]["idx"])
    (out * torch.tensor(R)).sum().backward()
    pairs = dict(u="du", centroids="d_centroids", w_gate_up="d_w_gate_up", w_down="d_w_down",
                 s_gate_up="d_s_gate_up", s_down="d_s_down")
    for k, mine in pairs.items():
        ref = t[k].grad.numpy()
        assert np.allclose(g[mine], ref, rtol=1e-10, atol=1e-12), k
    assert np.allclose(oracle.layer_forward(cfg, inp)["out"], out.detach().numpy(), rtol=1e-12, atol=1e-12)


def test_gate_backward_invariants():
    """Gates are scale-invariant in s (g(ls) = g(s)), so sum_k s_k ds_k = 0; with K = 1 the gate is the
    constant 1 and ds = 0; a d_gate equal on every slot gives ds = 0 (the gates sum to one)."""
    rng = np.random.default_rng(5)
    s = rng.uniform(0.05, 0.95, (20, 16))
    idx = np.stack([rng.choice(16, 4, replace=False) for _ in range(20)])
    dg = rng.standard_normal((20, 4))
    ds = oracle.gate_backward(s, idx, dg)
    assert np.allclose((np.take_along_axis(s, idx, axis=1) * ds).sum(axis=1), 0, atol=1e-12)
    assert np.all(oracle.gate_backward(s, idx[:, :1], dg[:, :1]) == 0)
    assert np.allclose(oracle.gate_backward(s, idx, np.ones((20, 4)) * 3.0), 0, atol=1e-12)


# ------------------------------------------------------------------ FP8 recipe

def test_requant_cols_pow2():
    """The 128x1 re-tiling: per (128-row block of a segment, column) one power-of-two scale with every value an
    E4M3 value times it and the block's largest magnitude in [224, 448] scale units; 128-row-aligned segments
    agree with the 1x128 quantiser on the transpose; blocks restart at each segment; idempotent; error within
    half an E4M3 step."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((556, 256)) * np.exp(rng.standard_normal((1, 256)))
    off = [0, 300, 300, 556]                                  # an empty segment, blocks of 128, 128, 44 and 128, 128
    r = oracle.requant_cols_pow2(x, off)
    e4m3_values = np.unique(np.abs(oracle.e4m3_decode(np.arange(256, dtype=np.uint8))))
    e4m3_values = e4m3_values[np.isfinite(e4m3_values)]
    for b0, b1 in [(0, 128), (128, 256), (256, 300), (300, 428), (428, 556)]:
        blk, xb = r[b0:b1], x[b0:b1]
        for c in (0, 77, 255):
            s = 2.0 ** np.ceil(np.log2(np.abs(xb[:, c]).max().astype(np.float32) / np.float32(448.0)))
            assert np.isin(np.abs(blk[:, c]) / s, e4m3_values).all()
            assert 224 <= np.abs(blk[:, c]).max() / s <= 448
            step = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(xb[:, c]) / s, 2.0 ** -6))) - 3) * s
            assert np.all(np.abs(blk[:, c] - xb[:, c]) <= 0.5 * step + 1e-300)
    aligned = oracle.requant_cols_pow2(x[:256], [0, 256])
    c_, s_ = oracle.quantize_tiles(x[:256].T, pow2=True)
    assert np.array_equal(aligned, oracle.dequantize_tiles(c_, s_).T)
    assert np.array_equal(oracle.requant_cols_pow2(r, off), r)
    # the block [256, 300) ends its segment: the rows after it (next segment) do not enter its scale
    y = x.copy()
    y[300:] *= 1e6
    assert np.array_equal(oracle.requant_cols_pow2(y, off)[:300], r[:300])


def _expert(seed, n=200, d=256, I=128):
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((n, d))
    wgu = oracle.quantize_blocks(rng.standard_normal((2 * I, d)) * 0.05)
    wd = oracle.quantize_blocks(rng.standard_normal((d, I)) * 0.05)
    dy = rng.standard_normal((n, d))
    return a, wgu, wd, dy


def test_ffn_backward_fp8_reduces_to_exact(monkeypatch):
    """With every activation quantisation replaced by the identity, the FP8 backward is the exact backward of
    the same (block-quantised) weights: each GEMM takes the right operands."""
    import oracle.backward as ob
    a, wgu, wd, dy = _expert(0)
    wgu64, wd64 = oracle.dequantize_blocks(*wgu), oracle.dequantize_blocks(*wd)
    monkeypatch.setattr(ob, "_q1x128", lambda x: np.asarray(x, np.float64))
    monkeypatch.setattr(ob, "requant_cols_pow2", lambda x, off: np.asarray(x, np.float64))
    monkeypatch.setattr(ob, "quantize_tiles", lambda x, pow2=False: (np.asarray(x, np.float64), None))
    monkeypatch.setattr(ob, "dequantize_tiles", lambda c, s: c)
    got = ob.ffn_backward_fp8(a, *wgu, *wd, dy)
    ref = oracle.ffn_backward(a, wgu64, wd64, dy)
    for g, r_ in zip(got, ref):
        np.testing.assert_allclose(g, r_, rtol=1e-12, atol=1e-12)


def test_ffn_backward_fp8_error_size():
    """The quantised backward stays within E4M3-sized relative error of the exact one (and is not exact)."""
    a, wgu, wd, dy = _expert(1)
    got = oracle.ffn_backward_fp8(a, *wgu, *wd, dy)
    ref = oracle.ffn_backward(a, oracle.dequantize_blocks(*wgu), oracle.dequantize_blocks(*wd), dy)
    for name, g, r_ in zip(("da", "dW_gate_up", "dW_down"), got, ref):
        rel = np.linalg.norm(g - r_) / np.linalg.norm(r_)
        assert 1e-3 < rel < 0.08, (name, rel)


def test_round_bf16():
    """The oracle's bf16 rounding (of the combine backward's output) equals torch's cast on wide-range values."""
    rng = np.random.default_rng(4)
    x = (rng.standard_normal(50000) * np.exp(rng.standard_normal(50000) * 6)).astype(np.float32)
    x[:4] = [0.0, -0.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8]               # exact ties round to even
    ref = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    assert np.array_equal(oracle.round_bf16(x), ref)
