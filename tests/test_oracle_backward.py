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
