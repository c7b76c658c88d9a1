"""Seeded synthetic inputs for the DeepSeekMoE layer forward.

This module is shared by the CPU oracle and the GPU path. It only draws
random tensors of the right shapes and distributions; it holds none of the
layer's arithmetic (no affinities, no selection, no quantisation).

Shapes and distributions follow the five workloads of this project:

* ``c1`` tiny fp32 layer: T=64, d=256, 16 routed experts in 4 groups of 4,
  top-2 limited to 2 groups, 1 shared expert, I=128.
* ``c2`` mid bf16 layer: T=4096, d=2048, 64 experts in 8 groups of 8,
  top-6 limited to 3 groups, 2 shared experts, I=1408.
* ``c3`` DeepSeek-V3-shaped bf16 layer: T=8192, d=7168, 256 experts in 8
  groups of 32, top-8 limited to 4 groups, 1 shared expert, I=2048
  (DeepSeek-V3 report, hyper-parameter section: 1 shared + 256 routed
  experts, 8 active, expert intermediate size 2048, 4-node limit).
* ``c4`` the same V3 shape with the expert GEMMs in fp8 e4m3.
* ``c5`` DeepSeek-V4-Pro-shaped decode batch in fp8: T=256, d=7168, 384
  experts, top-6 with no group limit, I=3072, Zipf-skewed popularity and
  10 steps of the bias update (V3/V4 infra digest, model paragraph).

Every tensor comes from its own torch generator, seeded from
``(seed, config, tensor, expert, step)`` through a NumPy ``SeedSequence``.
Values are drawn in fp32 and rounded to the storage dtype with
round-to-nearest-even (torch's cast). Generation on a CUDA device and on the
CPU give different (equally valid) draws; every consumer that needs the same
values as another reads one materialised copy.
"""
from __future__ import annotations

import math
import os
from dataclasses import dataclass, field, replace
from typing import Dict, Optional

import numpy as np
import torch

__all__ = ["MoEConfig", "CONFIGS", "get_config", "generate", "generate_tokens",
           "generate_expert", "generate_output_grad", "derive_seed", "zipf_norms"]


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int                 # tokens in the batch
    d: int                 # hidden size
    n_routed: int          # N_r
    n_groups: int          # G (expert groups; one per "node")
    topk_groups: int       # M, groups kept per token
    group_topn: int        # experts summed per group score
    topk: int              # K_r
    n_shared: int          # N_s
    inter: int             # SwiGLU intermediate size I
    gemm: str              # "f32" | "bf16" | "fp8" | "mxfp4" (E4M3 activations, MXFP4 weights)
    act: str               # storage dtype of u, centroids, weights: "f32" | "bf16"
    steps: int = 1         # bias-update steps
    gamma: float = 0.001   # bias update speed
    centroids: str = "iid"     # "iid" | "renorm" | "zipf"
    bias_init: str = "uniform"  # "uniform" U(-0.01, 0.01) | "zero"
    w_std: float = 0.02
    batch_invariant: int = 0    # 1: per-token results independent of the batch (router K split fixed by d)
    description: str = ""

    @property
    def group_size(self) -> int:
        return self.n_routed // self.n_groups

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.act == "f32" else torch.bfloat16

    def ffn_flops(self) -> float:
        """6*d*I per token-expert pair (gate, up and down projections)."""
        pairs = self.T * (self.topk + self.n_shared)
        return 6.0 * self.d * self.inter * pairs

    def router_flops(self) -> float:
        return 2.0 * self.T * self.d * self.n_routed


CONFIGS: Dict[str, MoEConfig] = {
    "c1": MoEConfig("c1", T=64, d=256, n_routed=16, n_groups=4, topk_groups=2, group_topn=2,
                    topk=2, n_shared=1, inter=128, gemm="f32", act="f32",
                    description="tiny fp32 MoE layer"),
    "c2": MoEConfig("c2", T=4096, d=2048, n_routed=64, n_groups=8, topk_groups=3, group_topn=2,
                    topk=6, n_shared=2, inter=1408, gemm="bf16", act="bf16",
                    description="mid bf16 MoE layer"),
    "c3": MoEConfig("c3", T=8192, d=7168, n_routed=256, n_groups=8, topk_groups=4, group_topn=2,
                    topk=8, n_shared=1, inter=2048, gemm="bf16", act="bf16", centroids="renorm",
                    description="DeepSeek-V3-shaped bf16 MoE layer"),
    "c4": MoEConfig("c4", T=8192, d=7168, n_routed=256, n_groups=8, topk_groups=4, group_topn=2,
                    topk=8, n_shared=1, inter=2048, gemm="fp8", act="bf16", centroids="renorm",
                    description="DeepSeek-V3-shaped MoE layer, fp8 e4m3 expert GEMMs"),
    "c5": MoEConfig("c5", T=256, d=7168, n_routed=384, n_groups=1, topk_groups=1, group_topn=2,
                    topk=6, n_shared=1, inter=3072, gemm="fp8", act="bf16", steps=10,
                    centroids="zipf", bias_init="zero",
                    description="DeepSeek-V4-Pro-shaped decode batch, fp8, Zipf(1.1) popularity"),
}

_CFG_ID = {"c1": 1, "c2": 2, "c3": 3, "c4": 3, "c5": 5}  # c4 reuses c3's draws
_TENSOR_ID = {"u": 1, "centroids": 2, "bias": 3, "w_gate_up": 4, "w_down": 5,
              "s_gate_up": 6, "s_down": 7, "d_out": 8}


def get_config(name: str, **overrides) -> MoEConfig:
    cfg = CONFIGS[name]
    return replace(cfg, **overrides) if overrides else cfg


def derive_seed(seed: int, cfg: MoEConfig, tensor: str, expert: int = 0, step: int = 0) -> int:
    """A 63-bit seed for one (config, tensor, expert, step) substream."""
    cid = _CFG_ID.get(cfg.name, 99)
    ss = np.random.SeedSequence([seed, cid, _TENSOR_ID[tensor], expert, step])
    return int(ss.generate_state(2, dtype=np.uint32).astype(np.uint64).dot(
        np.array([1, 1 << 32], dtype=np.uint64)) & np.uint64((1 << 63) - 1))


def _gen(device, s: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(s)
    return g


def _normal(shape, std, dtype, device, s):
    x = torch.randn(shape, generator=_gen(device, s), device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


_ZIPF_TABLE = os.path.join(os.path.dirname(__file__), "zipf_norms_c5.txt")


def zipf_norms(n: int) -> np.ndarray:
    """Per-expert centroid norms (by popularity rank) for the Zipf-skewed workload.

    Read from the stored table that ``calibrate_zipf.py`` writes. If the table
    is missing, fall back to a plain power law of the rank.
    """
    if os.path.exists(_ZIPF_TABLE):
        v = np.loadtxt(_ZIPF_TABLE, dtype=np.float64)
        if v.shape == (n,):
            return v
    r = np.arange(1, n + 1, dtype=np.float64)
    return 1.5 * r ** (-0.35)


def _centroids(cfg: MoEConfig, device, seed: int) -> torch.Tensor:
    n, d = cfg.n_routed, cfg.d
    s = derive_seed(seed, cfg, "centroids")
    e = torch.randn((n, d), generator=_gen(device, s), device=device, dtype=torch.float32)
    if cfg.centroids == "iid":
        e.mul_(cfg.w_std)
    elif cfg.centroids == "renorm":
        # iid rows rescaled to the common norm w_std*sqrt(d): equal-norm
        # centroids make every expert equally likely by symmetry.
        e.mul_((cfg.w_std * math.sqrt(d)) / e.norm(dim=1, keepdim=True))
    elif cfg.centroids == "zipf":
        # rows of norm sigma_rank; the popularity rank of each expert is a
        # seeded permutation so popular experts are scattered over the index range.
        norms = torch.tensor(zipf_norms(n), dtype=torch.float32, device=device)
        perm = torch.from_numpy(np.random.default_rng(
            derive_seed(seed, cfg, "centroids", expert=1)).permutation(n)).to(device)
        e.mul_(norms[perm].unsqueeze(1) / e.norm(dim=1, keepdim=True))
    else:
        raise ValueError(cfg.centroids)
    return e.to(cfg.torch_dtype)


def generate_tokens(cfg: MoEConfig, device="cpu", step: int = 0, seed: int = 0) -> torch.Tensor:
    """u [T, d] ~ N(0, 1) in the activation dtype (fresh draw per step)."""
    return _normal((cfg.T, cfg.d), 1.0, cfg.torch_dtype, device, derive_seed(seed, cfg, "u", step=step))


def generate_output_grad(cfg: MoEConfig, device="cpu", step: int = 0, seed: int = 0) -> torch.Tensor:
    """d_out [T, d] ~ N(0, 1) in the activation dtype: the gradient of a loss w.r.t. the layer output."""
    return _normal((cfg.T, cfg.d), 1.0, cfg.torch_dtype, device, derive_seed(seed, cfg, "d_out", step=step))


def generate_expert(cfg: MoEConfig, e: int, shared: bool = False, device="cpu", seed: int = 0):
    """(w_gate_up [2I, d], w_down [d, I]) of routed expert e or shared expert e.

    w_gate_up holds the gate rows [0, I) then the up rows [I, 2I); both are
    K-contiguous (row-major with d as the fast axis). Entries ~ N(0, w_std^2).
    """
    tg, td = ("s_gate_up", "s_down") if shared else ("w_gate_up", "w_down")
    wg = _normal((2 * cfg.inter, cfg.d), cfg.w_std, cfg.torch_dtype, device, derive_seed(seed, cfg, tg, expert=e))
    wd = _normal((cfg.d, cfg.inter), cfg.w_std, cfg.torch_dtype, device, derive_seed(seed, cfg, td, expert=e))
    return wg, wd


def generate(cfg: MoEConfig, device="cpu", seed: int = 0, with_weights: bool = True) -> Dict[str, torch.Tensor]:
    """All inputs of one layer forward at step 0.

    Returns u [T,d], centroids [N_r,d], bias [N_r] (fp32), and, if requested,
    w_gate_up [N_r,2I,d], w_down [N_r,d,I], s_gate_up [N_s,2I,d], s_down [N_s,d,I].
    """
    out = {
        "u": generate_tokens(cfg, device, 0, seed),
        "centroids": _centroids(cfg, device, seed),
    }
    if cfg.bias_init == "uniform":
        b = torch.rand((cfg.n_routed,), generator=_gen(device, derive_seed(seed, cfg, "bias")),
                       device=device, dtype=torch.float32)
        out["bias"] = (b * 0.02 - 0.01).contiguous()
    else:
        out["bias"] = torch.zeros((cfg.n_routed,), dtype=torch.float32, device=device)
    if with_weights:
        I, d = cfg.inter, cfg.d
        wgu = torch.empty((cfg.n_routed, 2 * I, d), dtype=cfg.torch_dtype, device=device)
        wdn = torch.empty((cfg.n_routed, d, I), dtype=cfg.torch_dtype, device=device)
        for e in range(cfg.n_routed):
            wgu[e], wdn[e] = generate_expert(cfg, e, False, device, seed)
        sgu = torch.empty((cfg.n_shared, 2 * I, d), dtype=cfg.torch_dtype, device=device)
        sdn = torch.empty((cfg.n_shared, d, I), dtype=cfg.torch_dtype, device=device)
        for e in range(cfg.n_shared):
            sgu[e], sdn[e] = generate_expert(cfg, e, True, device, seed)
        out.update(w_gate_up=wgu, w_down=wdn, s_gate_up=sgu, s_down=sdn)
    return out
