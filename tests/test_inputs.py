"""The seeded synthetic workloads have the shapes and statistics they claim (CPU)."""
import numpy as np
import torch

import oracle
from moe_inputs import get_config, generate, generate_tokens


def test_shapes_and_dtypes():
    for name in ("c1", "c2"):
        cfg = get_config(name)
        inp = generate(cfg, "cpu", with_weights=False)
        assert inp["u"].shape == (cfg.T, cfg.d) and inp["u"].dtype == cfg.torch_dtype
        assert inp["centroids"].shape == (cfg.n_routed, cfg.d)
        assert inp["bias"].dtype == torch.float32 and inp["bias"].abs().max() <= 0.01


def test_seeded_and_step_dependent():
    cfg = get_config("c1")
    a = generate_tokens(cfg, "cpu", 0)
    assert torch.equal(a, generate_tokens(cfg, "cpu", 0))
    assert not torch.equal(a, generate_tokens(cfg, "cpu", 1))


def test_v3_centroids_give_near_uniform_load():
    cfg = get_config("c3", T=2048)
    inp = generate(cfg, "cpu", with_weights=False)
    norms = inp["centroids"].float().norm(dim=1)
    assert torch.allclose(norms, torch.full_like(norms, 0.02 * cfg.d ** 0.5), rtol=1e-2)
    r = oracle.route(inp["u"], inp["centroids"], inp["bias"], cfg.n_groups, cfg.topk_groups, cfg.group_topn,
                     cfg.topk)
    mean = cfg.T * cfg.topk / cfg.n_routed
    assert r["load"].max() < 2.0 * mean and r["load"].min() > 0.3 * mean


def test_decode_workload_popularity_is_zipf():
    """Selection frequency by popularity rank follows rank^-1.1 (head capped at 0.45)."""
    cfg = get_config("c5", T=4096)
    inp = generate(cfg, "cpu", with_weights=False)
    r = oracle.route(inp["u"], inp["centroids"], inp["bias"], 1, 1, 2, cfg.topk)
    p = np.sort(r["load"] / cfg.T)[::-1]
    assert 0.38 < p[0] < 0.5
    ranks = np.arange(1, len(p) + 1)
    sel = slice(4, 120)
    slope = np.polyfit(np.log(ranks[sel]), np.log(np.maximum(p[sel], 1e-6)), 1)[0]
    assert -1.4 < slope < -0.8, slope
    # a 256-token step leaves many experts empty
    r256 = oracle.route(inp["u"][:256], inp["centroids"], inp["bias"], 1, 1, 2, cfg.topk)
    assert 60 < int((r256["load"] == 0).sum()) < 250
