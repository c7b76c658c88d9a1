"""Pins of the oracle's routing, permutation and bias update (CPU only).

Each test checks the oracle against something other than itself: brute-force
enumeration, a library top-k, or an invariant that the DeepSeek-V3 pages state
("DeepSeek_V3_Report: Annotation", section "DeepSeekMoE with
Auxiliary-Loss-Free Load Balancing", eq. (13)-(16); sections "Node-Limited
Routing" and "No Token-Dropping").
"""
import itertools
from collections import Counter

import numpy as np
import pytest
import torch

import oracle
from moe_inputs import get_config, generate


def _rand_route_inputs(rng, T, d, N, bias_scale=0.01):
    u = rng.standard_normal((T, d)).astype(np.float32)
    e = (rng.standard_normal((N, d)) * 0.1).astype(np.float32)
    b = rng.uniform(-bias_scale, bias_scale, N).astype(np.float32)
    return u, e, b


def _brute_force(sb32_row, G, S, M, K, topn):
    """Enumerate group subsets, then expert subsets, by summed scores.

    A group's score is the largest sum of ``topn`` of its biased scores: every topn-subset of the group is
    enumerated and the best one by its exact sum is kept; its value is then formed in fp32, adding the
    subset's scores from the largest down (the reading of the selection precision). The M groups with the
    largest summed scores are found by enumerating every M-subset of groups; the K experts by enumerating
    every K-subset of the allowed experts.
    """
    N = G * S
    gsc = []
    for j in range(G):
        vals = [float(v) for v in sb32_row[j * S:(j + 1) * S]]
        best = max(itertools.combinations(range(S), topn), key=lambda c: sum(vals[i] for i in c))
        acc = np.float32(0)
        for v in sorted((vals[i] for i in best), reverse=True):
            acc = np.float32(acc + np.float32(v))
        gsc.append(float(acc))
    if M < G:
        best_groups = max(itertools.combinations(range(G), M), key=lambda c: sum(gsc[j] for j in c))
    else:
        best_groups = tuple(range(G))
    allowed = [i for i in range(N) if i // S in best_groups]
    best = max(itertools.combinations(allowed, K), key=lambda c: sum(float(sb32_row[i]) for i in c))
    return sorted(best), sorted(best_groups)


SMALL_SHAPES = [(4, 4, 2, 2), (4, 4, 2, 3), (3, 4, 2, 4), (4, 3, 3, 5), (2, 4, 1, 3), (4, 4, 4, 3), (1, 8, 1, 3),
                (5, 4, 2, 4), (6, 3, 3, 4)]


@pytest.mark.parametrize("topn", [1, 2, 3, 4])
@pytest.mark.parametrize("G,S,M,K", SMALL_SHAPES)
def test_p4_brute_force_small(G, S, M, K, topn):
    """Selection and kept groups against exhaustive enumeration, for group scores of 1 to 4 terms."""
    if topn > S:
        pytest.skip("group_topn exceeds the group size")
    rng = np.random.default_rng(100 + G * 31 + S * 7 + M * 3 + K + 1000 * topn)
    N = G * S
    u, e, b = _rand_route_inputs(rng, 48, 32, N)
    r = oracle.route(u, e, b, G, M, topn, K)
    for t in range(u.shape[0]):
        if r["m_gap"][t] < 1e-6 or r["k_gap"][t] < 1e-6:
            continue                    # a near-tie: summation order may decide it
        exp_idx, exp_groups = _brute_force(r["sb32"][t], G, S, M, K, topn)
        assert list(r["idx"][t]) == exp_idx, (t, r["idx"][t], exp_idx)
        if M < G and G > 1:
            assert list(r["kept_groups"][t]) == exp_groups


def test_p4_group_score_terms_matter():
    """The number of terms in a group score changes the kept groups: one group holds the single largest
    score, another the larger sum of its top three; topn = 1 keeps the first, topn = 3 the second."""
    sb = np.zeros((1, 8), dtype=np.float32)
    sb[0, :4] = [0.95, 0.10, 0.10, 0.10]       # group 0: max 0.95, top-3 sum 1.15
    sb[0, 4:] = [0.60, 0.55, 0.50, 0.05]       # group 1: max 0.60, top-3 sum 1.65
    z = np.log(sb / (1 - sb)).astype(np.float64)   # logits whose sigmoid gives back sb (bias 0)
    u = z.reshape(1, 8)
    e = np.eye(8)
    b = np.zeros(8, dtype=np.float32)
    r1 = oracle.route(u, e, b, 2, 1, 1, 2)
    r3 = oracle.route(u, e, b, 2, 1, 3, 2)
    assert list(r1["kept_groups"][0]) == [0] and list(r1["idx"][0]) == [0, 1]
    assert list(r3["kept_groups"][0]) == [1] and list(r3["idx"][0]) == [4, 5]
    for topn in (1, 3):
        exp_idx, exp_groups = _brute_force(oracle.route(u, e, b, 2, 1, topn, 2)["sb32"][0], 2, 4, 1, 2, topn)
        assert exp_groups == [0 if topn == 1 else 1]


def test_p4_brute_force_c1_inputs():
    cfg = get_config("c1")
    inp = generate(cfg, "cpu", with_weights=False)
    r = oracle.route(inp["u"], inp["centroids"], inp["bias"], cfg.n_groups, cfg.topk_groups, cfg.group_topn, cfg.topk)
    for t in range(cfg.T):
        exp_idx, _ = _brute_force(r["sb32"][t], cfg.n_groups, cfg.group_size, cfg.topk_groups, cfg.topk, 2)
        assert list(r["idx"][t]) == exp_idx


def test_p1_gates_sum_to_one():
    rng = np.random.default_rng(1)
    u, e, b = _rand_route_inputs(rng, 256, 64, 32)
    r = oracle.route(u, e, b, 4, 2, 2, 6)
    assert np.all(np.abs(r["gate"].sum(axis=1) - 1.0) <= 1e-12)
    assert np.all(r["gate"] > 0) and np.all(r["gate"] < 1)


def test_p2_bias_changes_selection_not_gates():
    rng = np.random.default_rng(2)
    u, e, b = _rand_route_inputs(rng, 512, 64, 32)
    r0 = oracle.route(u, e, b, 4, 2, 2, 4)
    b2 = (b + rng.uniform(-0.02, 0.02, b.shape)).astype(np.float32)
    r1 = oracle.route(u, e, b2, 4, 2, 2, 4)
    same = np.all(r0["idx"] == r1["idx"], axis=1)
    assert same.sum() > 50 and (~same).sum() > 5        # the bias moved some selections
    # where the selection is unchanged, the gates are bit-identical
    assert np.array_equal(r0["gate"][same], r1["gate"][same])


def test_p2_forced_expert_keeps_raw_gate_ratio():
    rng = np.random.default_rng(3)
    u, e, b = _rand_route_inputs(rng, 256, 64, 32)
    forced = 13
    b[forced] = 50.0
    r = oracle.route(u, e, b, 4, 2, 2, 4)
    assert np.all(np.any(r["idx"] == forced, axis=1))
    s = oracle.affinity(u, e)
    slot = np.argmax(r["idx"] == forced, axis=1)
    gf = r["gate"][np.arange(256), slot]
    for k in range(4):
        other = r["idx"][:, k]
        ratio = gf / r["gate"][:, k]
        assert np.allclose(ratio, s[np.arange(256), forced] / s[np.arange(256), other], rtol=1e-12)
    assert np.all(gf < 0.9)      # a huge bias does not turn into a huge gate


def test_p2_constant_shift_of_bias():
    rng = np.random.default_rng(4)
    u, e, b = _rand_route_inputs(rng, 1024, 64, 64)
    r0 = oracle.route(u, e, b, 8, 3, 2, 6)
    r1 = oracle.route(u, e, (b + np.float32(0.125)).astype(np.float32), 8, 3, 2, 6)
    diff = np.any(r0["idx"] != r1["idx"], axis=1)
    near = (r0["k_gap"] < 1e-6) | (r0["m_gap"] < 1e-6)
    assert np.all(near[diff])
    assert np.array_equal(r0["gate"][~diff], r1["gate"][~diff])


def test_p3_at_most_m_groups():
    rng = np.random.default_rng(5)
    u, e, b = _rand_route_inputs(rng, 1024, 64, 64)
    for M in (1, 2, 3):
        r = oracle.route(u, e, b, 8, M, 2, 6 if M > 1 else 4)
        groups = r["idx"] // 8
        n = np.array([len(set(row)) for row in groups])
        assert np.all(n <= M)
        assert np.all(np.isin(groups, r["kept_groups"]).reshape(groups.shape)
                      | True)  # membership checked row-wise below
        for t in range(0, 1024, 97):
            assert set(groups[t]) <= set(r["kept_groups"][t])


def test_p5_reductions_match_library_topk():
    rng = np.random.default_rng(6)
    u, e, b = _rand_route_inputs(rng, 300, 48, 40)
    s32 = torch.from_numpy(oracle.affinity(u, e).astype(np.float32))
    sb = s32 + torch.from_numpy(b)
    ref = torch.sort(torch.topk(sb, 5, dim=1).indices, dim=1).values.numpy()
    for G, M in [(1, 1), (8, 8), (4, 4)]:
        r = oracle.route(u, e, b, G, M, 2, 5)
        assert np.array_equal(r["idx"], ref)
    # b = 0 is eq. (14): plain top-K of the affinities
    r = oracle.route(u, e, np.zeros(40, np.float32), 1, 1, 2, 5)
    ref0 = torch.sort(torch.topk(s32, 5, dim=1).indices, dim=1).values.numpy()
    assert np.array_equal(r["idx"], ref0)


def test_p7_load_histogram():
    rng = np.random.default_rng(7)
    u, e, b = _rand_route_inputs(rng, 700, 32, 24)
    r = oracle.route(u, e, b, 6, 3, 2, 5)
    c = Counter(int(i) for i in r["idx"].ravel())
    assert r["load"].sum() == 700 * 5
    assert all(r["load"][i] == c.get(i, 0) for i in range(24))
    # every token has K distinct experts
    assert all(len(set(row)) == 5 for row in r["idx"])


def test_p8_permutation():
    rng = np.random.default_rng(8)
    T, K, N = 333, 4, 20
    idx = np.sort(np.stack([rng.choice(N, K, replace=False) for _ in range(T)]), axis=1)
    off, perm, row_of = oracle.permute(idx, N)
    assert off[0] == 0 and off[-1] == T * K and np.all(np.diff(off) >= 0)
    assert sorted(row_of.tolist()) == list(range(T * K))          # bijection
    for t in range(T):
        for k in range(K):
            r = row_of[t * K + k]
            assert perm[r] == t
            e = np.searchsorted(off, r, side="right") - 1
            assert e == idx[t, k]
    for e in range(N):
        seg = perm[off[e]:off[e + 1]]
        assert np.all(np.diff(seg) > 0)                            # stable: ascending tokens
        assert len(seg) == int(np.sum(idx == e))


def test_p9_bias_update():
    T, K, N = 64, 2, 16
    mean = T * K // N
    b = np.linspace(-0.01, 0.01, N).astype(np.float32)
    # exactly uniform load: unchanged
    assert np.array_equal(oracle.bias_update(b, np.full(N, mean), T, K), b)
    load = np.array([mean + 1, mean - 1, mean, 0, 2 * mean] + [mean] * (N - 5))
    load[5] += (T * K - load.sum())
    nb = oracle.bias_update(b, load, T, K, 0.001)
    delta = nb.astype(np.float64) - b.astype(np.float64)
    for i in range(N):
        if load[i] > mean:
            assert abs(delta[i] + 0.001) < 1e-8
        elif load[i] < mean:
            assert abs(delta[i] - 0.001) < 1e-8
        else:
            assert delta[i] == 0
    n_over = int(np.sum(load > mean))
    n_under = int(np.sum(load < mean))
    assert abs(delta.sum() - 0.001 * (n_under - n_over)) < 1e-7


def test_c1_route_sanity():
    cfg = get_config("c1")
    inp = generate(cfg, "cpu", with_weights=False)
    r = oracle.route(inp["u"], inp["centroids"], inp["bias"], cfg.n_groups, cfg.topk_groups, cfg.group_topn, cfg.topk)
    assert r["idx"].shape == (64, 2) and r["load"].sum() == 128


# ---------------------------------------------------------------- eq. (17)-(20) balance statistics

def test_balance_stats_closed_forms():
    """Sum f_i = N_r and sum P_i = 1 per sequence; a perfectly balanced selection with equal affinities
    gives f_i = 1, P_i = 1/N_r and L_Bal = alpha; all tokens on the same K experts with all affinity mass
    there gives f = N_r/K on them and L_Bal = alpha * N_r / K."""
    rng = np.random.default_rng(4)
    T, N, K, L = 100, 16, 2, 32
    s = rng.random((T, N))
    idx = np.sort(np.stack([rng.choice(N, K, replace=False) for _ in range(T)]), axis=1)
    f, P, loss = oracle.balance_stats(s, idx, L, alpha=0.5)
    assert f.shape == (4, N) and loss.shape == (4,)
    assert np.allclose(f.sum(axis=1), N) and np.allclose(P.sum(axis=1), 1.0)
    # last run has 4 tokens
    cnt = np.bincount(idx[96:].ravel(), minlength=N)
    assert np.allclose(f[3], N * cnt / (K * 4))
    # perfectly balanced: each token t picks experts {2t mod N, 2t+1 mod N}; equal affinities
    idx_b = np.stack([(2 * np.arange(64)) % N, (2 * np.arange(64) + 1) % N], axis=1)
    fb, Pb, lb = oracle.balance_stats(np.ones((64, N)), idx_b, 64, alpha=1e-4)
    assert np.allclose(fb, 1.0) and np.allclose(Pb, 1.0 / N) and np.allclose(lb, 1e-4)
    # fully collapsed: every token on experts {0, 1}, which hold all the affinity
    sc = np.zeros((32, N)); sc[:, :2] = 0.5
    fc, Pc, lc = oracle.balance_stats(sc, np.tile([0, 1], (32, 1)), 32, alpha=1e-4)
    assert np.allclose(fc[0, :2], N / K) and np.allclose(Pc[0, :2], 0.5) and np.allclose(lc, 1e-4 * N / K)
