"""GPU parity of each libmoe call and of the whole layer against the CPU oracle.

Every call is fed inputs that the generator or the oracle produced (never the
output of another GPU call), so a near-tie routing flip cannot cascade. The
small workloads are checked element by element; the V3-shaped one on its full
routing and permutation and on sampled experts / tokens for the FFN.
"""
import numpy as np
import pytest
import torch

import oracle
from moe_inputs import get_config, generate, generate_expert, generate_tokens
from mixture_experts_layer_gate_amd import binding as B
from mixture_experts_layer_gate_amd import MoELayer
from gpu_common import i32, inputs, oracle_ffn_rows, oracle_route, oracle_wq, workspace
from parity import TOL, np64, npi, rel_l2, report, routing_mismatches, tile_e4m3

pytestmark = pytest.mark.gpu

DEV = "cuda"


_i32 = i32
_inputs = inputs
_oracle_route = oracle_route
_ws = workspace


ROUTE_CASES = [
    ("c1", {}),
    ("c2", {}),
    ("c2", dict(n_groups=1, topk_groups=1)),           # no group limit
    ("c2", dict(topk_groups=8)),                        # every group kept
    ("c2", dict(T=1000, n_groups=4, topk_groups=1, topk=3, group_topn=3)),  # ragged T, 3-term group score
    ("c2", dict(n_routed=96, n_groups=8, topk_groups=3)),   # 3 experts per lane, 4-lane groups
    ("c2", dict(n_routed=68, n_groups=4, topk_groups=2)),   # 17-expert groups: the LDS form of the selection
    ("c2", dict(n_routed=18, n_groups=3, topk_groups=2, topk=4)),   # N_r % 4 != 0: the four-wave logits kernel
    ("c3", {}),
    ("c5", {}),                                             # 384 experts, no group limit: 6 per lane
    # the supported maxima: 1024 experts in 64 groups, top-16 of 8 groups, 4-term group scores; ragged T
    ("c2", dict(T=300, d=256, inter=128, n_routed=1024, n_groups=64, topk_groups=8, group_topn=4, topk=16)),
    # a 4096-token batch with 512 experts in 64 groups, top-16 of 8 groups, 4-term group scores (8 per lane)
    ("c2", dict(d=256, inter=128, n_routed=512, n_groups=64, topk_groups=8, group_topn=4, topk=16)),
]


@pytest.mark.parametrize("name,over", ROUTE_CASES)
def test_route(name, over):
    cfg, inp = _inputs(name, **over)
    sh = B.moe_shape.of(cfg)
    T, K, N = cfg.T, cfg.topk, cfg.n_routed
    idx = torch.empty((T, K), dtype=torch.int32, device=DEV)
    gate = torch.empty((T, K), dtype=torch.float32, device=DEV)
    load = torch.full((N,), -7, dtype=torch.int32, device=DEV)
    scores = torch.empty((T, N), dtype=torch.float32, device=DEV)
    B.moe_route(sh, inp["u"], inp["centroids"], inp["bias"], idx, gate, load, scores, _ws(cfg))
    torch.cuda.synchronize()
    r = _oracle_route(cfg, inp)
    ds = np.abs(np64(scores) - r["s"]).max()
    print(f"[parity] {name} {over}: max |s_gpu - s_oracle| = {ds:.2e}")
    assert ds < 1e-5
    bad = routing_mismatches(idx, r)
    gi = npi(idx)
    assert np.all(np.diff(gi, axis=1) > 0), "topk_idx must be ascending per token"
    assert np.array_equal(npi(load), np.bincount(gi.ravel(), minlength=N))
    if bad.size == 0:
        assert np.array_equal(npi(load), r["load"])
    ok = np.ones(T, dtype=bool)
    ok[bad] = False
    report(f"{name} gates", rel_l2(np64(gate)[ok], r["gate"][ok]), 1e-5)
    # groups touched per token never exceed M
    S = N // cfg.n_groups
    assert max(len(set(row)) for row in (gi // S)) <= cfg.topk_groups


def test_route_token_rows_past_4gib():
    """u of 4 GiB (T = 2048 rows of d = 2^20 bf16): the router cuts its token range into launches whose
    rows stay within 32-bit byte offsets (1792 + 256 tokens here). Tokens on both sides of the cut and at the end
    against the oracle; the load histogram against the bincount of every selection. Seeded inputs made on the
    device: u ~ N(0, 1), centroids ~ N(0, (1.7 / sqrt(d))^2) (logits of about the V3 spread), bias ~ U(-0.01, 0.01).
    Affinities and gates to the same 1e-5 as at the V3 shape, although each fp32 sum runs over 2^20 products."""
    T, d, N, G, M, K = 2048, 1 << 20, 16, 4, 2, 2
    cfg = get_config("c2", T=T, d=d, n_routed=N, n_groups=G, topk_groups=M, topk=K, inter=128, n_shared=0)
    sh = B.moe_shape.of(cfg)
    assert T * d * 2 >= (1 << 32)                   # past the last byte a 32-bit offset reaches
    gen = torch.Generator(device=DEV).manual_seed(20261204)
    u = torch.randn((T, d), generator=gen, device=DEV, dtype=torch.bfloat16)
    cent = (torch.randn((N, d), generator=gen, device=DEV) * (1.7 / d ** 0.5)).to(torch.bfloat16)
    bias = (torch.rand((N,), generator=gen, device=DEV) * 0.02 - 0.01).float()
    idx = torch.empty((T, K), dtype=torch.int32, device=DEV)
    gate = torch.empty((T, K), dtype=torch.float32, device=DEV)
    load = torch.full((N,), -7, dtype=torch.int32, device=DEV)
    scores = torch.empty((T, N), dtype=torch.float32, device=DEV)
    ws = torch.empty(B.moe_workspace_bytes(sh, B.MOE_BF16), dtype=torch.uint8, device=DEV)
    B.moe_route(sh, u, cent, bias, idx, gate, load, scores, ws)
    torch.cuda.synchronize()
    gi = npi(idx)
    assert np.array_equal(npi(load), np.bincount(gi.ravel(), minlength=N))
    rows = np.r_[0:16, 1776:1808, 2032:2048]
    r = oracle.route(np64(u[torch.from_numpy(rows).to(DEV)]), np64(cent), np64(bias), G, M, cfg.group_topn, K)
    ds = np.abs(np64(scores)[rows] - r["s"]).max()
    print(f"[parity] d = 2^20, T = {T}: max |s_gpu - s_oracle| = {ds:.2e} over {rows.size} tokens")
    assert ds < 1e-5
    bad = routing_mismatches(idx[torch.from_numpy(rows).to(DEV)], r)
    ok = np.ones(rows.size, dtype=bool)
    ok[bad] = False
    report("d = 2^20 gates", rel_l2(np64(gate)[rows][ok], r["gate"][ok]), 1e-5)


@pytest.mark.parametrize("name", ["c1", "c3"])
def test_route_without_scores(name):
    """scores = NULL: the affinities are not written (bf16) or pass through the workspace (fp32); the
    selection, gates and loads are bit-identical to a call that writes them."""
    cfg, inp = _inputs(name)
    sh = B.moe_shape.of(cfg)
    T, K, N = cfg.T, cfg.topk, cfg.n_routed
    outs = []
    for with_scores in (True, False):
        idx = torch.empty((T, K), dtype=torch.int32, device=DEV)
        gate = torch.empty((T, K), dtype=torch.float32, device=DEV)
        load = torch.empty((N,), dtype=torch.int32, device=DEV)
        scores = torch.empty((T, N), dtype=torch.float32, device=DEV) if with_scores else None
        B.moe_route(sh, inp["u"], inp["centroids"], inp["bias"], idx, gate, load, scores, _ws(cfg))
        torch.cuda.synchronize()
        outs.append((idx.cpu(), gate.cpu(), load.cpu()))
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_route_exact_ties():
    """Exact ties follow the tie rule: experts in classes of four identical ones (same centroid and bias; groups
    4..7 copy groups 0..3, so groups tie too). Within a class, a picked expert's lower-index twins are picked."""
    cfg, inp = _inputs("c2")
    N, K, T = cfg.n_routed, cfg.topk, cfg.T
    cls = (np.arange(N) % 32) // 2                         # {2c, 2c+1, 2c+32, 2c+33} share class c
    cent = inp["centroids"][torch.from_numpy(cls).to(DEV)].contiguous()
    bias = inp["bias"][torch.from_numpy(cls).to(DEV)].contiguous()
    sh = B.moe_shape.of(cfg)
    idx = torch.empty((T, K), dtype=torch.int32, device=DEV)
    gate = torch.empty((T, K), dtype=torch.float32, device=DEV)
    load = torch.empty((N,), dtype=torch.int32, device=DEV)
    B.moe_route(sh, inp["u"], cent, bias, idx, gate, load, None, _ws(cfg))
    torch.cuda.synchronize()
    gi = npi(idx)
    members = [np.where(cls == c)[0] for c in range(16)]
    for t in range(T):
        picked = set(gi[t].tolist())
        for m in members:
            flags = [int(e) in picked for e in m]            # members in ascending index order
            assert flags == sorted(flags, reverse=True), f"token {t}: class {m} picked {flags}"
    r = oracle.route(inp["u"], cent, bias, cfg.n_groups, cfg.topk_groups, cfg.group_topn, K)
    bad = routing_mismatches(idx, r)
    ok = np.ones(T, dtype=bool)
    ok[bad] = False
    assert np.array_equal(gi[ok], r["idx"][ok])
    report("tie gates", rel_l2(np64(gate)[ok], r["gate"][ok]), 1e-5)


@pytest.mark.parametrize("name,seq_len", [("c2", 4096), ("c2", 1000), ("c2", 1), ("c3", 4096), ("c5", 100)])
def test_balance_stats(name, seq_len):
    """Eq. (17)-(20) per sequence on the oracle's own routing (affinities rounded to fp32): f exact up to
    one fp32 rounding, P and the loss to 1e-5 relative; sum f = N_r per sequence."""
    cfg, inp = _inputs(name)
    sh = B.moe_shape.of(cfg)
    T, N = cfg.T, cfg.n_routed
    r = _oracle_route(cfg, inp)
    s32 = r["s"].astype(np.float32)
    n_seq = -(-T // seq_len)
    f = torch.empty((n_seq, N), dtype=torch.float32, device=DEV)
    P = torch.empty((n_seq, N), dtype=torch.float32, device=DEV)
    loss = torch.empty((n_seq,), dtype=torch.float32, device=DEV)
    B.moe_balance_stats(sh, torch.from_numpy(s32).to(DEV), _i32(r["idx"]), seq_len, 1e-4, f, P, loss, _ws(cfg))
    torch.cuda.synchronize()
    of, oP, ol = oracle.balance_stats(s32, r["idx"], seq_len, alpha=1e-4)
    assert np.allclose(np64(f), of, rtol=2 ** -23, atol=0)
    report(f"{name} seq {seq_len} P", rel_l2(np64(P), oP), 1e-5)
    report(f"{name} seq {seq_len} loss", rel_l2(np64(loss), ol), 1e-5)
    assert np.allclose(np64(f).sum(axis=1), N, rtol=1e-5)


PERM_CASES = ["c1", "c2", "c3", "one_expert", "ragged", "single_token"]


def _perm_idx(case):
    rng = np.random.default_rng(11)
    if case in ("c1", "c2", "c3"):
        cfg, inp = _inputs(case)
        return cfg, _oracle_route(cfg, inp)["idx"]
    if case == "one_expert":      # every token picks experts {0..K-1}: most experts empty
        cfg = get_config("c2", T=777)
        return cfg, np.tile(np.arange(cfg.topk), (cfg.T, 1))
    if case == "ragged":
        cfg = get_config("c2", T=4096 + 37)
        return cfg, np.sort(np.stack([rng.choice(cfg.n_routed, cfg.topk, replace=False) for _ in range(cfg.T)]), 1)
    cfg = get_config("c3", T=1)
    return cfg, np.sort(rng.choice(cfg.n_routed, cfg.topk, replace=False))[None, :]


@pytest.mark.parametrize("case", PERM_CASES)
def test_permute_maps(case):
    cfg, idx = _perm_idx(case)
    sh = B.moe_shape.of(cfg)
    T, K, N = cfg.T, cfg.topk, cfg.n_routed
    off = torch.full((N + 1,), -1, dtype=torch.int32, device=DEV)
    perm = torch.full((T * K,), -1, dtype=torch.int32, device=DEV)
    row_of = torch.full((T * K,), -1, dtype=torch.int32, device=DEV)
    B.moe_permute(sh, _i32(idx), None, off, perm, row_of, workspace=_ws(cfg))
    torch.cuda.synchronize()
    o_off, o_perm, o_row = oracle.permute(idx, N)
    assert np.array_equal(npi(off), o_off)
    assert np.array_equal(npi(perm), o_perm)
    assert np.array_equal(npi(row_of), o_row)


def test_permute_drops_invalid_pairs():
    """Pairs with an expert id outside [0, N_r) or repeating an earlier id of the same token get no row
    (row_of = -1); offsets count the remaining pairs, and perm_token past them holds -1. Expected maps from
    the plain definition: a stable sort of the kept pairs by (expert, token)."""
    cfg = get_config("c2", T=300)
    T, K, N = cfg.T, cfg.topk, cfg.n_routed
    rng = np.random.default_rng(17)
    idx = np.sort(np.stack([rng.choice(N, K, replace=False) for _ in range(T)]), 1)
    idx[3, 2] = N                   # out of range
    idx[7, 0] = -5
    idx[11, 4] = idx[11, 1]         # duplicate inside a token
    idx[12] = idx[12, 0]            # every slot the same expert
    idx[250:, :] = N + 3            # a run of tokens with no valid pair
    keep = np.zeros((T, K), dtype=bool)
    for t in range(T):
        seen = set()
        for k in range(K):
            e = int(idx[t, k])
            if 0 <= e < N and e not in seen:
                keep[t, k] = True
                seen.add(e)
    pairs = sorted((int(idx[t, k]), t, k) for t in range(T) for k in range(K) if keep[t, k])
    load = np.bincount([p[0] for p in pairs], minlength=N)
    o_off = np.concatenate([[0], np.cumsum(load)])
    o_perm = np.full(T * K, -1)
    o_row = np.full(T * K, -1)
    for r, (e, t, k) in enumerate(pairs):
        o_perm[r] = t
        o_row[t * K + k] = r
    sh = B.moe_shape.of(cfg)
    off = torch.full((N + 1,), -7, dtype=torch.int32, device=DEV)
    perm = torch.full((T * K,), -7, dtype=torch.int32, device=DEV)
    row_of = torch.full((T * K,), -7, dtype=torch.int32, device=DEV)
    B.moe_permute(sh, _i32(idx), None, off, perm, row_of, workspace=_ws(cfg))
    torch.cuda.synchronize()
    assert np.array_equal(npi(off), o_off)
    assert np.array_equal(npi(perm), o_perm)
    assert np.array_equal(npi(row_of), o_row)


@pytest.mark.parametrize("name", ["c1", "c2"])
def test_permute_gather_rows(name):
    cfg, inp = _inputs(name)
    sh = B.moe_shape.of(cfg)
    T, K, N, d = cfg.T, cfg.topk, cfg.n_routed, cfg.d
    r = _oracle_route(cfg, inp)
    o_off, o_perm, _ = oracle.permute(r["idx"], N)
    off = torch.empty((N + 1,), dtype=torch.int32, device=DEV)
    perm = torch.empty((T * K,), dtype=torch.int32, device=DEV)
    row_of = torch.empty((T * K,), dtype=torch.int32, device=DEV)
    a = torch.empty((T * K, d), dtype=inp["u"].dtype, device=DEV)
    B.moe_permute(sh, _i32(r["idx"]), inp["u"], off, perm, row_of, a, None, None, 1, _ws(cfg))
    torch.cuda.synchronize()
    assert torch.equal(a.cpu(), inp["u"].cpu()[torch.from_numpy(o_perm)])


@pytest.mark.parametrize("gather", [0, 1])
def test_permute_fp8_quantisation_bit_exact(gather):
    cfg, inp = _inputs("c2")
    sh = B.moe_shape.of(cfg)
    T, K, N, d = cfg.T, cfg.topk, cfg.n_routed, cfg.d
    r = _oracle_route(cfg, inp)
    o_off, o_perm, _ = oracle.permute(r["idx"], N)
    rows = T * K if gather else T
    u = inp["u"].clone()
    u[5] = 0                         # an all-zero row: scale 1, zero codes
    u[9, :128] = 0
    off = torch.empty((N + 1,), dtype=torch.int32, device=DEV)
    perm = torch.empty((T * K,), dtype=torch.int32, device=DEV)
    row_of = torch.empty((T * K,), dtype=torch.int32, device=DEV)
    q = torch.empty((rows, d), dtype=torch.uint8, device=DEV)
    sc = torch.empty((rows, d // 128), dtype=torch.float32, device=DEV)
    B.moe_permute(sh, _i32(r["idx"]), u, off, perm, row_of, q, B.MOE_F8E4M3, sc, gather, _ws(cfg))
    torch.cuda.synchronize()
    codes, scale = oracle.quantize_tiles(u.cpu().float().numpy())
    if gather:
        codes, scale = codes[o_perm], scale[o_perm]
    assert np.array_equal(q.cpu().numpy(), codes)
    assert np.array_equal(sc.cpu().numpy(), scale)


def _e4m3_edge_row(d):
    """bf16-exact values that probe the E4M3 encode: every code's value, the midpoints between neighbouring
    codes (ties to even), the subnormal grid and its midpoints, and values just off the ties; each 128-wide
    tile holds 448 so its scale is exactly 1 and the encode sees the values unchanged."""
    import numpy as _np
    vals = []
    for e in range(-9, 9):
        for m in range(8):
            v = (1 + m / 8) * 2.0 ** e if e >= -6 else m / 8 * 2.0 ** -6
            vals.append(v)
    vals = sorted(set(v for v in vals if v <= 448))
    mids = [(a + b) / 2 for a, b in zip(vals, vals[1:])]
    off = [m * (1 + 2 ** -7) for m in mids] + [m * (1 - 2 ** -7) for m in mids]
    pool = _np.array(vals + mids + off, dtype=_np.float64)
    pool = _np.concatenate([pool, -pool])
    row = _np.resize(pool, d).astype(_np.float32)
    row[::128] = 448.0
    return torch.from_numpy(row).to(torch.bfloat16)


def test_permute_fp8_quantisation_edge_values():
    """Ties, subnormals and saturation through the 1x128 row quantisation, bit-exact against the oracle."""
    cfg, inp = _inputs("c2")
    sh = B.moe_shape.of(cfg)
    T, d = cfg.T, cfg.d
    u = inp["u"].clone()
    for t in range(8):
        u[t] = torch.roll(_e4m3_edge_row(d), shifts=t * 37)
        u[t, ::128] = 448.0
    u[8] = _e4m3_edge_row(d) * 1e4   # beyond 448 in every tile: saturates after scaling
    idx = _i32(_oracle_route(cfg, inp)["idx"])
    off = torch.empty((cfg.n_routed + 1,), dtype=torch.int32, device=DEV)
    perm = torch.empty((T * cfg.topk,), dtype=torch.int32, device=DEV)
    row_of = torch.empty((T * cfg.topk,), dtype=torch.int32, device=DEV)
    q = torch.empty((T, d), dtype=torch.uint8, device=DEV)
    sc = torch.empty((T, d // 128), dtype=torch.float32, device=DEV)
    B.moe_permute(sh, idx, u, off, perm, row_of, q, B.MOE_F8E4M3, sc, 0, _ws(cfg))
    torch.cuda.synchronize()
    codes, scale = oracle.quantize_tiles(u.cpu().float().numpy())
    assert np.array_equal(q.cpu().numpy()[:16], codes[:16])
    assert np.array_equal(sc.cpu().numpy()[:16], scale[:16])
    assert np.array_equal(q.cpu().numpy(), codes)


@pytest.mark.parametrize("gather", [0, 1])
def test_permute_fp8_pow2_scales_bit_exact(gather):
    """Power-of-two tile scales: codes and scales bit-exact against the oracle, with an all-zero row and
    tile, E4M3 ties, saturating rows, rows whose amax / 448 is itself a power of two, and tiny and huge
    magnitudes (scales far from 1 in both directions)."""
    cfg, inp = _inputs("c2")
    sh = B.moe_shape.of(cfg)
    T, K, N, d = cfg.T, cfg.topk, cfg.n_routed, cfg.d
    r = _oracle_route(cfg, inp)
    o_off, o_perm, _ = oracle.permute(r["idx"], N)
    rows = T * K if gather else T
    u = inp["u"].clone()
    u[5] = 0
    u[9, :128] = 0
    for t in range(10, 14):
        u[t] = torch.roll(_e4m3_edge_row(d), shifts=t * 29)
    u[14] = _e4m3_edge_row(d) * 1e4
    u[15] = u[15] * 2.0 ** -100
    u[16] = u[16] * 2.0 ** 100
    u[17, ::128] = 448.0 * 2.0 ** -3        # amax / 448 = 2^-3 in every tile
    u[18] = u[18] * 1e-36                   # amax / 448 below the fp32 normal range
    off = torch.empty((N + 1,), dtype=torch.int32, device=DEV)
    perm = torch.empty((T * K,), dtype=torch.int32, device=DEV)
    row_of = torch.empty((T * K,), dtype=torch.int32, device=DEV)
    q = torch.empty((rows, d), dtype=torch.uint8, device=DEV)
    sc = torch.empty((rows, d // 128), dtype=torch.float32, device=DEV)
    B.moe_permute(sh, _i32(r["idx"]), u, off, perm, row_of, q, B.MOE_F8E4M3_POW2, sc, gather, _ws(cfg))
    torch.cuda.synchronize()
    codes, scale = oracle.quantize_tiles(u.cpu().float().numpy(), pow2=True)
    if gather:
        codes, scale = codes[o_perm], scale[o_perm]
    assert np.array_equal(sc.cpu().numpy(), scale)
    assert np.array_equal(q.cpu().numpy(), codes)


def test_fp8_layer_pow2_act_scales():
    """The fp8 layer with power-of-two scales on the up-projection input: the token quantisation bit-exact,
    sampled experts and tokens against the oracle's fp8 FFN with the same input scales."""
    cfg, inp = _inputs("c2", gemm="fp8")
    T, K, N = cfg.T, cfg.topk, cfg.n_routed
    layer = MoELayer(cfg, inp, DEV, pow2_act_scales=True)
    layer.route(inp["u"])
    layer.permute(inp["u"])
    layer.ffn_routed_phases(inp["u"])
    layer.ffn_shared(inp["u"])
    layer.combine(inp["u"])
    out = layer.out
    torch.cuda.synchronize()
    r = _oracle_route(cfg, inp)
    bad = routing_mismatches(layer.topk_idx, r)
    u32 = inp["u"].cpu().float().numpy()
    codes, scale = oracle.quantize_tiles(u32, pow2=True)
    assert np.array_equal(layer.u_q.cpu().numpy(), codes)
    assert np.array_equal(layer.u_scale.cpu().numpy(), scale)
    load = r["load"]
    experts = sorted({0, N - 1, int(np.argmax(load)), int(np.argmin(load))})
    _check_fp8_experts(cfg, inp, layer, experts, "c2 pow2", pow2=True)
    u64 = np64(inp["u"])
    toks = [t for t in np.random.default_rng(2).choice(T, 6, replace=False) if t not in set(bad)][:3]
    for t in toks:
        acc = u64[t].copy()
        for sh_e in range(cfg.n_shared):
            acc = acc + oracle.ffn_fp8(u32[[t]], *oracle_wq(cfg, inp, sh_e, shared=True), pow2_input=True)[0]
        for k in range(K):
            e = int(r["idx"][t, k])
            acc = acc + r["gate"][t, k] * oracle.ffn_fp8(u32[[t]], *oracle_wq(cfg, inp, e), pow2_input=True)[0]
        report(f"c2 fp8 pow2 out-u token {t}", rel_l2(np64(out[t]) - u64[t], acc - u64[t]), TOL["fp8"])


@pytest.mark.parametrize("gemm", ["bf16", "fp8", "mxfp4"])
def test_batch_invariance(gemm):
    """batch_invariant = 1: 100 tokens of a 4096-token batch, placed among other tokens in a 160-token batch,
    and one of them alone, get bit-identical affinities, selections, gates and layer outputs. At d = 4096
    (32 chunks of 128) the default mode's router K split follows T (16 slices for the 4096-token batch, 32
    for the small ones), so there the affinities of the same tokens differ between the batches: checked, so
    that the mode is shown to matter."""
    from dataclasses import replace
    from moe_inputs import generate_tokens
    cfg, inp = _inputs("c2", gemm=gemm, batch_invariant=1, d=4096)
    T = cfg.T
    sel = np.random.default_rng(5).choice(T, 100, replace=False)
    other = generate_tokens(cfg, DEV, step=3)[:60]
    u_b = torch.cat([other[:30], inp["u"][torch.from_numpy(sel).to(DEV)], other[30:]]).contiguous()
    u_c = inp["u"][int(sel[7])].reshape(1, -1).contiguous()
    rows_b = np.arange(30, 130)
    res = {}
    for bi in (1, 0):
        outs = []
        for u in (inp["u"], u_b, u_c):
            c = replace(cfg, T=u.shape[0], batch_invariant=bi)
            layer = MoELayer(c, inp, DEV)
            layer.forward(u)
            torch.cuda.synchronize()
            outs.append({k: getattr(layer, k).cpu() for k in ("scores", "topk_idx", "topk_gate", "out")})
            del layer
        res[bi] = outs
    full, part, one = res[1]
    for k in ("scores", "topk_idx", "topk_gate", "out"):
        a = full[k][torch.from_numpy(sel)]
        assert torch.equal(a, part[k][torch.from_numpy(rows_b)]), k
        assert torch.equal(a[7:8], one[k]), k
    full0, part0, _ = res[0]
    n_diff = int((full0["scores"][torch.from_numpy(sel)] != part0["scores"][torch.from_numpy(rows_b)]).sum())
    print(f"[parity] {gemm} batch-invariant mode: 0 differing results; default mode: {n_diff} of "
          f"{100 * cfg.n_routed} affinities differ between the two batches")
    assert n_diff > 0, "the default mode's K split should follow T at this shape"


@pytest.mark.parametrize("kind", ["gate_up", "down", "down_padded"])
def test_quantize_weights_bit_exact(kind):
    """E4M3 codes in the tiled layout and the block scales, bit for bit: c2's gate/up matrices (gate and up rows
    interleaved per 128 H columns), its down matrices, and 384-row matrices whose second tile is padded."""
    cfg, inp = _inputs("c2")
    if kind == "gate_up":
        w = inp["w_gate_up"][:3].contiguous()
    elif kind == "down":
        w = inp["w_down"][:3].contiguous()
    else:
        w = (torch.randn((2, 384, 256), generator=torch.Generator().manual_seed(3)) * 0.02).to(torch.bfloat16).to(DEV)
    n, rr, cc = w.shape
    codes = torch.empty((n, B.mx_rows(rr), cc), dtype=torch.uint8, device=DEV)
    scale = torch.empty((n, rr // 128, cc // 128), dtype=torch.float32, device=DEV)
    B.moe_quantize_weights(w, codes, scale, gate_up=(kind == "gate_up"))
    torch.cuda.synchronize()
    for e in range(n):
        oc, os_ = oracle.quantize_blocks(w[e].cpu().float().numpy())
        assert np.array_equal(codes[e].cpu().numpy().reshape(-1), tile_e4m3(oc, kind == "gate_up"))
        assert np.array_equal(scale[e].cpu().numpy(), os_)


_oracle_ffn_rows = oracle_ffn_rows


@pytest.mark.parametrize("name,mode", [("c1", "gather"), ("c1", "direct"), ("c2", "gather"), ("c2", "direct")])
def test_grouped_ffn_routed(name, mode):
    cfg, inp = _inputs(name)
    sh = B.moe_shape.of(cfg)
    T, K, N, d = cfg.T, cfg.topk, cfg.n_routed, cfg.d
    r = _oracle_route(cfg, inp)
    o_off, o_perm, _ = oracle.permute(r["idx"], N)
    wdt = B.MOE_F32 if cfg.gemm == "f32" else B.MOE_BF16
    y = torch.empty((T * K, d), dtype=torch.float32 if cfg.gemm == "f32" else torch.bfloat16, device=DEV)
    if mode == "gather":
        a, a_rows, m, src = inp["u"], T, B.MOE_ROWS_GATHER, _i32(o_perm)
    else:
        a = inp["u"][torch.from_numpy(o_perm).to(DEV)].contiguous()
        a_rows, m, src = T * K, B.MOE_ROWS_DIRECT, None
    B.moe_grouped_ffn(sh, wdt, N, T * K, _i32(o_off), m, src, a, None, a_rows, inp["w_gate_up"], None,
                      inp["w_down"], None, y, _ws(cfg))
    torch.cuda.synchronize()
    ref = np.zeros((T * K, d))
    for e in range(N):
        lo, hi = o_off[e], o_off[e + 1]
        if hi > lo:
            ref[lo:hi] = _oracle_ffn_rows(cfg, inp, e, o_perm[lo:hi])
    report(f"{name} routed y ({mode})", rel_l2(y, ref), TOL[cfg.gemm])


@pytest.mark.parametrize("name", ["c1", "c2"])
def test_grouped_ffn_shared_segments(name):
    cfg, inp = _inputs(name)
    sh = B.moe_shape.of(cfg)
    T, Ns, d = cfg.T, cfg.n_shared, cfg.d
    wdt = B.MOE_F32 if cfg.gemm == "f32" else B.MOE_BF16
    y = torch.empty((Ns * T, d), dtype=torch.float32 if cfg.gemm == "f32" else torch.bfloat16, device=DEV)
    off = _i32(np.arange(Ns + 1) * T)
    B.moe_grouped_ffn(sh, wdt, Ns, Ns * T, off, B.MOE_ROWS_SEGMENT, None, inp["u"], None, T, inp["s_gate_up"],
                      None, inp["s_down"], None, y, _ws(cfg))
    torch.cuda.synchronize()
    ref = np.concatenate([_oracle_ffn_rows(cfg, inp, s, np.arange(T), shared=True) for s in range(Ns)])
    report(f"{name} shared y", rel_l2(y, ref), TOL[cfg.gemm])


def test_grouped_ffn_ragged_and_empty_experts():
    """Segments of 0, 1, 127, 128, 129 and 300 rows across experts (bf16)."""
    cfg = get_config("c2", n_routed=8, n_groups=1, topk_groups=1, T=512, topk=2)
    inp = generate(cfg, DEV)
    sh = B.moe_shape.of(cfg)
    sizes = [0, 1, 127, 128, 129, 0, 300, 339]
    assert sum(sizes) == cfg.T * cfg.topk
    off = np.concatenate([[0], np.cumsum(sizes)])
    src = np.random.default_rng(5).integers(0, cfg.T, off[-1])
    y = torch.empty((off[-1], cfg.d), dtype=torch.bfloat16, device=DEV)
    B.moe_grouped_ffn(sh, B.MOE_BF16, 8, int(off[-1]), _i32(off), B.MOE_ROWS_GATHER, _i32(src), inp["u"], None,
                      cfg.T, inp["w_gate_up"], None, inp["w_down"], None, y, _ws(cfg))
    torch.cuda.synchronize()
    ref = np.zeros((off[-1], cfg.d))
    for e in range(8):
        if sizes[e]:
            ref[off[e]:off[e + 1]] = _oracle_ffn_rows(cfg, inp, e, src[off[e]:off[e + 1]])
    report("ragged y", rel_l2(y, ref), TOL["bf16"])


@pytest.mark.parametrize("mode", ["gather", "direct"])
def test_grouped_ffn_tile_shapes(mode):
    """Expert segment sizes that reach every block shape of the bf16 kernels.

    Rows are cut into 32-row sub-tiles and an expert's sub-tiles into
    ceil(n32 / 8) near-equal blocks of at most 256 rows, each wave row taking
    every other sub-tile. Sizes: empty, 1 and 2 sub-tiles, exactly 8, 9 with a
    1-row tail (5 + 4), 9 full, 10 ragged and full, 11, 17 (3 blocks), 20 and 21.
    """
    cfg = get_config("c2", n_routed=12, n_groups=1, topk_groups=1, T=2048, topk=2)
    inp = generate(cfg, DEV)
    sh = B.moe_shape.of(cfg)
    sizes = [0, 1, 33, 256, 257, 288, 289, 320, 321, 544, 640, 672]
    off = np.concatenate([[0], np.cumsum(sizes)])
    n = int(off[-1])
    assert n <= cfg.T * cfg.topk
    rng = np.random.default_rng(17)
    src = rng.integers(0, cfg.T, n)
    y = torch.empty((n, cfg.d), dtype=torch.bfloat16, device=DEV)
    if mode == "gather":
        B.moe_grouped_ffn(sh, B.MOE_BF16, 12, n, _i32(off), B.MOE_ROWS_GATHER, _i32(src), inp["u"], None,
                          cfg.T, inp["w_gate_up"], None, inp["w_down"], None, y, _ws(cfg))
    else:
        a = inp["u"][torch.from_numpy(src).to(DEV)].contiguous()
        B.moe_grouped_ffn(sh, B.MOE_BF16, 12, n, _i32(off), B.MOE_ROWS_DIRECT, None, a, None,
                          n, inp["w_gate_up"], None, inp["w_down"], None, y, _ws(cfg))
    torch.cuda.synchronize()
    for e in range(12):
        if sizes[e]:
            ref = _oracle_ffn_rows(cfg, inp, e, src[off[e]:off[e + 1]])
            report(f"{mode} expert {e} ({sizes[e]} rows) y", rel_l2(y[off[e]:off[e + 1]], ref), TOL["bf16"])


@pytest.mark.parametrize("d", [384, 640])
def test_grouped_ffn_bf16_half_column_tile(d):
    """d % 256 == 128: the down projection's last output-column tile has 128 columns (the other half of the
    tile must be neither computed into y nor written past the row)."""
    cfg = get_config("c2", n_routed=4, n_groups=1, topk_groups=1, T=512, topk=2, d=d, inter=256)
    inp = generate(cfg, DEV)
    sh = B.moe_shape.of(cfg)
    sizes = [0, 40, 300, 129]
    off = np.concatenate([[0], np.cumsum(sizes)])
    n = int(off[-1])
    src = np.random.default_rng(5).integers(0, cfg.T, n)
    y = torch.full((n + 1, d), 7.0, dtype=torch.bfloat16, device=DEV)     # one guard row past the end
    B.moe_grouped_ffn(sh, B.MOE_BF16, 4, n, _i32(off), B.MOE_ROWS_GATHER, _i32(src), inp["u"], None, cfg.T,
                      inp["w_gate_up"], None, inp["w_down"], None, y[:n], _ws(cfg))
    torch.cuda.synchronize()
    assert torch.all(y[n] == 7.0)
    for e in range(4):
        if sizes[e]:
            ref = _oracle_ffn_rows(cfg, inp, e, src[off[e]:off[e + 1]])
            report(f"d={d} expert {e} ({sizes[e]} rows) y", rel_l2(y[off[e]:off[e + 1]], ref), TOL["bf16"])


def test_grouped_ffn_bf16_gather_near_4gib():
    """The bf16 gate/up gathers token rows through 32-bit byte offsets: an a of a_rows * d * 2 bytes just under
    4 GiB (a_rows = 299,593 at d = 7168, the most the call accepts) with rows picked at both ends of it, three
    experts, row-major and tiled weights. y against the oracle; the tiled run equals the row-major one bit for bit.
    Seeded inputs made on the device: a ~ N(0, 1) bf16; the experts' weights as the workload generator draws them."""
    d, I, E = 7168, 256, 3
    a_rows = ((1 << 32) - 1) // (2 * d)
    cfg = get_config("c2", T=a_rows, d=d, inter=I, n_routed=E, n_groups=1, topk_groups=1, topk=1, n_shared=0)
    sh = B.moe_shape.of(cfg)
    gen = torch.Generator(device=DEV).manual_seed(4242)
    a = torch.randn((a_rows, d), generator=gen, device=DEV, dtype=torch.bfloat16)
    ws_ = [generate_expert(cfg, e, device=DEV) for e in range(E)]
    wgu = torch.stack([w[0] for w in ws_]).contiguous()
    wd = torch.stack([w[1] for w in ws_]).contiguous()
    sizes = [40, 33, 23]
    off = np.concatenate([[0], np.cumsum(sizes)])
    n = int(off[-1])
    rng = np.random.default_rng(11)
    src = np.concatenate([np.arange(a_rows - 48, a_rows), np.arange(0, 16), rng.integers(0, a_rows, n - 64)])
    rng.shuffle(src)
    ws = torch.empty(B.moe_workspace_bytes(sh, B.MOE_BF16_TILED), dtype=torch.uint8, device=DEV)
    y0 = torch.empty((n, d), dtype=torch.bfloat16, device=DEV)
    B.moe_grouped_ffn(sh, B.MOE_BF16, E, n, _i32(off), B.MOE_ROWS_GATHER, _i32(src), a, None, a_rows, wgu, None, wd,
                      None, y0, ws)
    tg = torch.empty((E, B.mx_rows(2 * I), d), dtype=torch.bfloat16, device=DEV)
    td = torch.empty((E, B.mx_rows(d), I), dtype=torch.bfloat16, device=DEV)
    B.moe_tile_weights_bf16(wgu, tg, gate_up=True)
    B.moe_tile_weights_bf16(wd, td, gate_up=False)
    y1 = torch.empty((n, d), dtype=torch.bfloat16, device=DEV)
    B.moe_grouped_ffn(sh, B.MOE_BF16_TILED, E, n, _i32(off), B.MOE_ROWS_GATHER, _i32(src), a, None, a_rows, tg, None,
                      td, None, y1, ws)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
    a_rows_used = a[torch.from_numpy(src).to(DEV)].float().cpu()
    for e in range(E):
        ref = oracle.expert_ffn(a_rows_used[off[e]:off[e + 1]].double().numpy(), wgu[e].cpu(), wd[e].cpu(), "bf16")
        report(f"a near 4 GiB, expert {e} ({sizes[e]} rows) y", rel_l2(y0[off[e]:off[e + 1]], ref), TOL["bf16"])


def _down_rows_check(tag, y, h64, wd64, off, rows, tol):
    """y rows of the down projection against h64 @ wd64[e]^T (fp64) on the sampled rows of each expert."""
    for e in range(len(off) - 1):
        r = rows[(rows >= off[e]) & (rows < off[e + 1])]
        ref = h64[np.searchsorted(rows, r)] @ wd64[e].T
        report(f"{tag} expert {e} ({r.size} sampled rows) y", rel_l2(y[torch.from_numpy(r).to(DEV)], ref), tol)


def test_ffn_down_h_near_4gib():
    """The down projection reads H rows through 32-bit byte offsets: n_rows * inter * 2 bytes of bf16 H just
    under 4 GiB (n_rows = 1,048,575 at inter = 2048, the most the call accepts; d = 1024 keeps y at 2 GiB), two
    experts, row-major and tiled weights; sampled rows at the start, the expert boundary and the end against
    the oracle. Seeded inputs made on the device: H ~ N(0, 1) bf16, W_d ~ N(0, 0.02^2) bf16."""
    d, I, E = 1024, 2048, 2
    n = ((1 << 32) - 1) // (2 * I)
    cfg = get_config("c2", T=128, d=d, inter=I, n_routed=E, n_groups=1, topk_groups=1, topk=1, n_shared=0)
    sh = B.moe_shape.of(cfg)
    gen = torch.Generator(device=DEV).manual_seed(777)
    h = torch.randn((n, I), generator=gen, device=DEV, dtype=torch.bfloat16)
    wd = (torch.randn((E, d, I), generator=gen, device=DEV) * 0.02).to(torch.bfloat16)
    off = np.array([0, n // 2 + 5, n])
    rows = np.unique(np.concatenate([np.arange(0, 16), np.arange(off[1] - 16, off[1] + 16), np.arange(n - 16, n),
                                     np.random.default_rng(3).integers(0, n, 32)]))
    h64 = np64(h[torch.from_numpy(rows).to(DEV)])
    wd64 = np64(wd)
    ws = torch.empty(256, dtype=torch.uint8, device=DEV)
    y = torch.empty((n, d), dtype=torch.bfloat16, device=DEV)
    B.moe_ffn_down(sh, B.MOE_BF16, E, n, _i32(off), h, None, wd, None, y, ws)
    torch.cuda.synchronize()
    _down_rows_check("bf16 H near 4 GiB", y, h64, wd64, off, rows, TOL["bf16"])
    td = torch.empty((E, B.mx_rows(d), I), dtype=torch.bfloat16, device=DEV)
    B.moe_tile_weights_bf16(wd, td, gate_up=False)
    y1 = torch.empty_like(y)
    B.moe_ffn_down(sh, B.MOE_BF16_TILED, E, n, _i32(off), h, None, td, None, y1, ws)
    torch.cuda.synchronize()
    assert torch.equal(y[torch.from_numpy(rows).to(DEV)], y1[torch.from_numpy(rows).to(DEV)])


def test_ffn_down_fp8_h_near_4gib():
    """fp8 down projection with n_rows * inter bytes of E4M3 H codes just under 4 GiB (n_rows = 2,097,151 at
    inter = 2048, the most the call accepts; d = 1024), two experts on the eight-wave loop; sampled rows against
    the oracle on the dequantised operands. H: seeded random finite E4M3 codes (magnitude codes 0 .. 0x7E, either
    sign) with 1x128 scales ~ U(1e-3, 2e-3); W_d: the oracle's 128x128 quantisation of N(0, 0.02^2) weights."""
    d, I, E = 1024, 2048, 2
    n = ((1 << 32) - 1) // I
    cfg = get_config("c2", T=128, d=d, inter=I, n_routed=E, n_groups=1, topk_groups=1, topk=1, n_shared=0,
                     gemm="fp8")
    sh = B.moe_shape.of(cfg)
    gen = torch.Generator(device=DEV).manual_seed(778)
    h = torch.randint(0, 0x7F, (n, I), generator=gen, device=DEV, dtype=torch.uint8)
    h |= (torch.randint(0, 2, (n, I), generator=gen, device=DEV, dtype=torch.uint8) << 7)
    hs = torch.rand((n, I // 128), generator=gen, device=DEV) * 1e-3 + 1e-3
    w32 = (np.random.default_rng(5).standard_normal((E, d, I)) * 0.02).astype(np.float32)
    wq = [oracle.quantize_blocks(w32[e]) for e in range(E)]
    dev8 = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    wdn = dev8(np.stack([tile_e4m3(q, False) for q, _ in wq]))
    wds = dev8(np.stack([sc for _, sc in wq]))
    off = np.array([0, n // 2 - 7, n])
    rows = np.unique(np.concatenate([np.arange(0, 16), np.arange(off[1] - 16, off[1] + 16), np.arange(n - 16, n),
                                     np.random.default_rng(4).integers(0, n, 32)]))
    sel = torch.from_numpy(rows).to(DEV)
    h64 = oracle.dequantize_tiles(h[sel].cpu().numpy(), hs[sel].cpu().numpy())
    wd64 = np.stack([oracle.dequantize_blocks(q, sc) for q, sc in wq])
    ws = torch.empty(256, dtype=torch.uint8, device=DEV)
    y = torch.empty((n, d), dtype=torch.bfloat16, device=DEV)
    B.moe_ffn_down(sh, B.MOE_F8E4M3, E, n, _i32(off), h, hs, wdn, wds, y, ws)
    torch.cuda.synchronize()
    _down_rows_check("fp8 H near 4 GiB", y, h64, wd64, off, rows, TOL["fp8"])


@pytest.mark.parametrize("kind", ["gate_up", "down_padded"])
def test_tile_weights_bf16_bit_exact(kind):
    """The tiled bf16 layout, byte for byte: the rows' bytes rearranged exactly as the E4M3 tiles (64-byte steps,
    gate/up interleave, zero padding rows), rebuilt here with the NumPy transform."""
    if kind == "gate_up":
        cfg, inp = _inputs("c2")
        w = inp["w_gate_up"][:2].contiguous()
    else:
        w = (torch.randn((2, 384, 256), generator=torch.Generator().manual_seed(4)) * 0.02).to(torch.bfloat16).to(DEV)
    n, rr, cc = w.shape
    out = torch.empty((n, B.mx_rows(rr), cc), dtype=torch.bfloat16, device=DEV)
    B.moe_tile_weights_bf16(w, out, gate_up=(kind == "gate_up"))
    torch.cuda.synchronize()
    got = out.cpu().view(torch.uint8).numpy().reshape(n, -1)
    raw = w.cpu().view(torch.uint8).numpy()                      # [n, rr, 2 cc] bytes
    for e in range(n):
        assert np.array_equal(got[e], tile_e4m3(raw[e], kind == "gate_up"))


@pytest.mark.parametrize("d,mode", [(2048, "gather"), (2048, "direct"), (384, "gather"), (1408, "gather"),
                                    (3328, "direct")])
def test_grouped_ffn_bf16_tiled_equals_row_major(d, mode):
    """MOE_BF16_TILED only changes where the weight bytes are read from: its outputs equal MOE_BF16's bit for bit
    (c2-sized experts). The tiled down kernel runs up to four column tiles of a block as one stream: d = 2048 is
    two full streams, d = 384 one stream of a full and a 128-column tile, d = 1408 a stream of four and one of two
    ending in a 128-column tile, d = 3328 streams of 4, 4, 4 and 1 tiles. Nothing is written past the last row."""
    cfg = get_config("c2", n_routed=6, n_groups=1, topk_groups=1, T=1024, topk=2, d=d, inter=1408)
    inp = generate(cfg, DEV)
    sh = B.moe_shape.of(cfg)
    sizes = [0, 1, 97, 256, 300, 700]
    off = np.concatenate([[0], np.cumsum(sizes)])
    n = int(off[-1])
    src = np.random.default_rng(8).integers(0, cfg.T, n)
    if mode == "gather":
        a, a_rows, m, rs = inp["u"], cfg.T, B.MOE_ROWS_GATHER, _i32(src)
    else:
        a, a_rows, m, rs = inp["u"][torch.from_numpy(src).to(DEV)].contiguous(), n, B.MOE_ROWS_DIRECT, None
    tg = torch.empty((6, B.mx_rows(2 * cfg.inter), d), dtype=torch.bfloat16, device=DEV)
    td = torch.empty((6, B.mx_rows(d), cfg.inter), dtype=torch.bfloat16, device=DEV)
    B.moe_tile_weights_bf16(inp["w_gate_up"], tg, gate_up=True)
    B.moe_tile_weights_bf16(inp["w_down"], td, gate_up=False)
    y0 = torch.empty((n, d), dtype=torch.bfloat16, device=DEV)
    y1g = torch.full((n + 1, d), 7.0, dtype=torch.bfloat16, device=DEV)    # one guard row past the end
    y1 = y1g[:n]
    B.moe_grouped_ffn(sh, B.MOE_BF16, 6, n, _i32(off), m, rs, a, None, a_rows, inp["w_gate_up"], None, inp["w_down"],
                      None, y0, _ws(cfg))
    B.moe_grouped_ffn(sh, B.MOE_BF16_TILED, 6, n, _i32(off), m, rs, a, None, a_rows, tg, None, td, None, y1, _ws(cfg))
    torch.cuda.synchronize()
    assert torch.all(y1g[n] == 7.0)
    assert torch.equal(y0, y1)
    ref = _oracle_ffn_rows(cfg, inp, 5, src[off[5]:off[6]])
    report(f"tiled bf16 d={d} expert 5 y", rel_l2(y1[off[5]:off[6]], ref), TOL["bf16"])


@pytest.mark.parametrize("name", ["c1", "c2"])
def test_combine(name):
    cfg, inp = _inputs(name)
    sh = B.moe_shape.of(cfg)
    T, K, N, d, Ns = cfg.T, cfg.topk, cfg.n_routed, cfg.d, cfg.n_shared
    rng = np.random.default_rng(3)
    r = _oracle_route(cfg, inp)
    _, _, o_row = oracle.permute(r["idx"], N)
    dt = inp["u"].dtype
    # y inputs drawn here (the combine is linear; any y exercises it)
    y = torch.from_numpy(rng.standard_normal((T * K, d))).to(dt).to(DEV)
    ysh = torch.from_numpy(rng.standard_normal((Ns * T, d))).to(dt).to(DEV)
    out = torch.empty((T, d), dtype=dt, device=DEV)
    B.moe_combine(sh, inp["u"], y, _i32(o_row), torch.from_numpy(r["gate"]).float().to(DEV), ysh, out)
    torch.cuda.synchronize()
    g32 = r["gate"].astype(np.float32).astype(np.float64)
    ref = oracle.combine(inp["u"], y, o_row, g32, np64(ysh).reshape(Ns, T, d))
    report(f"{name} combine out", rel_l2(out, ref), TOL[cfg.gemm] if cfg.gemm == "f32" else 4e-3)


def test_bias_update_bit_exact():
    cfg = get_config("c2")
    sh = B.moe_shape.of(cfg)
    N, mean = cfg.n_routed, cfg.T * cfg.topk // cfg.n_routed
    rng = np.random.default_rng(9)
    load = rng.integers(mean - 3, mean + 4, N)
    load[:4] = mean
    b0 = rng.uniform(-0.01, 0.01, N).astype(np.float32)
    bias = torch.from_numpy(b0).to(DEV)
    B.moe_bias_update(sh, _i32(load), 0.001, bias)
    torch.cuda.synchronize()
    assert np.array_equal(bias.cpu().numpy(), oracle.bias_update(b0, load, cfg.T, cfg.topk, 0.001))


def test_bias_state_resume(tmp_path):
    """Checkpoint and resume of the balancing state: a layer saved after 3 steps of the Zipf-skewed decode
    routing and reloaded into a fresh layer continues the bias trajectory bit for bit (same tokens per step),
    with the step counter restored; the file holds the bias exactly as the device had it."""
    cfg = get_config("c5", gemm="bf16", T=96, d=512, inter=256, n_routed=64)
    inp = generate(cfg, DEV)
    a = MoELayer(cfg, inp, DEV, keep_scores=False)
    for step in range(3):
        a.step(generate_tokens(cfg, DEV, step))
    path = str(tmp_path / "bias.bin")
    a.save_state(path)
    saved = a.bias.cpu().numpy().copy()
    for step in range(3, 6):
        a.step(generate_tokens(cfg, DEV, step))
    b = MoELayer(cfg, inp, DEV, keep_scores=False)
    assert not np.array_equal(b.bias.cpu().numpy(), saved)
    b.load_state(path)
    assert b.step_count == 3 and np.array_equal(b.bias.cpu().numpy().view(np.uint32), saved.view(np.uint32))
    for step in range(3, 6):
        b.step(generate_tokens(cfg, DEV, step))
    torch.cuda.synchronize()
    assert b.step_count == a.step_count == 6
    assert np.array_equal(b.bias.cpu().numpy().view(np.uint32), a.bias.cpu().numpy().view(np.uint32))
    assert not np.array_equal(a.bias.cpu().numpy(), saved)


# ------------------------------------------------------------------ fp8 (E4M3, 1x128 / 128x128 scales)

def _check_fp8_experts(cfg, inp, layer, experts, tag, pow2=False):
    goff = npi(layer.expert_offsets)
    gperm = npi(layer.perm_token)
    u32 = inp["u"].cpu().float().numpy()
    for e in experts:
        lo, hi = goff[e], goff[e + 1]
        if hi == lo:
            continue
        wq = oracle_wq(cfg, inp, e)
        ref, aux = oracle.ffn_fp8(u32[gperm[lo:hi]], *wq, return_h=True, pow2_input=pow2)
        report(f"{tag} fp8 expert {e} ({hi - lo} rows) y", rel_l2(layer.y_routed[lo:hi], ref), TOL["fp8"])
        if hasattr(layer, "h"):
            codes = layer.h[lo:hi].cpu().numpy()
            same = float(np.mean(codes == aux["h_codes"]))
            sdiff = np.max(np.abs(layer.h_scale[lo:hi].cpu().numpy() / aux["h_scale"] - 1))
            print(f"[parity] {tag} expert {e}: H codes equal {same:.4f}, max rel scale diff {sdiff:.2e}")
            assert same > 0.99 and sdiff < 1e-4


def test_grouped_ffn_fp8_gather_near_4gib():
    """The fp8 gate/up gathers E4M3 token rows through 32-bit byte offsets: codes of a_rows * d bytes just under
    4 GiB (a_rows = 599,186 at d = 7168, the most the call accepts), rows picked at both ends, three experts on the
    eight-wave loops (d and inter multiples of 1024). Only the picked rows hold data: each is a seeded N(0, 1) row
    quantised by the oracle's 1x128 rule; the other rows are zero codes with scale 1 and are never read. y and the
    H codes against the oracle."""
    d, I, E = 7168, 1024, 3
    a_rows = ((1 << 32) - 1) // d
    cfg = get_config("c2", gemm="fp8", d=d, inter=I, n_routed=E, n_groups=1, topk_groups=1, T=128, topk=1,
                     n_shared=0)
    inp = generate(cfg, DEV)
    sh = B.moe_shape.of(cfg)
    sizes = [40, 33, 23]
    off = np.concatenate([[0], np.cumsum(sizes)])
    n = int(off[-1])
    rng = np.random.default_rng(13)
    mid = rng.choice(np.arange(16, a_rows - 48), n - 64, replace=False)
    src = np.concatenate([np.arange(a_rows - 48, a_rows), np.arange(0, 16), mid])
    rng.shuffle(src)
    u32 = rng.standard_normal((n, d)).astype(np.float32)        # row i of u32 is token row src[i]
    uq, us = oracle.quantize_tiles(u32)
    a = torch.zeros((a_rows, d), dtype=torch.uint8, device=DEV)
    a_s = torch.ones((a_rows, d // 128), dtype=torch.float32, device=DEV)
    si = torch.from_numpy(src).to(DEV)
    a[si] = torch.from_numpy(uq).to(DEV)
    a_s[si] = torch.from_numpy(us).to(DEV)
    wq = [oracle_wq(cfg, inp, e) for e in range(E)]
    dev8 = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    wgu = dev8(np.stack([tile_e4m3(w[0], True) for w in wq])); wgs = dev8(np.stack([w[1] for w in wq]))
    wdn = dev8(np.stack([tile_e4m3(w[2], False) for w in wq])); wds = dev8(np.stack([w[3] for w in wq]))
    h = torch.empty((n, I), dtype=torch.uint8, device=DEV)
    hs = torch.empty((n, I // 128), dtype=torch.float32, device=DEV)
    y = torch.empty((n, d), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(256, dtype=torch.uint8, device=DEV)
    B.moe_ffn_gate_up(sh, B.MOE_F8E4M3, E, n, _i32(off), B.MOE_ROWS_GATHER, _i32(src), a, a_s, a_rows, wgu, wgs, h, hs,
                      ws)
    B.moe_ffn_down(sh, B.MOE_F8E4M3, E, n, _i32(off), h, hs, wdn, wds, y, ws)
    torch.cuda.synchronize()
    for e in range(E):
        lo, hi = off[e], off[e + 1]
        ref, aux = oracle.ffn_fp8(u32[lo:hi], *wq[e], return_h=True)
        report(f"fp8 a near 4 GiB, expert {e} ({hi - lo} rows) y", rel_l2(y[lo:hi], ref), TOL["fp8"])
        same = float(np.mean(h[lo:hi].cpu().numpy() == aux["h_codes"]))
        print(f"[parity] expert {e}: H codes equal {same:.4f}")
        assert same > 0.99


@pytest.mark.parametrize("inter,mode", [(128, "gather"), (1408, "gather"), (1408, "direct")])
def test_grouped_ffn_fp8_tile_shapes(inter, mode):
    """fp8 grouped FFN on expert segments that reach every block shape.

    Blocks hold at most four 32-row sub-tiles (two per wave row). Sizes: empty,
    1 row, 1 and 2 sub-tiles, 3 with a tail, exactly 4, 5 (split 2 + 3), 9 and
    13 (four blocks). inter = 128 gives the down projection a two-stage K loop
    (one 128 chunk); 1408 an odd number of chunks (11), which ends the loop on
    its drain branch. Inputs: oracle-quantised activations and weights; the
    H codes and scales are compared as well.
    """
    cfg = get_config("c2", gemm="fp8", n_routed=10, n_groups=1, topk_groups=1, T=1024, topk=2, inter=inter)
    inp = generate(cfg, DEV)
    sh = B.moe_shape.of(cfg)
    sizes = [0, 1, 32, 64, 65 + 30, 128, 160, 288, 0, 416]
    off = np.concatenate([[0], np.cumsum(sizes)])
    n = int(off[-1])
    assert n <= cfg.T * cfg.topk
    rng = np.random.default_rng(23)
    src = rng.integers(0, cfg.T, n)
    u32 = inp["u"].cpu().float().numpy()
    uq, us = oracle.quantize_tiles(u32)
    wq = [oracle_wq(cfg, inp, e) for e in range(cfg.n_routed)]
    dev8 = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    wgu = dev8(np.stack([tile_e4m3(w[0], True) for w in wq])); wgs = dev8(np.stack([w[1] for w in wq]))
    wdn = dev8(np.stack([tile_e4m3(w[2], False) for w in wq])); wds = dev8(np.stack([w[3] for w in wq]))
    h = torch.empty((n, inter), dtype=torch.uint8, device=DEV)
    hs = torch.empty((n, inter // 128), dtype=torch.float32, device=DEV)
    y = torch.empty((n, cfg.d), dtype=torch.bfloat16, device=DEV)
    if mode == "gather":
        a, a_s, a_rows, rmode, rsrc = dev8(uq), dev8(us), cfg.T, B.MOE_ROWS_GATHER, _i32(src)
    else:
        a, a_s, a_rows, rmode, rsrc = dev8(uq[src]), dev8(us[src]), n, B.MOE_ROWS_DIRECT, None
    ws = torch.empty(256, dtype=torch.uint8, device=DEV)
    B.moe_ffn_gate_up(sh, B.MOE_F8E4M3, cfg.n_routed, n, _i32(off), rmode, rsrc, a, a_s, a_rows, wgu, wgs, h, hs, ws)
    B.moe_ffn_down(sh, B.MOE_F8E4M3, cfg.n_routed, n, _i32(off), h, hs, wdn, wds, y, ws)
    torch.cuda.synchronize()
    for e in range(cfg.n_routed):
        lo, hi = off[e], off[e + 1]
        if hi == lo:
            continue
        ref, aux = oracle.ffn_fp8(u32[src[lo:hi]], *wq[e], return_h=True)
        report(f"fp8 I={inter} {mode} expert {e} ({hi - lo} rows) y", rel_l2(y[lo:hi], ref), TOL["fp8"])
        same = float(np.mean(h[lo:hi].cpu().numpy() == aux["h_codes"]))
        sdiff = np.max(np.abs(hs[lo:hi].cpu().numpy() / aux["h_scale"] - 1))
        print(f"[parity] expert {e}: H codes equal {same:.4f}, max rel scale diff {sdiff:.2e}")
        assert same > 0.99 and sdiff < 1e-4


@pytest.mark.parametrize("mode", ["gather", "direct"])
def test_grouped_ffn_fp8_eight_wave_blocks(mode):
    """The eight-wave fp8 loop (K % 1024 == 0, whole 256-column output tiles): 256-row token blocks of one to
    eight 32-row sub-tiles, experts just over 256 rows split into two near-equal blocks, empty experts. d = 3072
    gives the gate/up K loop three token-scale windows (an odd count, so the window slots alternate across the
    four output-column tiles a unit streams); I = 2048 gives down two windows and d / 256 = 12 output tiles
    (three units of four). H codes and scales are compared as well."""
    cfg = get_config("c2", gemm="fp8", n_routed=10, n_groups=1, topk_groups=1, T=1024, topk=2, d=3072, inter=2048)
    inp = generate(cfg, DEV)
    sh = B.moe_shape.of(cfg)
    sizes = [0, 1, 31, 33, 129, 255, 256, 257, 300, 520]
    off = np.concatenate([[0], np.cumsum(sizes)])
    n = int(off[-1])
    assert n <= cfg.T * cfg.topk
    src = np.random.default_rng(29).integers(0, cfg.T, n)
    u32 = inp["u"].cpu().float().numpy()
    uq, us = oracle.quantize_tiles(u32)
    wq = [oracle_wq(cfg, inp, e) for e in range(cfg.n_routed)]
    dev8 = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    wgu = dev8(np.stack([tile_e4m3(w[0], True) for w in wq])); wgs = dev8(np.stack([w[1] for w in wq]))
    wdn = dev8(np.stack([tile_e4m3(w[2], False) for w in wq])); wds = dev8(np.stack([w[3] for w in wq]))
    h = torch.empty((n + 1, cfg.inter), dtype=torch.uint8, device=DEV)
    hs = torch.empty((n + 1, cfg.inter // 128), dtype=torch.float32, device=DEV)
    h[n] = 0x5A
    hs[n] = 3.0
    y = torch.full((n + 1, cfg.d), 7.0, dtype=torch.bfloat16, device=DEV)
    if mode == "gather":
        a, a_s, a_rows, rmode, rsrc = dev8(uq), dev8(us), cfg.T, B.MOE_ROWS_GATHER, _i32(src)
    else:
        a, a_s, a_rows, rmode, rsrc = dev8(uq[src]), dev8(us[src]), n, B.MOE_ROWS_DIRECT, None
    ws = torch.empty(256, dtype=torch.uint8, device=DEV)
    B.moe_ffn_gate_up(sh, B.MOE_F8E4M3, cfg.n_routed, n, _i32(off), rmode, rsrc, a, a_s, a_rows, wgu, wgs, h[:n],
                      hs[:n], ws)
    B.moe_ffn_down(sh, B.MOE_F8E4M3, cfg.n_routed, n, _i32(off), h[:n], hs[:n], wdn, wds, y[:n], ws)
    torch.cuda.synchronize()
    # nothing past the last row is written
    assert torch.all(h[n] == 0x5A) and torch.all(hs[n] == 3.0) and torch.all(y[n] == 7.0)
    for e in range(cfg.n_routed):
        lo, hi = off[e], off[e + 1]
        if hi == lo:
            continue
        ref, aux = oracle.ffn_fp8(u32[src[lo:hi]], *wq[e], return_h=True)
        report(f"fp8 eight-wave {mode} expert {e} ({hi - lo} rows) y", rel_l2(y[lo:hi], ref), TOL["fp8"])
        same = float(np.mean(h[lo:hi].cpu().numpy() == aux["h_codes"]))
        sdiff = np.max(np.abs(hs[lo:hi].cpu().numpy() / aux["h_scale"] - 1))
        print(f"[parity] expert {e}: H codes equal {same:.4f}, max rel scale diff {sdiff:.2e}")
        assert same > 0.99 and sdiff < 1e-4


@pytest.mark.parametrize("d,inter", [(10240, 256), (256, 10240)])
def test_grouped_ffn_fp8_max_k(d, inter):
    """fp8 at the largest supported K, 10240 = 80 chunks of 128: in the gate/up projection (d) and in the down
    projection (inter), with an empty expert between two ragged ones."""
    cfg = get_config("c2", gemm="fp8", n_routed=3, n_groups=1, topk_groups=1, T=256, topk=1, d=d, inter=inter)
    inp = generate(cfg, DEV)
    sh = B.moe_shape.of(cfg)
    sizes = [77, 0, 179]
    off = np.concatenate([[0], np.cumsum(sizes)])
    n = int(off[-1])
    src = np.random.default_rng(31).integers(0, cfg.T, n)
    u32 = inp["u"].cpu().float().numpy()
    uq, us = oracle.quantize_tiles(u32)
    wq = [oracle_wq(cfg, inp, e) for e in range(cfg.n_routed)]
    dev8 = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    wgu = dev8(np.stack([tile_e4m3(w[0], True) for w in wq])); wgs = dev8(np.stack([w[1] for w in wq]))
    wdn = dev8(np.stack([tile_e4m3(w[2], False) for w in wq])); wds = dev8(np.stack([w[3] for w in wq]))
    h = torch.empty((n, inter), dtype=torch.uint8, device=DEV)
    hs = torch.empty((n, inter // 128), dtype=torch.float32, device=DEV)
    y = torch.empty((n, d), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(256, dtype=torch.uint8, device=DEV)
    B.moe_ffn_gate_up(sh, B.MOE_F8E4M3, cfg.n_routed, n, _i32(off), B.MOE_ROWS_GATHER, _i32(src), dev8(uq), dev8(us),
                      cfg.T, wgu, wgs, h, hs, ws)
    B.moe_ffn_down(sh, B.MOE_F8E4M3, cfg.n_routed, n, _i32(off), h, hs, wdn, wds, y, ws)
    torch.cuda.synchronize()
    for e in (0, 2):
        lo, hi = off[e], off[e + 1]
        ref = oracle.ffn_fp8(u32[src[lo:hi]], *wq[e])
        report(f"fp8 d={d} I={inter} expert {e} ({hi - lo} rows) y", rel_l2(y[lo:hi], ref), TOL["fp8"])


@pytest.mark.parametrize("d", [384, 640])
def test_grouped_ffn_fp8_half_column_tile(d):
    """fp8 with d % 256 == 128: the last 128 output columns form a unit of their own (rows past d read as zero,
    no weight-block scale, no store past the row); d also sets the gate/up K loop to 3 or 5 chunks."""
    cfg = get_config("c2", gemm="fp8", n_routed=4, n_groups=1, topk_groups=1, T=512, topk=2, d=d, inter=256)
    inp = generate(cfg, DEV)
    sh = B.moe_shape.of(cfg)
    sizes = [0, 40, 300, 129]
    off = np.concatenate([[0], np.cumsum(sizes)])
    n = int(off[-1])
    src = np.random.default_rng(6).integers(0, cfg.T, n)
    u32 = inp["u"].cpu().float().numpy()
    uq, us = oracle.quantize_tiles(u32)
    wq = [oracle_wq(cfg, inp, e) for e in range(cfg.n_routed)]
    dev8 = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    wgu = dev8(np.stack([tile_e4m3(w[0], True) for w in wq])); wgs = dev8(np.stack([w[1] for w in wq]))
    wdn = dev8(np.stack([tile_e4m3(w[2], False) for w in wq])); wds = dev8(np.stack([w[3] for w in wq]))
    h = torch.empty((n, cfg.inter), dtype=torch.uint8, device=DEV)
    hs = torch.empty((n, cfg.inter // 128), dtype=torch.float32, device=DEV)
    y = torch.full((n + 1, d), 7.0, dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(256, dtype=torch.uint8, device=DEV)
    B.moe_ffn_gate_up(sh, B.MOE_F8E4M3, 4, n, _i32(off), B.MOE_ROWS_GATHER, _i32(src), dev8(uq), dev8(us), cfg.T,
                      wgu, wgs, h, hs, ws)
    B.moe_ffn_down(sh, B.MOE_F8E4M3, 4, n, _i32(off), h, hs, wdn, wds, y[:n], ws)
    torch.cuda.synchronize()
    assert torch.all(y[n] == 7.0)
    for e in range(4):
        lo, hi = off[e], off[e + 1]
        if hi > lo:
            ref = oracle.ffn_fp8(u32[src[lo:hi]], *wq[e])
            report(f"fp8 d={d} expert {e} ({hi - lo} rows) y", rel_l2(y[lo:hi], ref), TOL["fp8"])


def test_fp8_accumulation_k4096():
    """The pages' K = 4096 experiment on this path: E4M3 operands (unit scales) through the fp8 down GEMM
    accumulate at fp32 grade -- the bf16 output equals the exact product rounded to bf16 almost everywhere --
    while the limited-precision accumulator of the pages' reading shows ~2% error on the same matrices."""
    M, Dout, K = 64, 128, 4096
    cfg = get_config("c2", gemm="fp8", n_routed=1, n_groups=1, topk_groups=1, group_topn=1, topk=1, T=M, d=Dout,
                     inter=K)
    sh = B.moe_shape.of(cfg)
    rng = np.random.default_rng(41)
    ha = oracle.e4m3_encode(rng.standard_normal((M, K)).astype(np.float32))
    wb = oracle.e4m3_encode(rng.standard_normal((Dout, K)).astype(np.float32))
    A, W = oracle.e4m3_decode(ha), oracle.e4m3_decode(wb)
    exact = A @ W.T
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    y = torch.empty((M, Dout), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(256, dtype=torch.uint8, device=DEV)
    B.moe_ffn_down(sh, B.MOE_F8E4M3, 1, M, _i32(np.array([0, M])), dev(ha), dev(np.ones((M, K // 128), np.float32)),
                   dev(tile_e4m3(wb, False)[None]), dev(np.ones((1, Dout // 128, K // 128), np.float32)), y, ws)
    torch.cuda.synchronize()
    yg = np64(y)
    rounded = torch.from_numpy(exact).to(torch.bfloat16).double().numpy()
    same = float(np.mean(yg == rounded))
    err = np.abs(yg - exact).max() / np.abs(exact).max()
    lim = oracle.limited_precision_gemm(A, W)
    err_lim = np.abs(lim - exact).max() / np.abs(exact).max()
    # fp32 accumulation in any order errs by at most K * 2^-24 * sum |a_k w_k| (recursive-summation
    # bound); the bf16 output adds at most one ulp of the value (8 significant bits)
    ulp = np.ldexp(1.0, np.frexp(np.abs(exact))[1] - 8)
    bound = ulp + K * 2.0 ** -24 * (np.abs(A) @ np.abs(W).T)
    print(f"[parity] K=4096 fp8: GPU max err {err:.2e} (bf16 output), equal to rounded exact {same:.4f}, "
          f"max |err| / fp32 bound {np.max(np.abs(yg - exact) / bound):.3f}; limited-precision accumulator "
          f"{err_lim:.2e}")
    assert np.all(np.abs(yg - exact) <= bound) and same > 0.97 and err < 2.0 ** -8
    assert 0.01 < err_lim < 0.03


@pytest.mark.parametrize("inter", [1408, 2048])
def test_fp8_layer_two_phase_calls(inter):
    """The fp8 layer through the two-phase calls (moe_ffn_gate_up, moe_ffn_down) and the separate shared
    call, on the mid shape: token quantisation bit for bit, sampled experts with their H codes, the shared
    expert on 64 tokens and the output on 3 tokens. inter = 1408 sends the down projection to the four-wave
    loop (K % 1024 != 0), inter = 2048 both projections to the eight-wave one."""
    name = "c2"
    cfg, inp = _inputs(name, gemm="fp8", inter=inter)
    T, K, N, d = cfg.T, cfg.topk, cfg.n_routed, cfg.d
    layer = MoELayer(cfg, inp, DEV)
    layer.route(inp["u"])
    layer.permute(inp["u"])
    layer.ffn_routed_phases(inp["u"])       # keeps H codes for the diagnostic
    layer.ffn_shared(inp["u"])
    layer.combine(inp["u"])
    layer.bias_update()
    out = layer.out
    torch.cuda.synchronize()
    r = _oracle_route(cfg, inp)
    bad = routing_mismatches(layer.topk_idx, r)
    # token quantisation is bit-exact with the oracle's 1x128 rule
    codes, scale = oracle.quantize_tiles(inp["u"].cpu().float().numpy())
    assert np.array_equal(layer.u_q.cpu().numpy(), codes)
    assert np.array_equal(layer.u_scale.cpu().numpy(), scale)
    load = r["load"]
    experts = sorted({0, N - 1, int(np.argmax(load)), int(np.argmin(load)), N // 3})
    _check_fp8_experts(cfg, inp, layer, experts, name)
    u32 = inp["u"].cpu().float().numpy()
    sample = np.random.default_rng(0).choice(T, 64, replace=False)
    sq = oracle_wq(cfg, inp, 0, shared=True)
    ref_sh = oracle.ffn_fp8(u32[sample], *sq)
    report(f"{name} fp8 shared y (64 tokens)", rel_l2(layer.y_shared[torch.from_numpy(sample).to(DEV)], ref_sh),
           TOL["fp8"])
    n_tok = 3 if T <= 4096 else 1
    toks = [t for t in np.random.default_rng(1).choice(T, 6, replace=False) if t not in set(bad)][:n_tok]
    u64 = np64(inp["u"])
    for t in toks:
        acc = u64[t].copy()
        for sh_e in range(cfg.n_shared):
            acc = acc + oracle.ffn_fp8(u32[[t]], *oracle_wq(cfg, inp, sh_e, shared=True))[0]
        for k in range(K):
            e = int(r["idx"][t, k])
            acc = acc + r["gate"][t, k] * oracle.ffn_fp8(u32[[t]], *oracle_wq(cfg, inp, e))[0]
        report(f"{name} fp8 out-u token {t}", rel_l2(np64(out[t]) - u64[t], acc - u64[t]), TOL["fp8"])
