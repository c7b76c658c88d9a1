"""GPU parity of the MXFP4 expert-weight path (E2M1 weights with E8M0 1x32 scales, E4M3 activations)
against the CPU oracle: the weight quantiser bit for bit, the grouped FFN on every block shape, the
FP4 -> FP8 lossless conversion served through the fp8 kernels, and the layer on sampled experts."""
import numpy as np
import pytest
import torch

import oracle
from moe_inputs import generate, generate_expert, get_config
from mixture_experts_layer_gate_amd import binding as B
from mixture_experts_layer_gate_amd import MoELayer
from parity import TOL, np64, npi, rel_l2, report, routing_mismatches, tile_e4m3, tile_mxfp4

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _i32(x):
    return torch.as_tensor(np.asarray(x), dtype=torch.int32, device=DEV).contiguous()


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def _oracle_mx(w, gate_up):
    """Oracle MXFP4 of one matrix [R, K] in the library's tiled layout, plus the oracle's own (codes, scales)."""
    codes, scales = oracle.quantize_mxfp4(w)
    tc, ts = tile_mxfp4(codes, scales, gate_up, oracle.pack_e2m1)
    return tc, ts, (codes, scales)


def _edge_rows(K):
    """bf16-exact rows that probe the E2M1 encode: with amax 5 (scale 2^0) every decision point and its
    neighbours; a saturating row (amax 7.5 -> 6); an all-zero block; -0 and tiny values; very small and very
    large magnitudes (scales 2^-127 .. 2^100)."""
    pts = [0.0, 0.25, 0.5, 0.75, 1.0, 1.25, 1.5, 1.75, 2.0, 2.5, 3.0, 3.5, 4.0, 5.0]
    near = [p * (1 + s * 2.0 ** -6) for p in pts[1:] for s in (-1, 1)]
    base = np.array(pts + near + [-p for p in pts + near] + [-0.0, 1e-20, -1e-20], dtype=np.float64)
    rows = []
    r0 = np.resize(base, K); r0[::32] = 5.0
    rows.append(r0)
    r1 = np.resize(base * 1.5, K); r1[::32] = 7.5
    rows.append(r1)
    r2 = np.resize(base, K); r2[:32] = 0.0; r2[32::32] = 5.0
    rows.append(r2)
    rows.append(np.resize(base, K) * 2.0 ** -122)     # amax 5 * 2^-122: k = -122
    rows.append(np.resize(base, K) * 2.0 ** -130)     # amax 5 * 2^-130: k clamps at -127
    rows.append(np.resize(base, K) * 2.0 ** 100)
    return np.stack(rows)


@pytest.mark.parametrize("shape,gate_up", [((3, 256, 512), False), ((2, 384, 256), False), ((2, 512, 384), True)])
def test_quantize_weights_mxfp4_bit_exact(shape, gate_up):
    """Codes and scales in the tiled layout, bit for bit: random weights plus edge rows (every E2M1 decision
    point, saturation, an all-zero block, -0, scales from 2^-127 to 2^100); a 384-row matrix pads its second
    tile; gate_up = 1 interleaves gate and up rows per 128 H columns."""
    rng = np.random.default_rng(31)
    n, R, K = shape
    w = (rng.standard_normal(shape) * 0.02).astype(np.float32)
    w[1, :6] = _edge_rows(K)
    w[1, R - 6:] = _edge_rows(K)[::-1]
    wb = torch.from_numpy(w).to(torch.bfloat16)
    w32 = wb.float().numpy()
    Rt = -(-R // 256) * 256
    codes = torch.empty((n, Rt * K // 2,), dtype=torch.uint8, device=DEV)
    scales = torch.empty((n, Rt * K // 32), dtype=torch.uint8, device=DEV)
    B.moe_quantize_weights_mxfp4(wb.to(DEV), codes, scales, gate_up=gate_up)
    torch.cuda.synchronize()
    gc, gs = codes.cpu().numpy(), scales.cpu().numpy()
    for i in range(n):
        tc, ts, _ = _oracle_mx(w32[i], gate_up)
        assert np.array_equal(gs[i], ts), i
        assert np.array_equal(gc[i], tc), i


def _mx_ffn_case(cfg, sizes, seed, mode):
    """Oracle-quantised activations and MXFP4 weights of cfg's routed experts; runs the two FFN calls."""
    inp = generate(cfg, DEV)
    sh = B.moe_shape.of(cfg)
    off = np.concatenate([[0], np.cumsum(sizes)])
    n = int(off[-1])
    src = np.random.default_rng(seed).integers(0, cfg.T, n)
    u32 = inp["u"].cpu().float().numpy()
    uq, us = oracle.quantize_tiles(u32)
    mg = [_oracle_mx(inp["w_gate_up"][e].cpu().float().numpy(), True) for e in range(cfg.n_routed)]
    md = [_oracle_mx(inp["w_down"][e].cpu().float().numpy(), False) for e in range(cfg.n_routed)]
    wgu, wgs = _dev(np.stack([m[0] for m in mg])), _dev(np.stack([m[1] for m in mg]))
    wdn, wds = _dev(np.stack([m[0] for m in md])), _dev(np.stack([m[1] for m in md]))
    I, d = cfg.inter, cfg.d
    h = torch.empty((n, I), dtype=torch.uint8, device=DEV)
    hs = torch.empty((n, I // 128), dtype=torch.float32, device=DEV)
    y = torch.empty((n, d), dtype=torch.bfloat16, device=DEV)
    if mode == "gather":
        a, a_s, a_rows, rmode, rsrc = _dev(uq), _dev(us), cfg.T, B.MOE_ROWS_GATHER, _i32(src)
    else:
        a, a_s, a_rows, rmode, rsrc = _dev(uq[src]), _dev(us[src]), n, B.MOE_ROWS_DIRECT, None
    ws = torch.empty(256, dtype=torch.uint8, device=DEV)
    B.moe_ffn_gate_up(sh, B.MOE_F4E2M1, cfg.n_routed, n, _i32(off), rmode, rsrc, a, a_s, a_rows, wgu, wgs, h, hs, ws)
    B.moe_ffn_down(sh, B.MOE_F4E2M1, cfg.n_routed, n, _i32(off), h, hs, wdn, wds, y, ws)
    torch.cuda.synchronize()
    return dict(off=off, src=src, u32=u32, mg=mg, md=md, h=h, hs=hs, y=y, inp=inp, n=n)


def _check_mx_experts(cfg, r, tag):
    off, src = r["off"], r["src"]
    for e in range(cfg.n_routed):
        lo, hi = off[e], off[e + 1]
        if hi == lo:
            continue
        ref, aux = oracle.ffn_mxfp4(r["u32"][src[lo:hi]], *r["mg"][e][2], *r["md"][e][2], return_h=True)
        report(f"mxfp4 {tag} expert {e} ({hi - lo} rows) y", rel_l2(r["y"][lo:hi], ref), TOL["mxfp4"])
        same = float(np.mean(r["h"][lo:hi].cpu().numpy() == aux["h_codes"]))
        sdiff = np.max(np.abs(r["hs"][lo:hi].cpu().numpy() / aux["h_scale"] - 1))
        print(f"[parity] mxfp4 {tag} expert {e}: H codes equal {same:.4f}, max rel scale diff {sdiff:.2e}")
        assert same > 0.99 and sdiff < 1e-4


@pytest.mark.parametrize("inter,mode", [(128, "gather"), (1408, "gather"), (1408, "direct")])
def test_grouped_ffn_mxfp4_tile_shapes(inter, mode):
    """Expert segments that reach every block shape (empty, 1 row, 1..4 sub-tiles, split blocks); inter = 128
    gives the down projection one K chunk, 1408 an odd number (11)."""
    cfg = get_config("c2", gemm="mxfp4", n_routed=10, n_groups=1, topk_groups=1, T=1024, topk=2, inter=inter)
    sizes = [0, 1, 32, 64, 65 + 30, 128, 160, 288, 0, 416]
    _check_mx_experts(cfg, _mx_ffn_case(cfg, sizes, 23, mode), f"I={inter} {mode}")


@pytest.mark.parametrize("d,inter", [(384, 256), (640, 256), (640, 128)])
def test_grouped_ffn_mxfp4_half_column_tile(d, inter):
    """d % 256 == 128: the last 128 output columns form a unit of their own (code rows past d read as zero,
    scale loads clamped inside the expert's scales, no store past the row). With inter = 128 that unit's
    down stream is two stages long, the shortest the seven-stage ring's prologue handles."""
    cfg = get_config("c2", gemm="mxfp4", n_routed=4, n_groups=1, topk_groups=1, T=512, topk=2, d=d, inter=inter)
    _check_mx_experts(cfg, _mx_ffn_case(cfg, [0, 40, 300, 129], 6, "gather"), f"d={d} inter={inter}")


def test_grouped_ffn_mxfp4_gather_near_4gib():
    """The MXFP4 gate/up gathers E4M3 token rows through 32-bit byte offsets: codes of a_rows * d bytes just under
    4 GiB (a_rows = 599,186 at d = 7168, the most the call accepts), rows picked at both ends, three experts. Only
    the picked rows hold data (seeded N(0, 1) rows quantised by the oracle's 1x128 rule); the rest are zero codes
    with scale 1 and are never read. y and the H codes against the oracle."""
    d, I, E = 7168, 1024, 3
    a_rows = ((1 << 32) - 1) // d
    cfg = get_config("c2", gemm="mxfp4", d=d, inter=I, n_routed=E, n_groups=1, topk_groups=1, T=128, topk=1,
                     n_shared=0)
    inp = generate(cfg, DEV)
    sh = B.moe_shape.of(cfg)
    sizes = [40, 33, 23]
    off = np.concatenate([[0], np.cumsum(sizes)])
    n = int(off[-1])
    rng = np.random.default_rng(17)
    mid = rng.choice(np.arange(16, a_rows - 48), n - 64, replace=False)
    src = np.concatenate([np.arange(a_rows - 48, a_rows), np.arange(0, 16), mid])
    rng.shuffle(src)
    u32 = rng.standard_normal((n, d)).astype(np.float32)        # row i of u32 is token row src[i]
    uq, us = oracle.quantize_tiles(u32)
    a = torch.zeros((a_rows, d), dtype=torch.uint8, device=DEV)
    a_s = torch.ones((a_rows, d // 128), dtype=torch.float32, device=DEV)
    si = torch.from_numpy(src).to(DEV)
    a[si] = _dev(uq)
    a_s[si] = _dev(us)
    mg = [_oracle_mx(inp["w_gate_up"][e].cpu().float().numpy(), True) for e in range(E)]
    md = [_oracle_mx(inp["w_down"][e].cpu().float().numpy(), False) for e in range(E)]
    wgu, wgs = _dev(np.stack([m[0] for m in mg])), _dev(np.stack([m[1] for m in mg]))
    wdn, wds = _dev(np.stack([m[0] for m in md])), _dev(np.stack([m[1] for m in md]))
    h = torch.empty((n, I), dtype=torch.uint8, device=DEV)
    hs = torch.empty((n, I // 128), dtype=torch.float32, device=DEV)
    y = torch.empty((n, d), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(256, dtype=torch.uint8, device=DEV)
    B.moe_ffn_gate_up(sh, B.MOE_F4E2M1, E, n, _i32(off), B.MOE_ROWS_GATHER, _i32(src), a, a_s, a_rows, wgu, wgs, h,
                      hs, ws)
    B.moe_ffn_down(sh, B.MOE_F4E2M1, E, n, _i32(off), h, hs, wdn, wds, y, ws)
    torch.cuda.synchronize()
    for e in range(E):
        lo, hi = off[e], off[e + 1]
        ref, aux = oracle.ffn_mxfp4(u32[lo:hi], *mg[e][2], *md[e][2], return_h=True)
        report(f"mxfp4 a near 4 GiB, expert {e} ({hi - lo} rows) y", rel_l2(y[lo:hi], ref), TOL["mxfp4"])
        same = float(np.mean(h[lo:hi].cpu().numpy() == aux["h_codes"]))
        print(f"[parity] mxfp4 expert {e}: H codes equal {same:.4f}")
        assert same > 0.99


def test_ffn_down_mxfp4_h_near_4gib():
    """MXFP4 down projection on n_rows * inter bytes of E4M3 H codes just under 4 GiB (n_rows = 2,097,151 at
    inter = 2048, the most the call accepts; d = 1024), two experts; sampled rows at the start, the expert boundary
    and the end against the oracle on the dequantised operands. H: seeded random finite E4M3 codes (magnitude codes
    0 .. 0x7E, either sign) with 1x128 scales ~ U(1e-3, 2e-3); W_d: the oracle's MXFP4 of N(0, 0.02^2) weights."""
    d, I, E = 1024, 2048, 2
    n = ((1 << 32) - 1) // I
    cfg = get_config("c2", gemm="mxfp4", T=128, d=d, inter=I, n_routed=E, n_groups=1, topk_groups=1, topk=1,
                     n_shared=0)
    sh = B.moe_shape.of(cfg)
    gen = torch.Generator(device=DEV).manual_seed(779)
    h = torch.randint(0, 0x7F, (n, I), generator=gen, device=DEV, dtype=torch.uint8)
    h |= (torch.randint(0, 2, (n, I), generator=gen, device=DEV, dtype=torch.uint8) << 7)
    hs = torch.rand((n, I // 128), generator=gen, device=DEV) * 1e-3 + 1e-3
    w32 = (np.random.default_rng(6).standard_normal((E, d, I)) * 0.02).astype(np.float32)
    md = [_oracle_mx(w32[e], False) for e in range(E)]
    wdn, wds = _dev(np.stack([m[0] for m in md])), _dev(np.stack([m[1] for m in md]))
    off = np.array([0, n // 2 + 3, n])
    rows = np.unique(np.concatenate([np.arange(0, 16), np.arange(off[1] - 16, off[1] + 16), np.arange(n - 16, n),
                                     np.random.default_rng(7).integers(0, n, 32)]))
    sel = torch.from_numpy(rows).to(DEV)
    h64 = oracle.dequantize_tiles(h[sel].cpu().numpy(), hs[sel].cpu().numpy())
    wd64 = np.stack([oracle.dequantize_mxfp4(*m[2]) for m in md])
    ws = torch.empty(256, dtype=torch.uint8, device=DEV)
    y = torch.empty((n, d), dtype=torch.bfloat16, device=DEV)
    B.moe_ffn_down(sh, B.MOE_F4E2M1, E, n, _i32(off), h, hs, wdn, wds, y, ws)
    torch.cuda.synchronize()
    for e in range(E):
        r = rows[(rows >= off[e]) & (rows < off[e + 1])]
        ref = h64[np.searchsorted(rows, r)] @ wd64[e].T
        report(f"mxfp4 H near 4 GiB expert {e} ({r.size} sampled rows) y", rel_l2(y[torch.from_numpy(r).to(DEV)], ref),
               TOL["mxfp4"])


def test_mxfp4_through_fp8_kernels_on_lossless_conversion():
    """The pages' lossless FP4 -> FP8 conversion, on the GPU: the same MXFP4 weights converted by the oracle to
    E4M3 128x128 blocks and run through the fp8 kernels give the native MXFP4 kernels' results (both multiply
    the same exact weight values; only the fp32 rounding of the scaled sums differs)."""
    cfg = get_config("c2", gemm="mxfp4", n_routed=4, n_groups=1, topk_groups=1, T=512, topk=2, inter=512)
    r = _mx_ffn_case(cfg, [100, 0, 257, 155], 9, "gather")
    sh = B.moe_shape.of(cfg)
    conv_g = [oracle.mxfp4_to_e4m3_blocks(*m[2]) for m in r["mg"]]
    conv_d = [oracle.mxfp4_to_e4m3_blocks(*m[2]) for m in r["md"]]
    assert all(np.all(c[2]) for c in conv_g + conv_d)
    wgu, wgs = _dev(np.stack([tile_e4m3(c[0], True) for c in conv_g])), _dev(np.stack([c[1] for c in conv_g]))
    wdn, wds = _dev(np.stack([tile_e4m3(c[0], False) for c in conv_d])), _dev(np.stack([c[1] for c in conv_d]))
    n, off, src = r["n"], r["off"], r["src"]
    uq, us = oracle.quantize_tiles(r["u32"])
    h8 = torch.empty_like(r["h"]); hs8 = torch.empty_like(r["hs"]); y8 = torch.empty_like(r["y"])
    ws = torch.empty(256, dtype=torch.uint8, device=DEV)
    B.moe_ffn_gate_up(sh, B.MOE_F8E4M3, cfg.n_routed, n, _i32(off), B.MOE_ROWS_GATHER, _i32(src), _dev(uq), _dev(us),
                      cfg.T, wgu, wgs, h8, hs8, ws)
    B.moe_ffn_down(sh, B.MOE_F8E4M3, cfg.n_routed, n, _i32(off), h8, hs8, wdn, wds, y8, ws)
    torch.cuda.synchronize()
    same = float((h8 == r["h"]).float().mean())
    err = rel_l2(y8, np64(r["y"]))
    print(f"[parity] fp8 kernels on converted MXFP4 weights vs native MXFP4: H codes equal {same:.5f}, "
          f"y rel_l2 {err:.2e}")
    assert same > 0.999 and err < 2e-3


@pytest.mark.parametrize("name", ["c2", "c5"])
def test_mxfp4_layer_sampled(name):
    """The layer with MXFP4 expert weights (quantised on the GPU): token quantisation bit-exact, weight codes
    of sampled experts bit-exact, sampled experts' rows and tokens' outputs against the oracle."""
    cfg = get_config(name, gemm="mxfp4")
    inp = generate(cfg, DEV)
    T, K, N = cfg.T, cfg.topk, cfg.n_routed
    layer = MoELayer(cfg, inp, DEV)
    out = layer.forward(inp["u"])
    torch.cuda.synchronize()
    r = oracle.route(inp["u"], inp["centroids"], inp["bias"], cfg.n_groups, cfg.topk_groups, cfg.group_topn, K)
    bad = routing_mismatches(layer.topk_idx, r)
    u32 = inp["u"].cpu().float().numpy()
    codes, scale = oracle.quantize_tiles(u32)
    assert np.array_equal(layer.u_q.cpu().numpy(), codes) and np.array_equal(layer.u_scale.cpu().numpy(), scale)
    load = r["load"]
    experts = sorted({0, int(np.argmax(load)), N - 1})
    goff, gperm = npi(layer.expert_offsets), npi(layer.perm_token)
    mq = {}
    for e in experts:
        g = _oracle_mx(inp["w_gate_up"][e].cpu().float().numpy(), True)
        dn = _oracle_mx(inp["w_down"][e].cpu().float().numpy(), False)
        assert np.array_equal(layer.w["w_gate_up"][e].cpu().numpy().reshape(-1), g[0])
        assert np.array_equal(layer.w["w_gate_up_scale"][e].cpu().numpy().reshape(-1), g[1])
        assert np.array_equal(layer.w["w_down"][e].cpu().numpy().reshape(-1), dn[0])
        assert np.array_equal(layer.w["w_down_scale"][e].cpu().numpy().reshape(-1), dn[1])
        mq[e] = (*g[2], *dn[2])
        lo, hi = goff[e], goff[e + 1]
        if hi > lo:
            ref = oracle.ffn_mxfp4(u32[gperm[lo:hi]], *mq[e])
            report(f"{name} mxfp4 expert {e} ({hi - lo} rows) y", rel_l2(layer.y_routed[lo:hi], ref), TOL["mxfp4"])
    shq = []
    for si in range(cfg.n_shared):
        sg = _oracle_mx(inp["s_gate_up"][si].cpu().float().numpy(), True)
        sd = _oracle_mx(inp["s_down"][si].cpu().float().numpy(), False)
        shq.append((*sg[2], *sd[2]))
    sample = np.random.default_rng(0).choice(T, min(T, 64), replace=False)
    ref_sh = oracle.ffn_mxfp4(u32[sample], *shq[0])
    report(f"{name} mxfp4 shared y ({len(sample)} tokens)",
           rel_l2(layer.y_shared[torch.from_numpy(sample).to(DEV)], ref_sh), TOL["mxfp4"])
    u64 = np64(inp["u"])
    n_tok = 2 if T <= 4096 else 1
    toks = [t for t in np.random.default_rng(1).choice(T, 6, replace=False) if t not in set(bad)][:n_tok]
    for t in toks:
        acc = u64[t].copy()
        for q in shq:
            acc = acc + oracle.ffn_mxfp4(u32[[t]], *q)[0]
        for k in range(K):
            e = int(r["idx"][t, k])
            if e not in mq:
                g = _oracle_mx(inp["w_gate_up"][e].cpu().float().numpy(), True)
                dn = _oracle_mx(inp["w_down"][e].cpu().float().numpy(), False)
                mq[e] = (*g[2], *dn[2])
            acc = acc + r["gate"][t, k] * oracle.ffn_mxfp4(u32[[t]], *mq[e])[0]
        report(f"{name} mxfp4 out-u token {t}", rel_l2(np64(out[t]) - u64[t], acc - u64[t]), TOL["mxfp4"])
