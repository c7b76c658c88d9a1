"""The five workloads end to end on the GPU against the CPU oracle, one test each (two for the tiny one).

Each test runs the layer the way the library's users run it (``MoELayer.step``: route, permute, one
grouped FFN call over routed and shared experts, combine, bias update) and checks:

* routing against the oracle: expert indices, loads, offsets, permutation and row_of bit for bit,
  except tokens whose oracle K-th / (K+1)-th biased scores (or M-th / (M+1)-th group scores) are closer
  than 1e-6, which are counted and reported;
* the bias after the step bit for bit ("DeepSeek_V3_Report: Annotation", auxiliary-loss-free load
  balancing: the step-end -gamma / +gamma rule);
* every routed expert's output rows and the shared experts' rows against the oracle's FFN of the same
  tokens, per expert and as a whole;
* the layer output of eq. (12) on every token without a near-tie flip, as out and as out - u (the
  residual dominates ||out||).

The V3-shaped and decode workloads run the oracle on every expert, split over the host's cores.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_common import DEV, inputs, oracle_experts, oracle_route, oracle_shared_all_rows
from moe_inputs import generate_tokens
from mixture_experts_layer_gate_amd import MoELayer
from parity import TOL, np64, npi, rel_l2, report, routing_mismatches

pytestmark = pytest.mark.gpu


def _check_routing(cfg, layer, r, b_before):
    """Selection, load, permutation and the step-end bias against the oracle; returns the flipped tokens."""
    N, K, T = cfg.n_routed, cfg.topk, cfg.T
    bad = routing_mismatches(layer.topk_idx, r)
    gidx = npi(layer.topk_idx)
    assert np.all(np.diff(gidx, axis=1) > 0), "topk_idx must be ascending per token"
    load = npi(layer.expert_load)
    assert np.array_equal(load, np.bincount(gidx.ravel(), minlength=N))
    S = N // cfg.n_groups
    assert max(len(set(row)) for row in (gidx // S)) <= cfg.topk_groups
    if bad.size == 0:
        o_off, o_perm, o_row = oracle.permute(r["idx"], N)
        assert np.array_equal(load, r["load"])
        assert np.array_equal(npi(layer.expert_offsets), o_off)
        assert np.array_equal(npi(layer.perm_token), o_perm)
        assert np.array_equal(npi(layer.row_of), o_row)
        load_ref = r["load"]
    else:
        # the selection differs from the oracle's only at exempt near-ties, where either choice is valid;
        # the update must then follow the selection actually made
        load_ref = load
    b_ref = oracle.bias_update(b_before, load_ref, T, K, cfg.gamma)
    assert np.array_equal(layer.bias.cpu().numpy(), b_ref), "bias after the step differs from the oracle's"
    return bad


def _snapshot(layer, r, u, bad, tag):
    """What the FFN and combine checks need from one step, copied to the host."""
    return dict(offsets=npi(layer.expert_offsets), perm=npi(layer.perm_token), y=layer.y_routed.cpu(),
                ysh=layer.y_shared.cpu() if layer.cfg.n_shared else None, out=layer.out.cpu(), r=r,
                u=u.cpu(), bad=bad, tag=tag)


def _expert_rows_and_out(cfg, inp, snaps):
    """Every routed expert's rows, the shared experts' rows and the layer output against the oracle, for
    one or more steps (one oracle pass over the experts serves all of them)."""
    T, K, N, d, Ns = cfg.T, cfg.topk, cfg.n_routed, cfg.d, cfg.n_shared
    tol = TOL[cfg.gemm]
    perms = [oracle.permute(sn["r"]["idx"], N) for sn in snaps]
    u32s = [sn["u"].to(torch.float32).numpy() for sn in snaps]
    req = {e: [u32[o_perm[o_off[e]:o_off[e + 1]]] for u32, (o_off, o_perm, _) in zip(u32s, perms)]
           for e in range(N)}
    ref = oracle_experts(cfg, inp, req, tag=" + ".join(sn["tag"] for sn in snaps))
    del req
    for i, sn in enumerate(snaps):
        tag, bad, u = sn["tag"], sn["bad"], sn["u"]
        o_off, o_perm, o_row = perms[i]
        y_ref = np.zeros((T * K, d))
        for e, blocks in ref.items():
            y_ref[o_off[e]:o_off[e + 1]] = blocks[i]
        ysh_ref = np.stack([oracle_shared_all_rows(cfg, inp, s, u) for s in range(Ns)]) if Ns else None
        # routed rows: the GPU row of (expert, token) found through the GPU's own permutation
        goff, gperm = sn["offsets"], sn["perm"]
        errs, gpu_rows, ref_rows = [], [], []
        for e in range(N):
            toks = o_perm[o_off[e]:o_off[e + 1]]
            seg = gperm[goff[e]:goff[e + 1]]
            if len(toks) == 0:
                continue
            if np.array_equal(toks, seg):
                g_idx, o_idx = goff[e] + np.arange(len(toks)), o_off[e] + np.arange(len(toks))
            else:                           # a near-tie flip moved tokens into or out of this expert
                common = np.intersect1d(toks, seg)
                g_idx = goff[e] + np.searchsorted(seg, common)
                o_idx = o_off[e] + np.searchsorted(toks, common)
            err = rel_l2(sn["y"][torch.from_numpy(g_idx)], y_ref[o_idx])
            errs.append((err, e, len(toks)))
            assert err <= tol, f"{tag} expert {e} ({len(toks)} rows): rel_l2 {err:.3e} > {tol:.0e}"
            gpu_rows.append(g_idx)
            ref_rows.append(o_idx)
        errs.sort()
        print(f"[parity] {tag}: {len(errs)} routed experts, rel_l2 min {errs[0][0]:.2e} median "
              f"{errs[len(errs) // 2][0]:.2e} max {errs[-1][0]:.2e} (expert {errs[-1][1]}, {errs[-1][2]} rows)")
        gr, orr = np.concatenate(gpu_rows), np.concatenate(ref_rows)
        report(f"{tag} all routed rows", rel_l2(sn["y"][torch.from_numpy(gr)], y_ref[orr]), tol)
        if Ns:
            report(f"{tag} shared rows", rel_l2(np64(sn["ysh"]).reshape(Ns, T, d), ysh_ref), tol)
        out_ref = oracle.combine(u, y_ref, o_row, sn["r"]["gate"], ysh_ref)
        del y_ref
        ok = np.ones(T, dtype=bool)
        ok[bad] = False
        u64, out = np64(u), np64(sn["out"])
        report(f"{tag} out ({int(ok.sum())} tokens)", rel_l2(out[ok], out_ref[ok]), tol)
        report(f"{tag} out - u ({int(ok.sum())} tokens)", rel_l2((out - u64)[ok], (out_ref - u64)[ok]), tol)


@pytest.mark.parametrize("gather", [True, False])
def test_c1_tiny_fp32_layer(gather):
    """Tiny fp32 layer: the whole layer against oracle.layer_forward at 1e-4."""
    cfg, inp = inputs("c1")
    layer = MoELayer(cfg, inp, DEV, gather_in_gemm=gather)
    b0 = layer.bias.cpu().numpy().copy()
    out = layer.step(inp["u"])
    torch.cuda.synchronize()
    res = oracle.layer_forward(cfg, inp)
    bad = _check_routing(cfg, layer, res["route"], b0)
    ok = np.ones(cfg.T, dtype=bool)
    ok[bad] = False
    u64 = np64(inp["u"])
    if bad.size == 0:
        report("c1 routed y", rel_l2(layer.y_routed, res["y"]), TOL["f32"])
    report("c1 out", rel_l2(np64(out)[ok], res["out"][ok]), TOL["f32"])
    report("c1 out - u", rel_l2((np64(out) - u64)[ok], (res["out"] - u64)[ok]), TOL["f32"])


def test_c2_mid_bf16_layer():
    """Mid bf16 layer (4096 tokens, 64 experts, top-6 of 3 groups, 2 shared experts): everything."""
    cfg, inp = inputs("c2")
    layer = MoELayer(cfg, inp, DEV)
    b0 = layer.bias.cpu().numpy().copy()
    layer.step(inp["u"])
    torch.cuda.synchronize()
    r = oracle_route(cfg, inp)
    bad = _check_routing(cfg, layer, r, b0)
    _expert_rows_and_out(cfg, inp, [_snapshot(layer, r, inp["u"], bad, "c2")])


@pytest.mark.timeout(900)
def test_c3_v3_bf16_layer():
    """DeepSeek-V3-shaped bf16 layer: all 256 routed experts' rows, the shared expert's 8192 rows and the
    output of every token against the fp64 oracle."""
    cfg, inp = inputs("c3")
    layer = MoELayer(cfg, inp, DEV)
    b0 = layer.bias.cpu().numpy().copy()
    layer.step(inp["u"])
    torch.cuda.synchronize()
    r = oracle_route(cfg, inp)
    bad = _check_routing(cfg, layer, r, b0)
    _expert_rows_and_out(cfg, inp, [_snapshot(layer, r, inp["u"], bad, "c3")])


@pytest.mark.timeout(900)
def test_c4_v3_fp8_layer():
    """The V3 shape with E4M3 expert GEMMs (1x128 activation tiles, 128x128 weight blocks, fp32 scales):
    the token quantisation bit for bit, then every expert's rows, the shared expert and every token's
    output against the quantisation-emulating oracle at 1e-2."""
    cfg, inp = inputs("c4")
    layer = MoELayer(cfg, inp, DEV)
    b0 = layer.bias.cpu().numpy().copy()
    layer.step(inp["u"])
    torch.cuda.synchronize()
    codes, scale = oracle.quantize_tiles(inp["u"].cpu().float().numpy())
    assert np.array_equal(layer.u_q.cpu().numpy(), codes)
    assert np.array_equal(layer.u_scale.cpu().numpy(), scale)
    r = oracle_route(cfg, inp)
    bad = _check_routing(cfg, layer, r, b0)
    _expert_rows_and_out(cfg, inp, [_snapshot(layer, r, inp["u"], bad, "c4")])


@pytest.mark.timeout(900)
def test_c5_v4pro_decode_fp8_ten_bias_steps():
    """Zipf-skewed V4-Pro-shaped decode batch in fp8, ten steps of route -> FFN -> combine -> bias update.

    Every step: selection, load and permutation against the oracle routed with the bias the layer holds
    (itself checked bit for bit after every step, so the trajectory is the oracle's), and the bias update
    bit for bit. Steps 0 and 9: every touched expert's rows and the output of every token."""
    cfg, inp = inputs("c5")
    T, K, N = cfg.T, cfg.topk, cfg.n_routed
    layer = MoELayer(cfg, inp, DEV)
    b_traj = inp["bias"].cpu().numpy().copy()     # the oracle's own trajectory while no flip intervenes
    flips, own, snaps = 0, True, []
    for step in range(cfg.steps):
        u = generate_tokens(cfg, DEV, step)
        b_before = layer.bias.cpu().numpy().copy()
        if own:
            assert np.array_equal(b_before, b_traj)
        layer.step(u)
        torch.cuda.synchronize()
        r = oracle_route(cfg, inp, u=u, bias=b_before)
        bad = _check_routing(cfg, layer, r, b_before)
        flips += bad.size
        b_traj = oracle.bias_update(b_traj, r["load"], T, K, cfg.gamma)
        own = own and bad.size == 0
        load = r["load"]
        print(f"[parity] c5 step {step}: experts touched {int((load > 0).sum())}, empty {int((load == 0).sum())}, "
              f"max load {int(load.max())}, flips {bad.size}", flush=True)
        if step in (0, cfg.steps - 1):
            snaps.append(_snapshot(layer, r, u, bad, f"c5 step {step}"))
    _expert_rows_and_out(cfg, inp, snaps)
    print(f"[parity] c5: {flips} exempt near-tie flips over {cfg.steps} steps; bias trajectory "
          f"{'identical to the oracle' if own else 'checked step by step'}; final |b| max "
          f"{np.abs(layer.bias.cpu().numpy()).max():.4f}")
