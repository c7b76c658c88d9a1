#!/usr/bin/env python3
"""MoE-layer forward throughput on one MI355X.

One step = one pass of the whole layer on one batch: moe_route, moe_permute,
the grouped FFN over the routed and the shared experts together
(moe_ffn_gate_up + moe_ffn_down), moe_combine and the step-end
moe_bias_update. Inputs (seeded synthetic tokens and random-init weights of
the workload's shape) are resident in HBM before the timed region; before
each timed step a 1 GiB scratch buffer is written (outside the timed region)
so that nothing of the step's inputs sits in the 256 MB Infinity Cache.

By default the line carries the DeepSeek-V3-shaped layer (T=8192, d=7168,
256 routed experts in 8 groups, top-8 of 4 groups, 1 shared expert, I=2048)
in bf16 as its value, and the same shape with E4M3 expert GEMMs (1x128
activation tiles, 128x128 weight blocks) as its "fp8" object; ``--config cN``
runs one workload.

The line holds the throughput, the roofline of the dominant kernel (the
gate/up launch, timed with HIP events on its launch stream; algorithmic bytes
from each step's own expert load), per-call times and HBM fractions, the
measured MFMA / HBM peaks and the CPU oracle timed on a bounded token sample.

``--backward`` times one training step of the layer instead: the forward
with the SwiGLU-input cache, the backward to du, the centroid and the
expert-weight gradients (moe_combine_backward, moe_ffn_backward,
moe_route_backward, moe_input_grad) and the bias update; no optimizer.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12               # bytes/s, MI355X published
# dense MFMA; E2M1 x E4M3 products run at the fp8 rate (the fp4 rate needs both operands in fp4/fp6)
MFMA_PEAK = {"bf16": 2.5e15, "fp8": 5.0e15, "mxfp4": 5.0e15, "f32": 157.3e12}
# weight bytes per element: bf16 2, E4M3 1 (+ one fp32 per 128x128 block), E2M1 1/2 + one E8M0 byte per 32
WEIGHT_BYTES = {"bf16": 2.0, "f32": 4.0, "fp8": 1.0 + 4.0 / 16384, "mxfp4": 0.5 + 1.0 / 32}
METRIC = "MoE-layer fwd tokens/s at V3 shape + % of MFMA peak (bf16, fp8)"
CALLS = ["route", "permute", "ffn_gate_up", "ffn_down", "combine", "bias_update"]
CALLS_TRAIN = ["route", "permute", "ffn_gate_up", "ffn_down", "combine", "combine_bwd", "ffn_bwd", "route_bwd",
               "input_grad", "bias_update"]
METRIC_TRAIN = "MoE-layer fwd+bwd tokens/s (gradients of u, centroids and expert weights)"


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default=None, choices=["c2", "c3", "c4", "c5"],
                    help="one workload (default: the V3-shaped layer in bf16, with its fp8 form as the 'fp8' "
                         "object of the same line)")
    ap.add_argument("--no-flush", action="store_true",
                    help="do not write the 1 GiB scratch buffer before each timed step")
    ap.add_argument("--batch-invariant", action="store_true",
                    help="router K split fixed by d, so per-token results do not depend on the batch")
    ap.add_argument("--mxfp4", action="store_true",
                    help="fp8 workloads: MXFP4 expert weights (E2M1 with E8M0 1x32 scales) instead of E4M3 blocks")
    ap.add_argument("--pow2-act-scales", action="store_true",
                    help="fp8: power-of-two scales on the up-projection input")
    ap.add_argument("--backward", action="store_true",
                    help="bf16 workloads: time the training step (forward + backward + bias update)")
    ap.add_argument("--cpu-sample", type=int, default=None,
                    help="tokens for the CPU oracle baseline (0: skip; default 128, 8 with --backward: "
                         "10-30 s of host work either way)")
    ap.add_argument("--graph", action="store_true",
                    help="forward workloads: also record the step into a HIP graph and time its replays (flushed "
                         "and synchronised like the eager steps); value and ms_per_step then come from the replays, "
                         "calls and roofline from the eager steps of the same run")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB before timing (HBM counter calibration)")
    args = ap.parse_args()
    if args.cpu_sample is None:
        args.cpu_sample = 8 if args.backward else 128
    return args


FFN_SOURCES = {"bf16": ["ffn_bf16.hip", "gemm_w8.h", "gemm_pipe.h", "sched.h", "common.h"],
               "fp8": ["ffn_fp8.hip", "ffn_epi8.h", "gemm_f8w.h", "gemm_pipe8.h", "gemm_pipe.h", "sched.h", "common.h"],
               "mxfp4": ["ffn_fp4.hip", "ffn_epi8.h", "gemm_pipe4.h", "gemm_pipe8.h", "gemm_pipe.h", "sched.h",
                         "common.h"]}


def sources_hash(gemm: str) -> str:
    """First 16 hex digits of the sha256 of the grouped-FFN kernel sources of this GEMM dtype."""
    import hashlib
    csrc = os.path.join(ROOT, "mixture_experts_layer_gate_amd", "csrc")
    files = FFN_SOURCES.get(gemm, [])
    return hashlib.sha256(b"".join(open(os.path.join(csrc, f), "rb").read() for f in files)).hexdigest()[:16]


def recorded_traffic(kernel: str, workload: str, gemm: str):
    """HBM bytes per launch from the committed counter summary, if the kernel is unchanged since."""
    import re
    h = sources_hash(gemm)
    pdir = os.path.join(ROOT, "profiles")
    for name in (sorted(os.listdir(pdir)) if os.path.isdir(pdir) else []):
        for line in open(os.path.join(ROOT, "profiles", name)):
            m = re.match(r"traffic-record: (\{.*\})", line.strip())
            if m:
                rec = json.loads(m.group(1))
                if rec["kernel"] == kernel and rec["workload"] == workload and rec["sources_sha256_16"] == h:
                    return rec["fetch_bytes"] + rec["write_bytes"]
    return None


def _probe_lib():
    """libmoe_probe.so: the peak probes, a measurement library of its own beside libmoe.so."""
    import ctypes
    path = os.path.join(ROOT, "mixture_experts_layer_gate_amd", "libmoe_probe.so")
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built: run __graft_entry__.build()")
    P = ctypes.CDLL(path)
    P.probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    P.probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    P.probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    return P


def measure_peaks(dev):
    """MFMA (bf16, E4M3), device-copy and read rates of this GPU from the probe library, timed with HIP events
    on the stream the probes are launched on."""
    import torch
    P = _probe_lib()
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def ok(rc):
        if rc != 0:
            raise RuntimeError(f"peak probe failed with status {rc}")

    seed = torch.arange(1, 65, dtype=torch.int32, device=dev)
    nb = P.probe_mfma_blocks()
    out = torch.empty(nb * 256, dtype=torch.float32, device=dev)
    res = {}
    for name, fp8, flop in (("mfma_bf16", 0, 32768), ("mfma_fp8", 1, 131072)):
        ok(P.probe_mfma(fp8, 100, seed.data_ptr(), out.data_ptr(), sp))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        iters = 4000
        e0.record(stream)
        ok(P.probe_mfma(fp8, iters, seed.data_ptr(), out.data_ptr(), sp))
        e1.record(stream)
        torch.cuda.synchronize()
        res[name + "_TFLOP/s"] = nb * 4 * iters * 8 * flop / (e0.elapsed_time(e1) / 1e3) / 1e12
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    ok(P.probe_copy(src.data_ptr(), dst.data_ptr(), src.numel(), sp))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(5):
        ok(P.probe_copy(src.data_ptr(), dst.data_ptr(), src.numel(), sp))
    e1.record(stream)
    torch.cuda.synchronize()
    res["hbm_copy_GB/s"] = 5 * 2 * src.numel() / (e0.elapsed_time(e1) / 1e3) / 1e9
    del dst
    big = torch.empty(4 << 30, dtype=torch.uint8, device=dev)      # 4 GiB: far past the 256 MB Infinity Cache
    acc = torch.empty(P.probe_read_blocks() * 256, dtype=torch.int32, device=dev)
    ok(P.probe_read(big.data_ptr(), big.numel(), acc.data_ptr(), sp))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(3):
        ok(P.probe_read(big.data_ptr(), big.numel(), acc.data_ptr(), sp))
    e1.record(stream)
    torch.cuda.synchronize()
    res["hbm_read_GB/s"] = 3 * big.numel() / (e0.elapsed_time(e1) / 1e3) / 1e9
    del src, big
    return res


def touched_experts(load):
    return int((load > 0).sum())


def cpu_baseline(cfg, inp, layer, n_tok):
    """The oracle, as it stands, on the first n_tok tokens of the same batch (host cores)."""
    import numpy as np
    import torch
    import oracle

    u = inp["u"][:n_tok].cpu()
    cent, bias = inp["centroids"].cpu(), inp["bias"].cpu()
    r0 = oracle.route(u, cent, bias, cfg.n_groups, cfg.topk_groups, cfg.group_topn, cfg.topk)
    need = sorted(set(int(e) for e in r0["idx"].ravel()))
    wg = {e: inp["w_gate_up"][e].cpu() for e in need}          # host copies fetched before timing
    wd = {e: inp["w_down"][e].cpu() for e in need}
    sg = [inp["s_gate_up"][s].cpu() for s in range(cfg.n_shared)]
    sd = [inp["s_down"][s].cpu() for s in range(cfg.n_shared)]
    t0 = time.perf_counter()
    r = oracle.route(u, cent, bias, cfg.n_groups, cfg.topk_groups, cfg.group_topn, cfg.topk)
    off, perm, row_of = oracle.permute(r["idx"], cfg.n_routed)
    u64 = u.double().numpy()
    y = np.zeros((n_tok * cfg.topk, cfg.d))
    for e in range(cfg.n_routed):
        lo, hi = off[e], off[e + 1]
        if hi > lo:
            y[lo:hi] = oracle.expert_ffn(u64[perm[lo:hi]], wg[e], wd[e], cfg.gemm)
    ysh = np.stack([oracle.expert_ffn(u64, sg[s], sd[s], cfg.gemm) for s in range(cfg.n_shared)])
    oracle.combine(u64, y, row_of, r["gate"], ysh)
    oracle.bias_update(bias.numpy(), r["load"], n_tok, cfg.topk, cfg.gamma)
    dt = time.perf_counter() - t0
    try:
        from threadpoolctl import threadpool_info
        blas = max((i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"), default=1)
    except Exception:  # pragma: no cover
        blas = 1
    return {"value": n_tok / dt, "unit": "tokens/s", "cores": int(blas), "kind": "oracle",
            "sample": f"first {n_tok} tokens of the same {cfg.name} batch: full routing against all "
                      f"{cfg.n_routed} centroids, permutation, {len(need)} routed experts + {cfg.n_shared} shared "
                      f"FFN in fp64 (NumPy), combine, bias update; {dt:.1f} s wall",
            "host_cpus": len(os.sched_getaffinity(0))}


def calib_copy(mib, dev):
    """One plain device copy of mib MiB (the reference reading for the HBM byte counters)."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def cpu_baseline_backward(cfg, inp, d_out, n_tok):
    """The oracle's backward steps (route, per-expert FFN backward, gate and centroid gradients) on the first n_tok
    tokens of the same batch (host cores); the expert-weight gradients of the touched experts only."""
    import numpy as np
    import oracle

    u = inp["u"][:n_tok].cpu()
    cent, bias = inp["centroids"].cpu(), inp["bias"].cpu()
    r0 = oracle.route(u, cent, bias, cfg.n_groups, cfg.topk_groups, cfg.group_topn, cfg.topk)
    need = sorted(set(int(e) for e in r0["idx"].ravel()))
    wg = {e: inp["w_gate_up"][e].cpu() for e in need}
    wd = {e: inp["w_down"][e].cpu() for e in need}
    sg = [inp["s_gate_up"][s].cpu() for s in range(cfg.n_shared)]
    sd = [inp["s_down"][s].cpu() for s in range(cfg.n_shared)]
    fp8 = cfg.gemm == "fp8"
    if fp8:                                                  # weight blocks quantised before timing
        wq = {e: oracle.quantize_blocks(wg[e]) + oracle.quantize_blocks(wd[e]) for e in need}
        sq = [oracle.quantize_blocks(sg[s]) + oracle.quantize_blocks(sd[s]) for s in range(cfg.n_shared)]
    dO = d_out[:n_tok].cpu().double().numpy()
    t0 = time.perf_counter()
    r = oracle.route(u, cent, bias, cfg.n_groups, cfg.topk_groups, cfg.group_topn, cfg.topk)
    off, perm, _ = oracle.permute(r["idx"], cfg.n_routed)
    u64 = u.double().numpy()
    du = dO.copy()
    d_gate = np.zeros((n_tok, cfg.topk))
    for e in need:
        toks = perm[off[e]:off[e + 1]]
        slot = np.array([int(np.flatnonzero(r["idx"][t] == e)[0]) for t in toks])
        dy = r["gate"][toks, slot][:, None] * dO[toks]
        if fp8:
            d_gate[toks, slot] = (dO[toks] * oracle.ffn_fp8(u64[toks], *wq[e])).sum(axis=1)
            da = oracle.ffn_backward_fp8(u64[toks], *wq[e], oracle.round_bf16(dy))[0]
        else:
            d_gate[toks, slot] = (dO[toks] * oracle.swiglu_ffn(u64[toks], wg[e], wd[e])).sum(axis=1)
            da = oracle.ffn_backward(u64[toks], wg[e], wd[e], dy)[0]
        np.add.at(du, toks, da)
    for s in range(cfg.n_shared):
        du += (oracle.ffn_backward_fp8(u64, *sq[s], dO)[0] if fp8 else oracle.ffn_backward(u64, sg[s], sd[s], dO)[0])
    ds = oracle.gate_backward(r["s"], r["idx"], d_gate)
    s_sel = np.take_along_axis(r["s"], r["idx"], axis=1)
    dz = ds * s_sel * (1.0 - s_sel)
    c64 = cent.double().numpy()
    d_cent = np.zeros_like(c64)
    for k in range(cfg.topk):
        du += dz[:, k:k + 1] * c64[r["idx"][:, k]]
        np.add.at(d_cent, r["idx"][:, k], dz[:, k:k + 1] * u64)
    dt = time.perf_counter() - t0
    try:
        from threadpoolctl import threadpool_info
        blas = max((i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"), default=1)
    except Exception:  # pragma: no cover
        blas = 1
    return {"value": n_tok / dt, "unit": "tokens/s", "cores": int(blas), "kind": "oracle",
            "sample": f"first {n_tok} tokens of the same {cfg.name} batch: routing, the forward of the "
                      f"{len(need)} touched routed experts (for the gate gradients), their and the {cfg.n_shared} "
                      f"shared experts' FFN backward ({cfg.gemm} recipe), gate / centroid / input gradients in fp64 (NumPy); "
                      f"{dt:.1f} s wall", "host_cpus": len(os.sched_getaffinity(0))}


def main_backward(args, cfg):
    import numpy as np
    import torch
    from moe_inputs import generate, generate_output_grad
    from mixture_experts_layer_gate_amd import MoELayer

    dev = "cuda"
    torch.cuda.set_device(0)
    inp = generate(cfg, dev)
    d_out = generate_output_grad(cfg, dev)
    layer = MoELayer(cfg, inp, dev, train=True)
    u = inp["u"]
    stream = torch.cuda.current_stream()
    if args.calib_copy_mib > 0:
        calib_copy(args.calib_copy_mib, dev)
    parts = [lambda: layer.route(u), lambda: layer.permute(u), lambda: layer.ffn_gate_up_train(u),
             layer.ffn_down_train, lambda: layer.combine(u), lambda: layer.combine_backward(d_out),
             layer.ffn_backward, layer.route_backward, lambda: layer.input_grad(d_out), layer.bias_update]

    def step(ev=None):
        for j, f in enumerate(parts):
            if ev is not None:
                ev[j].record(stream)
            f()
        if ev is not None:
            ev[len(parts)].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(parts) + 1)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    per_call = {c: float(np.mean([events[i][j].elapsed_time(events[i][j + 1]) for i in range(args.steps)]))
                for j, c in enumerate(CALLS_TRAIN)}
    T, d, I, K, N, Ns = cfg.T, cfg.d, cfg.inter, cfg.topk, cfg.n_routed, cfg.n_shared
    rows = T * (K + Ns)
    # dominant call: the FFN backward, four GEMMs over every row (dh, da: Dgrad; dW_down, dW_gate_up: Wgrad).
    # fp8: the Dgrad GEMMs run on the fp8 MFMA, the Wgrad GEMMs on the bf16 MFMA (their re-tiled E4M3 operands
    # are exact in bf16), so the peak is the mix of the two rates over this FLOP split.
    dgrad_flops, wgrad_flops = 2.0 * rows * d * I * 3, 2.0 * rows * d * I * 3
    bwd_flops = dgrad_flops + wgrad_flops
    bwd_s = per_call["ffn_bwd"] / 1e3
    peak = bwd_flops / (dgrad_flops / MFMA_PEAK[cfg.gemm] + wgrad_flops / MFMA_PEAK["bf16"])
    roof = {"bound": "mfma", "achieved": bwd_flops / bwd_s / 1e12, "peak": peak / 1e12,
            "unit": "TFLOP/s", "frac": bwd_flops / bwd_s / peak, "traffic": None,
            "kernel": ("moe_ffn_backward_fp8" if cfg.gemm == "fp8" else "moe_ffn_backward")
                      + " (dh, SwiGLU backward, da, dW_down, dW_gate_up)"}
    fwd_flops = cfg.ffn_flops()
    calls = {c: {"ms": round(per_call[c], 4)} for c in CALLS_TRAIN}
    res = {
        "metric": METRIC_TRAIN, "value": T / (ms_step / 1e3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": cfg.gemm,
        "data": "synthetic: seeded N(0,1) tokens and output gradient, random-init N(0,0.02^2) weights",
        "config": {"workload": f"{cfg.name}: {cfg.description}, forward + backward", "T": T, "d": d,
                   "n_routed": N, "topk": K, "n_shared": Ns, "inter": I, "gemm": cfg.gemm},
        "roofline": roof,
        "train_step": {"TFLOP/s": (fwd_flops + bwd_flops) / (ms_step / 1e3) / 1e12,
                       "roofline_ms": ((fwd_flops + cfg.router_flops()) / MFMA_PEAK[cfg.gemm] + bwd_flops / peak) * 1e3},
        "calls": calls,
    }
    res["train_step"]["frac_of_roofline"] = res["train_step"]["roofline_ms"] / ms_step
    res["cpu_baseline"] = cpu_baseline_backward(cfg, inp, d_out, args.cpu_sample) if args.cpu_sample > 0 else None
    print(json.dumps(res))


FLUSH_BYTES = 1 << 30     # written before every timed step: four times the 256 MB Infinity Cache


def run_forward(args, cfg, dev, pow2_act_scales=False):
    """Time args.steps forward steps (+ bias update) of one workload; returns the measurements.

    Each timed step is bracketed by device synchronisations; before it (outside the timed region) a 1 GiB
    scratch buffer is written so no input of the step sits in the Infinity Cache, unless --no-flush. HIP
    events recorded on the launch stream time every call of every step. The algorithmic bytes of a step
    follow that step's own expert load (the bias update changes which experts a batch touches).
    """
    import numpy as np
    import torch
    from moe_inputs import generate
    from mixture_experts_layer_gate_amd import MoELayer

    inp = generate(cfg, dev)
    layer = MoELayer(cfg, inp, dev, pow2_act_scales=pow2_act_scales, keep_scores=False)
    u = inp["u"]
    stream = torch.cuda.current_stream()
    flush = None if args.no_flush else torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)

    def step(ev=None):
        rec = (lambda i: ev[i].record(stream)) if ev is not None else (lambda i: None)
        rec(0)
        layer.route(u)
        rec(1)
        layer.permute(u)
        rec(2)
        layer.ffn_all_phases(u, between=lambda: rec(3))
        rec(4)
        layer.combine(u)
        rec(5)
        layer.bias_update()
        rec(6)

    if args.calib_copy_mib > 0:
        calib_copy(args.calib_copy_mib, dev)
    # the load of every step run (warmup, timed, back to back), to price each launch a profiler sees
    all_loads = torch.empty((args.warmup + 2 * args.steps, cfg.n_routed), dtype=torch.int32, device=dev)
    for w in range(args.warmup):
        step()
        all_loads[w].copy_(layer.expert_load)
    torch.cuda.synchronize()
    n_calls = len(CALLS)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(n_calls + 1)] for _ in range(args.steps)]
    loads = torch.empty((args.steps, cfg.n_routed), dtype=torch.int32, device=dev)
    bias0, count0 = layer.bias.clone(), layer.step_count   # the graph replays below repeat the same steps
    wall = []
    for i in range(args.steps):
        if flush is not None:
            flush.fill_(float(i))
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        step(events[i])
        torch.cuda.synchronize()
        wall.append(time.perf_counter() - t0)
        loads[i].copy_(layer.expert_load)
        all_loads[args.warmup + i].copy_(layer.expert_load)
    torch.cuda.synchronize()
    # the same steps back to back with no flush and no synchronisation between them, for context
    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
        all_loads[args.warmup + args.steps + i].copy_(layer.expert_load)
    torch.cuda.synchronize()
    ms_b2b = (time.perf_counter() - t0) * 1e3 / args.steps
    ms_step = float(np.mean(wall)) * 1e3
    graph = None
    if getattr(args, "graph", False):
        # the same step recorded once and replayed: one submission per step instead of one per kernel
        g = layer.capture_step(u)
        g.replay()
        # back to the bias the timed eager steps started from: the replays run the same sequence of steps
        # (the decode batch's bias updates widen the set of touched experts from step to step)
        layer.bias.copy_(bias0)
        layer.step_count = count0
        torch.cuda.synchronize()
        gwall = []
        for i in range(args.steps):
            if flush is not None:
                flush.fill_(float(i))
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            g.replay()
            torch.cuda.synchronize()
            gwall.append(time.perf_counter() - t0)
        t0 = time.perf_counter()
        for i in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        graph = {"ms_per_step": float(np.mean(gwall)) * 1e3,
                 "ms_per_step_back_to_back": (time.perf_counter() - t0) * 1e3 / args.steps,
                 "eager_ms_per_step": ms_step, "eager_ms_per_step_back_to_back": ms_b2b,
                 "same_steps_as_eager": True}
        del g
    call_ms = np.array([[events[i][j].elapsed_time(events[i][j + 1]) for j in range(n_calls)]
                        for i in range(args.steps)])
    per_call = {c: float(call_ms[:, j].mean()) for j, c in enumerate(CALLS)}

    load = loads.cpu().numpy()
    touched = (load > 0).sum(axis=1)                    # experts with rows, per step
    T, d, I, K, N, Ns = cfg.T, cfg.d, cfg.inter, cfg.topk, cfg.n_routed, cfg.n_shared
    wb = WEIGHT_BYTES[cfg.gemm]                 # weight bytes per element (with scales)
    ab = 2                                      # u / out bytes per element (bf16)
    # dominant kernel: the gate/up projection of the routed and shared experts (one launch); its algorithmic
    # bytes are the gate/up weights of the experts that step touched (plus the shared ones) and u, read once
    gu_bytes = (touched + Ns) * 2 * I * d * wb + T * d * ab
    gu_flops = 2.0 * T * (K + Ns) * d * 2 * I
    gu_ms = call_ms[:, CALLS.index("ffn_gate_up")]
    gu_s_total = gu_ms.sum() / 1e3
    gu_bound = "hbm" if gu_bytes.mean() / HBM_PEAK >= gu_flops / MFMA_PEAK[cfg.gemm] else "mfma"
    if gu_bound == "hbm":
        roof = {"bound": "hbm", "achieved": gu_bytes.sum() / gu_s_total / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": gu_flops * args.steps / gu_s_total / 1e12,
                "peak": MFMA_PEAK[cfg.gemm] / 1e12, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = recorded_traffic(f"ffn_gate_up_{cfg.gemm} routed+shared", cfg.name, cfg.gemm)
    roof["kernel"] = "ffn_gate_up (routed + shared experts)"
    roof["algorithmic_bytes_per_launch"] = float(gu_bytes.mean())
    roof["launch_ms"] = float(gu_ms.mean())
    roof["mfma_frac"] = gu_flops * args.steps / gu_s_total / MFMA_PEAK[cfg.gemm]

    ffn_flops = cfg.ffn_flops()
    ffn_s = (per_call["ffn_gate_up"] + per_call["ffn_down"]) / 1e3
    layer_bytes = float(((touched + Ns) * 3 * I * d * wb).mean() + 2 * T * d * ab + N * d * ab)
    calls = {c: {"ms": round(per_call[c], 4)} for c in CALLS}
    route_bytes = T * d * ab + N * d * ab + T * K * 8 + N * 4           # u, centroids; idx, gates, load out
    combine_bytes = T * d * ab * 2 + (T * K + T * Ns) * d * ab + T * K * 8   # u, out, y rows; row_of, gates
    permute_bytes = T * K * 4 * 3 + (N + 1) * 4                        # idx in; perm_token, row_of, offsets out
    if cfg.gemm in ("fp8", "mxfp4"):
        permute_bytes += T * d * ab + T * d + T * d // 128 * 4          # u in; E4M3 codes and scales out
    for c, nb in (("route", route_bytes), ("permute", permute_bytes), ("combine", combine_bytes)):
        calls[c]["GB/s"] = round(nb / (per_call[c] / 1e3) / 1e9, 1)
        calls[c]["hbm_frac"] = round(nb / (per_call[c] / 1e3) / HBM_PEAK, 4)
    calls["ffn_gate_up"]["TFLOP/s"] = round(gu_flops / (per_call["ffn_gate_up"] / 1e3) / 1e12, 1)
    calls["ffn_gate_up"]["hbm_frac"] = round(float(gu_bytes.mean()) / (per_call["ffn_gate_up"] / 1e3) / HBM_PEAK, 4)
    dn_bytes = float(((touched + Ns) * I * d * wb).mean())
    calls["ffn_down"]["GB/s_weights"] = round(dn_bytes / (per_call["ffn_down"] / 1e3) / 1e9, 1)
    calls["ffn_down"]["hbm_frac_weights"] = round(dn_bytes / (per_call["ffn_down"] / 1e3) / HBM_PEAK, 4)
    calls["ffn_down"]["TFLOP/s"] = round(2.0 * T * (K + Ns) * I * d / (per_call["ffn_down"] / 1e3) / 1e12, 1)
    steps_ms = sorted(call_ms.sum(axis=1))
    pct = lambda q: float(steps_ms[min(len(steps_ms) - 1, int(q * (len(steps_ms) - 1) + 0.5))])
    res = {
        "ms_step": ms_step, "ms_b2b": ms_b2b, "roof": roof, "calls": calls,
        "ffn": {"TFLOP/s": ffn_flops / ffn_s / 1e12, "mfma_frac": ffn_flops / ffn_s / MFMA_PEAK[cfg.gemm],
                "hbm_frac_weights": float(((touched + Ns) * 3 * I * d * wb).mean()) / ffn_s / HBM_PEAK},
        "layer": {"algorithmic_GB": layer_bytes / 1e9, "roofline_ms": max(layer_bytes / HBM_PEAK,
                  (ffn_flops + cfg.router_flops()) / MFMA_PEAK[cfg.gemm]) * 1e3,
                  "experts_touched": int(touched[-1]), "experts_touched_range": [int(touched.min()), int(touched.max())],
                  "experts_touched_every_step": [int(x) for x in (all_loads.cpu().numpy() > 0).sum(axis=1)],
                  "max_load": int(load[-1].max()), "min_load": int(load[-1].min())},
        "step_ms_events": {"p10": pct(0.1), "p50": pct(0.5), "p90": pct(0.9)},
        "inp": inp, "layer_obj": layer, "graph": graph,
    }
    res["layer"]["frac_of_roofline"] = res["layer"]["roofline_ms"] / ms_step
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the layer runs on a single MI355X with no collectives; "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)
    both = args.config is None          # default: the V3-shaped layer in bf16, plus its fp8 form
    if both:
        args.config = "c3"
    if args.backward:
        from moe_inputs import get_config as _gc
        cfg = _gc(args.config)
        if args.graph:
            print("bench.py: --graph times forward steps; the training step runs eagerly", file=sys.stderr)
            sys.exit(2)
        if cfg.gemm not in ("bf16", "fp8") or args.mxfp4 or args.pow2_act_scales or args.batch_invariant:
            print("bench.py: --backward runs the bf16 (c2, c3) and fp8 (c4, c5) workloads", file=sys.stderr)
            sys.exit(2)
        main_backward(args, cfg)
        return

    import torch
    from moe_inputs import get_config

    over = dict(batch_invariant=int(args.batch_invariant))
    if args.mxfp4:
        if get_config(args.config).gemm != "fp8":
            print("bench.py: --mxfp4 applies to the fp8 workloads (c4, c5)", file=sys.stderr)
            sys.exit(2)
        over["gemm"] = "mxfp4"
    cfg = get_config(args.config, **over)
    dev = "cuda"
    torch.cuda.set_device(0)
    r = run_forward(args, cfg, dev, args.pow2_act_scales)
    T = cfg.T
    ms_main = r["graph"]["ms_per_step"] if r["graph"] else r["ms_step"]
    res = {
        "metric": METRIC,
        "value": T / (ms_main / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_main,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.gemm,
        "data": "synthetic: seeded N(0,1) tokens, random-init N(0,0.02^2) weights of the workload's shape",
        "config": {"workload": f"{cfg.name}: {cfg.description}" + (", MXFP4 expert weights" if cfg.gemm == "mxfp4"
                                                                     else ""), "T": T, "d": cfg.d,
                   "n_routed": cfg.n_routed, "groups": cfg.n_groups, "topk_groups": cfg.topk_groups,
                   "topk": cfg.topk, "n_shared": cfg.n_shared, "inter": cfg.inter, "gemm": cfg.gemm,
                   "batch_invariant": bool(args.batch_invariant),
                   "infinity_cache_flush": not args.no_flush, "hip_graph": bool(args.graph),
                   **({"act_scales": "pow2" if args.pow2_act_scales else "fp32"} if cfg.gemm == "fp8" else {})},
        "roofline": r["roof"],
        "ffn": r["ffn"],
        "layer": r["layer"],
        "calls": r["calls"],
        "step_ms_events": r["step_ms_events"],
        "ms_per_step_back_to_back": r["graph"]["ms_per_step_back_to_back"] if r["graph"] else r["ms_b2b"],
    }
    if r["graph"]:
        res["graph"] = r["graph"]
    cpu = cpu_baseline(cfg, r["inp"], r["layer_obj"], args.cpu_sample) if args.cpu_sample > 0 else None
    del r
    torch.cuda.empty_cache()
    if both:
        # the fp8 half of the metric: the same V3 shape with E4M3 expert GEMMs
        cfg8 = get_config("c4", **over)
        r8 = run_forward(args, cfg8, dev)
        ms8 = r8["graph"]["ms_per_step"] if r8["graph"] else r8["ms_step"]
        b2b8 = r8["graph"]["ms_per_step_back_to_back"] if r8["graph"] else r8["ms_b2b"]
        res["fp8"] = {"workload": f"{cfg8.name}: {cfg8.description}", "value": cfg8.T / (ms8 / 1e3),
                      "unit": "tokens/s", "ms_per_step": ms8, "ms_per_step_back_to_back": b2b8,
                      "roofline": r8["roof"], "ffn": r8["ffn"], "layer": r8["layer"], "calls": r8["calls"],
                      "step_ms_events": r8["step_ms_events"], **({"graph": r8["graph"]} if r8["graph"] else {})}
        del r8
        torch.cuda.empty_cache()
    peaks = measure_peaks(dev)
    res["peaks_measured"] = peaks
    for roof, gemm in [(res["roofline"], cfg.gemm)] + ([(res["fp8"]["roofline"], "fp8")] if both else []):
        roof["peak_measured"] = (peaks["hbm_read_GB/s"] if roof["bound"] == "hbm"
                                 else peaks["mfma_fp8_TFLOP/s" if gemm in ("fp8", "mxfp4") else "mfma_bf16_TFLOP/s"])
        roof["frac_of_measured"] = roof["achieved"] / roof["peak_measured"]
    res["cpu_baseline"] = cpu
    print(json.dumps(res))


if __name__ == "__main__":
    main()
