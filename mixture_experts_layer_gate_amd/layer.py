"""A DeepSeekMoE layer forward composed from the five libmoe calls.

``MoELayer`` holds the expert weights, centroids and the bias on the GPU and
runs, on one stream with no host synchronisation:

  moe_route -> moe_permute -> moe_grouped_ffn -> moe_combine, then
  moe_bias_update at the end of a step.

The grouped FFN covers the routed and the shared experts in one call: the
weights sit routed-then-shared in one array, shared expert s is expert
N_r + s with segment [T*K + s*T, T*K + (s+1)*T) and rows gathered through
the identity, so its tiles fill the routed experts' tail in the same
persistent launch. (With permuted copies instead of the fused gather the
two run as separate calls.)

Torch only allocates device memory and provides the stream; every step runs
in libmoe.so.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Optional

import torch

from . import binding as B
from .state import load_bias_state, save_bias_state


@dataclass
class LayerOutputs:
    topk_idx: torch.Tensor
    topk_gate: torch.Tensor
    expert_load: torch.Tensor
    expert_offsets: torch.Tensor
    perm_token: torch.Tensor
    row_of: torch.Tensor
    y_routed: torch.Tensor
    y_shared: Optional[torch.Tensor]
    out: torch.Tensor
    scores: Optional[torch.Tensor] = None
    a_q: Optional[torch.Tensor] = None
    a_scale: Optional[torch.Tensor] = None


class StepGraph:
    """A recorded MoELayer.step (see MoELayer.capture_step): replay() runs one step on the current stream."""

    def __init__(self, layer: "MoELayer", graph: "torch.cuda.CUDAGraph"):
        self.layer, self.graph = layer, graph

    def replay(self) -> torch.Tensor:
        self.graph.replay()
        self.layer.step_count += 1
        return self.layer.out


class MoELayer:
    """One MoE layer on the current CUDA device.

    cfg: an object with T, d, n_routed, n_groups, topk_groups, group_topn,
    topk, n_shared, inter, gemm ("f32" | "bf16" | "fp8" | "mxfp4"), gamma.
    weights: w_gate_up [N_r,2I,d], w_down [N_r,d,I], s_gate_up [N_s,2I,d],
    s_down [N_s,d,I] (fp32 or bf16), centroids [N_r,d], bias [N_r] fp32.
    For fp8 the bf16 weights are block-quantised on the device by
    moe_quantize_weights and the bf16 copies are dropped unless keep_bf16.

    train=True (bf16 weights only) also keeps the weights transposed for the
    input-gradient GEMMs and caches the SwiGLU inputs in forward_train, so that
    backward(d_out) returns du and leaves the centroid and expert-weight
    gradients in self.grads.

    keep_scores=False skips writing the affinities s [T, N_r] in route (they
    are only needed by balance_stats and the backward); the selection, gates
    and loads are the same.
    """

    def __init__(self, cfg, weights: Dict[str, torch.Tensor], device="cuda", keep_bf16: bool = False,
                 gather_in_gemm: bool = True, pow2_act_scales: bool = False, tiled_bf16: bool = True,
                 train: bool = False, keep_scores: bool = True):
        self.cfg = cfg
        if train and cfg.gemm not in ("bf16", "fp8"):
            raise ValueError("MoELayer(train=True) needs bf16 or fp8 expert GEMMs")
        self.train = train
        self.keep_scores = keep_scores or train
        self.shape = B.moe_shape.of(cfg)
        self.dev = torch.device(device)
        self.gemm = {"f32": B.MOE_F32, "bf16": B.MOE_BF16, "fp8": B.MOE_F8E4M3, "mxfp4": B.MOE_F4E2M1}[cfg.gemm]
        # E4M3 activations and H (fp8 and MXFP4 weights)
        self.q8 = self.gemm in (B.MOE_F8E4M3, B.MOE_F4E2M1)
        # bf16 weights copied once into the tiled layout (contiguous 16 KB stage blocks)
        if self.gemm == B.MOE_BF16 and tiled_bf16:
            self.gemm = B.MOE_BF16_TILED
        self.gather_in_gemm = gather_in_gemm
        # fp8: the up-projection input quantised with power-of-two tile scales
        self.a_qdtype = B.MOE_F8E4M3_POW2 if pow2_act_scales else B.MOE_F8E4M3
        to = lambda t: t.to(self.dev).contiguous()
        self.centroids = to(weights["centroids"])
        self.bias = weights["bias"].to(self.dev, torch.float32).clone()  # layer-owned state
        self.step_count = 0                                               # bias updates applied so far
        self.act_dtype = self.centroids.dtype
        N, Ns = cfg.n_routed, cfg.n_shared
        self.w = {}
        for kind in ("gate_up", "down"):
            # routed experts, then shared ones, in one array; the per-kind views alias it
            both = torch.cat([to(weights["w_" + kind]), to(weights["s_" + kind])]) if Ns else to(weights["w_" + kind])
            if self.q8:
                n, r, c = both.shape
                if self.gemm == B.MOE_F8E4M3:
                    codes = torch.empty((n, B.mx_rows(r), c), dtype=torch.uint8, device=self.dev)   # tiled
                    scale = torch.empty((n, r // 128, c // 128), dtype=torch.float32, device=self.dev)
                    B.moe_quantize_weights(both, codes, scale, gate_up=(kind == "gate_up"))
                    if train:                       # W^T in 128x128 blocks for the FP8 input-gradient GEMMs
                        wt = torch.empty((n, c, r), dtype=both.dtype, device=self.dev)
                        B.moe_transpose_bf16(both, wt)
                        ct = torch.empty((n, B.mx_rows(c), r), dtype=torch.uint8, device=self.dev)
                        st = torch.empty((n, c // 128, r // 128), dtype=torch.float32, device=self.dev)
                        B.moe_quantize_weights(wt, ct, st, gate_up=False)
                        del wt
                        self.w["all_" + kind + "_t"], self.w["all_" + kind + "_t_scale"] = ct, st
                else:
                    rt = B.mx_rows(r)               # tiled MXFP4: whole 256-row tiles
                    codes = torch.empty((n, rt, c // 2), dtype=torch.uint8, device=self.dev)
                    scale = torch.empty((n, rt, c // 32), dtype=torch.uint8, device=self.dev)
                    B.moe_quantize_weights_mxfp4(both, codes, scale, gate_up=(kind == "gate_up"))
                if keep_bf16:
                    self.w["w_" + kind + "_bf16"], self.w["s_" + kind + "_bf16"] = both[:N], both[N:]
                del both
                self.w["all_" + kind], self.w["all_" + kind + "_scale"] = codes, scale
                self.w["w_" + kind + "_scale"], self.w["s_" + kind + "_scale"] = scale[:N], scale[N:]
                both = codes
            elif self.gemm == B.MOE_BF16_TILED:
                n, r, c = both.shape
                tiled = torch.empty((n, B.mx_rows(r), c), dtype=both.dtype, device=self.dev)
                B.moe_tile_weights_bf16(both, tiled, gate_up=(kind == "gate_up"))
                if train:
                    wt = torch.empty((n, B.mx_rows(c), r), dtype=both.dtype, device=self.dev)
                    B.moe_transpose_weights_bf16(both, wt)
                    self.w["all_" + kind + "_t"] = wt
                del both
                both = tiled
            self.w["all_" + kind] = both
            self.w["w_" + kind], self.w["s_" + kind] = both[:N], both[N:]
        self.ws = torch.empty(max(B.moe_workspace_bytes(self.shape, self.gemm), 256), dtype=torch.uint8,
                              device=self.dev)
        if train and self.gemm not in (B.MOE_BF16_TILED, B.MOE_F8E4M3):
            raise ValueError("MoELayer(train=True) needs the tiled bf16 weights (tiled_bf16=True) or fp8")
        self._alloc()
        if train:
            self._alloc_train()

    def _alloc_train(self):
        c, dev = self.cfg, self.dev
        T, K, N, Ns, d, I = c.T, c.topk, c.n_routed, c.n_shared, c.d, c.inter
        n_rows = T * (K + Ns)
        bf = torch.bfloat16
        if self.q8:                                  # E4M3 H and [G, U] cache with their 1x128 scales
            self.h_all = torch.empty((n_rows, I), dtype=torch.uint8, device=dev)
            self.h_all_scale = torch.empty((n_rows, I // 128), dtype=torch.float32, device=dev)
            self.gu_cache = torch.empty((n_rows, 2 * I), dtype=torch.uint8, device=dev)
            self.gu_scale = torch.empty((n_rows, 2 * I // 128), dtype=torch.float32, device=dev)
        else:
            self.h_all = torch.empty((n_rows, I), dtype=bf, device=dev)
            self.h_all_scale = None
            self.gu_cache = torch.empty((n_rows, 2 * I), dtype=bf, device=dev)
        self.dy_all = torch.empty((n_rows, d), dtype=bf, device=dev)
        self.da_all = torch.empty((n_rows, d), dtype=bf, device=dev)
        self.d_gate = torch.empty((T, K), dtype=torch.float32, device=dev)
        self.du_router = torch.empty((T, d), dtype=torch.float32, device=dev)
        self.du = torch.empty((T, d), dtype=torch.float32, device=dev)
        dwg = torch.empty((N + Ns, 2 * I, d), dtype=torch.float32, device=dev)
        dwd = torch.empty((N + Ns, d, I), dtype=torch.float32, device=dev)
        self.grads = {"centroids": torch.empty((N, d), dtype=torch.float32, device=dev),
                      "all_gate_up": dwg, "all_down": dwd, "w_gate_up": dwg[:N], "w_down": dwd[:N],
                      "s_gate_up": dwg[N:], "s_down": dwd[N:]}
        wsb = (B.moe_ffn_backward_fp8_workspace_bytes(self.shape, n_rows, N + Ns) if self.q8
               else B.moe_ffn_backward_workspace_bytes(self.shape, n_rows))
        self.ws_bwd = torch.empty(max(wsb, T * K * 4, 256), dtype=torch.uint8, device=dev)

    def _alloc(self):
        c, dev = self.cfg, self.dev
        T, K, N, d = c.T, c.topk, c.n_routed, c.d
        ydt = torch.float32 if c.gemm == "f32" else torch.bfloat16
        self.topk_idx = torch.empty((T, K), dtype=torch.int32, device=dev)
        self.topk_gate = torch.empty((T, K), dtype=torch.float32, device=dev)
        self.expert_load = torch.empty((N,), dtype=torch.int32, device=dev)
        self.scores = torch.empty((T, N), dtype=torch.float32, device=dev)
        Ns = c.n_shared
        # routed entries first (written by moe_permute), then the shared experts' fixed ones
        self.offsets_all = torch.empty((N + Ns + 1,), dtype=torch.int32, device=dev)
        self.offsets_all[N + 1:] = T * K + T * torch.arange(1, Ns + 1, dtype=torch.int32, device=dev)
        self.expert_offsets = self.offsets_all[:N + 1]
        self.rows_all = torch.empty((T * K + Ns * T,), dtype=torch.int32, device=dev)
        self.rows_all[T * K:] = torch.arange(T, dtype=torch.int32, device=dev).repeat(Ns)
        self.perm_token = self.rows_all[:T * K]
        self.row_of = torch.empty((T * K,), dtype=torch.int32, device=dev)
        self.shared_offsets = (torch.arange(Ns + 1, dtype=torch.int32, device=dev) * T).contiguous()
        self.y_all = torch.empty((T * K + max(Ns, 1) * T, d), dtype=ydt, device=dev)
        self.y_routed = self.y_all[:T * K]
        self.y_shared = self.y_all[T * K:]
        self.out = torch.empty((T, d), dtype=self.act_dtype, device=dev)
        if self.q8:
            # u quantised once per token (1x128 tiles); the GEMMs gather its rows
            self.u_q = torch.empty((T, d), dtype=torch.uint8, device=dev)
            self.u_scale = torch.empty((T, d // 128), dtype=torch.float32, device=dev)
        elif not self.gather_in_gemm:
            self.a_perm = torch.empty((T * K, d), dtype=self.act_dtype, device=dev)

    # ---------------------------------------------------------------- steps
    def route(self, u):
        B.moe_route(self.shape, u, self.centroids, self.bias, self.topk_idx, self.topk_gate, self.expert_load,
                    self.scores if self.keep_scores else None, self.ws)

    def balance_stats(self, seq_len: int, alpha: float = 1e-4):
        """Eq. (17)-(20) on the last route's scores and selection: (f, P, loss) per run of seq_len tokens."""
        c = self.cfg
        n_seq = -(-c.T // seq_len)
        f = torch.empty((n_seq, c.n_routed), dtype=torch.float32, device=self.dev)
        P = torch.empty((n_seq, c.n_routed), dtype=torch.float32, device=self.dev)
        loss = torch.empty((n_seq,), dtype=torch.float32, device=self.dev)
        B.moe_balance_stats(self.shape, self.scores, self.topk_idx, seq_len, alpha, f, P, loss, self.ws)
        return f, P, loss

    def permute(self, u):
        if self.q8:
            B.moe_permute(self.shape, self.topk_idx, u, self.expert_offsets, self.perm_token, self.row_of,
                          self.u_q, self.a_qdtype, self.u_scale, 0, self.ws)
        elif self.gather_in_gemm:
            B.moe_permute(self.shape, self.topk_idx, u, self.expert_offsets, self.perm_token, self.row_of,
                          None, None, None, 1, self.ws)
        else:
            B.moe_permute(self.shape, self.topk_idx, u, self.expert_offsets, self.perm_token, self.row_of,
                          self.a_perm, None, None, 1, self.ws)

    def _a(self, u):
        """Token operand of the gathered FFN: u (or its fp8 codes and scales)."""
        if self.q8:
            return self.u_q, self.u_scale
        return u, None

    @property
    def fused(self) -> bool:
        """Routed and shared experts in one grouped call (needs the gather-in-GEMM path)."""
        return self.q8 or self.gather_in_gemm

    def ffn_all(self, u):
        """Routed and shared experts in one moe_grouped_ffn call."""
        c = self.cfg
        a, a_scale = self._a(u)
        n_rows = c.T * (c.topk + c.n_shared)
        B.moe_grouped_ffn(self.shape, self.gemm, c.n_routed + c.n_shared, n_rows, self.offsets_all,
                          B.MOE_ROWS_GATHER, self.rows_all, a, a_scale, c.T, self.w["all_gate_up"],
                          self.w.get("all_gate_up_scale"), self.w["all_down"], self.w.get("all_down_scale"),
                          self.y_all, self.ws)

    def ffn_all_phases(self, u, between=None):
        """ffn_all as its two calls (moe_ffn_gate_up, moe_ffn_down); ``between`` runs in between."""
        c = self.cfg
        n_rows = c.T * (c.topk + c.n_shared)
        if getattr(self, "h_all", None) is None:
            hdt = {B.MOE_F32: torch.float32, B.MOE_BF16: torch.bfloat16, B.MOE_F8E4M3: torch.uint8,
                   B.MOE_F4E2M1: torch.uint8, B.MOE_BF16_TILED: torch.bfloat16}[self.gemm]
            self.h_all = torch.empty((n_rows, c.inter), dtype=hdt, device=self.dev)
            self.h_all_scale = (torch.empty((n_rows, c.inter // 128), dtype=torch.float32, device=self.dev)
                                if self.q8 else None)
        a, a_scale = self._a(u)
        E = c.n_routed + c.n_shared
        B.moe_ffn_gate_up(self.shape, self.gemm, E, n_rows, self.offsets_all, B.MOE_ROWS_GATHER, self.rows_all,
                          a, a_scale, c.T, self.w["all_gate_up"], self.w.get("all_gate_up_scale"), self.h_all,
                          self.h_all_scale, self.ws)
        if between is not None:
            between()
        B.moe_ffn_down(self.shape, self.gemm, E, n_rows, self.offsets_all, self.h_all, self.h_all_scale,
                       self.w["all_down"], self.w.get("all_down_scale"), self.y_all, self.ws)

    def ffn_routed(self, u):
        c = self.cfg
        n_rows = c.T * c.topk
        a_scale = None
        if self.q8:
            a, a_scale, a_rows, mode = self.u_q, self.u_scale, c.T, B.MOE_ROWS_GATHER
        elif self.gather_in_gemm:
            a, a_rows, mode = u, c.T, B.MOE_ROWS_GATHER
        else:
            a, a_rows, mode = self.a_perm, n_rows, B.MOE_ROWS_DIRECT
        B.moe_grouped_ffn(self.shape, self.gemm, c.n_routed, n_rows, self.expert_offsets, mode,
                          self.perm_token if mode == B.MOE_ROWS_GATHER else None, a, a_scale, a_rows,
                          self.w["w_gate_up"], self.w.get("w_gate_up_scale"), self.w["w_down"],
                          self.w.get("w_down_scale"), self.y_routed, self.ws)

    def ffn_routed_phases(self, u, between=None):
        """The routed FFN as its two calls (moe_ffn_gate_up, moe_ffn_down); ``between`` runs in between."""
        c = self.cfg
        n_rows = c.T * c.topk
        if not hasattr(self, "h"):
            hdt = {B.MOE_F32: torch.float32, B.MOE_BF16: torch.bfloat16, B.MOE_F8E4M3: torch.uint8,
                   B.MOE_F4E2M1: torch.uint8, B.MOE_BF16_TILED: torch.bfloat16}[self.gemm]
            self.h = torch.empty((n_rows, c.inter), dtype=hdt, device=self.dev)
            self.h_scale = (torch.empty((n_rows, c.inter // 128), dtype=torch.float32, device=self.dev)
                            if self.q8 else None)
        a_scale = None
        if self.q8:
            a, a_scale, a_rows, mode = self.u_q, self.u_scale, c.T, B.MOE_ROWS_GATHER
        elif self.gather_in_gemm:
            a, a_rows, mode = u, c.T, B.MOE_ROWS_GATHER
        else:
            a, a_rows, mode = self.a_perm, n_rows, B.MOE_ROWS_DIRECT
        B.moe_ffn_gate_up(self.shape, self.gemm, c.n_routed, n_rows, self.expert_offsets, mode,
                          self.perm_token if mode == B.MOE_ROWS_GATHER else None, a, a_scale, a_rows,
                          self.w["w_gate_up"], self.w.get("w_gate_up_scale"), self.h, self.h_scale, self.ws)
        if between is not None:
            between()
        B.moe_ffn_down(self.shape, self.gemm, c.n_routed, n_rows, self.expert_offsets, self.h, self.h_scale,
                       self.w["w_down"], self.w.get("w_down_scale"), self.y_routed, self.ws)

    def ffn_shared(self, u):
        c = self.cfg
        if not c.n_shared:
            return
        if self.q8:
            a, a_scale = self.u_q, self.u_scale
        else:
            a, a_scale = u, None
        B.moe_grouped_ffn(self.shape, self.gemm, c.n_shared, c.n_shared * c.T, self.shared_offsets,
                          B.MOE_ROWS_SEGMENT, None, a, a_scale, c.T, self.w["s_gate_up"],
                          self.w.get("s_gate_up_scale"), self.w["s_down"], self.w.get("s_down_scale"),
                          self.y_shared, self.ws)

    def combine(self, u):
        B.moe_combine(self.shape, u, self.y_routed, self.row_of, self.topk_gate,
                      self.y_shared if self.cfg.n_shared else None, self.out)

    def bias_update(self):
        B.moe_bias_update(self.shape, self.expert_load, self.cfg.gamma, self.bias)
        self.step_count += 1

    def save_state(self, path: str) -> None:
        """Write the layer's persistent state (the expert bias and the step counter) to path; it waits for
        the work queued on the current stream, so the bias is the one after the last queued update."""
        save_bias_state(path, self.bias.cpu().numpy(), self.step_count)

    def load_state(self, path: str) -> None:
        """Restore the expert bias and the step counter written by save_state (bit-exact)."""
        b, step = load_bias_state(path, self.cfg.n_routed)
        self.bias.copy_(torch.from_numpy(b).to(self.dev))
        self.step_count = step

    def forward(self, u: torch.Tensor) -> torch.Tensor:
        """Layer output for tokens u [T, d] (no bias update)."""
        u = u.contiguous()
        self.route(u)
        self.permute(u)
        if self.fused:
            self.ffn_all(u)
        else:
            self.ffn_routed(u)
            self.ffn_shared(u)
        self.combine(u)
        self._ran = True
        return self.out

    def step(self, u: torch.Tensor) -> torch.Tensor:
        """forward + the step-end bias update."""
        out = self.forward(u)
        self.bias_update()
        return out

    def capture_step(self, u: torch.Tensor) -> "StepGraph":
        """Record step(u) once into a HIP graph, for replay without per-call host launches.

        Every buffer of the layer is allocated up front and no call allocates, copies to the host or
        synchronises, so the recorded launches replay unchanged: each replay routes the tokens then in
        u (same address, same shape) with the bias then current and updates the bias. The kernels are
        recorded, not run; the library sets its kernels' LDS limits on first use, so at least one eager
        step (or forward) must come before the capture.
        """
        if B._SYNC_DEBUG:
            raise RuntimeError("capture_step: MOE_SYNC_DEBUG=1 synchronises inside calls, which a capture forbids")
        if not getattr(self, "_ran", False):
            raise RuntimeError("capture_step: run one eager step (or forward) first")
        u = u.contiguous()
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream(device=self.dev)          # capture needs a stream other than the default one
        side.wait_stream(torch.cuda.current_stream(self.dev))
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                self.forward(u)
                B.moe_bias_update(self.shape, self.expert_load, self.cfg.gamma, self.bias)
        torch.cuda.current_stream(self.dev).wait_stream(side)
        return StepGraph(self, graph)

    # ---------------------------------------------------------------- training
    def forward_train(self, u: torch.Tensor) -> torch.Tensor:
        """forward() that also caches the SwiGLU inputs of every row for backward() (train=True)."""
        if not self.train:
            raise RuntimeError("forward_train needs MoELayer(train=True)")
        u = u.contiguous()
        self.route(u)
        self.permute(u)
        self.ffn_gate_up_train(u)
        self.ffn_down_train()
        self.combine(u)
        return self.out

    def ffn_gate_up_train(self, u):
        """Gate/up projection of every row that also writes the SwiGLU inputs [G | U] (routed + shared)."""
        c = self.cfg
        self.u_saved = u
        E, n_rows = c.n_routed + c.n_shared, c.T * (c.topk + c.n_shared)
        if self.q8:
            B.moe_ffn_gate_up_cache_fp8(self.shape, E, n_rows, self.offsets_all, B.MOE_ROWS_GATHER, self.rows_all,
                                        self.u_q, self.u_scale, c.T, self.w["all_gate_up"],
                                        self.w["all_gate_up_scale"], self.h_all, self.h_all_scale, self.gu_cache,
                                        self.gu_scale, self.ws)
            return
        B.moe_ffn_gate_up_cache(self.shape, self.gemm, E, n_rows, self.offsets_all, B.MOE_ROWS_GATHER, self.rows_all,
                                u, c.T, self.w["all_gate_up"], self.h_all, self.gu_cache, self.ws)

    def ffn_down_train(self):
        c = self.cfg
        E, n_rows = c.n_routed + c.n_shared, c.T * (c.topk + c.n_shared)
        B.moe_ffn_down(self.shape, self.gemm, E, n_rows, self.offsets_all, self.h_all,
                       self.h_all_scale if self.q8 else None, self.w["all_down"], self.w.get("all_down_scale"),
                       self.y_all, self.ws)

    def combine_backward(self, d_out):
        B.moe_combine_backward(self.shape, d_out, self.y_routed, self.row_of, self.topk_gate, self.dy_all, self.d_gate)

    def ffn_backward(self):
        c = self.cfg
        E, n_rows = c.n_routed + c.n_shared, c.T * (c.topk + c.n_shared)
        if self.q8:
            B.moe_ffn_backward_fp8(self.shape, E, n_rows, self.offsets_all, B.MOE_ROWS_GATHER, self.rows_all,
                                   self.u_q, self.u_scale, c.T, self.gu_cache, self.gu_scale,
                                   self.w["all_gate_up_t"], self.w["all_gate_up_t_scale"], self.w["all_down_t"],
                                   self.w["all_down_t_scale"], self.dy_all, self.da_all, self.grads["all_gate_up"],
                                   self.grads["all_down"], self.ws_bwd)
            return
        B.moe_ffn_backward(self.shape, E, n_rows, self.offsets_all, B.MOE_ROWS_GATHER, self.rows_all, self.u_saved,
                           c.T, self.gu_cache, self.w["all_gate_up_t"], self.w["all_down_t"], self.dy_all,
                           self.da_all, self.grads["all_gate_up"], self.grads["all_down"], self.ws_bwd)

    def route_backward(self):
        B.moe_route_backward(self.shape, self.u_saved, self.centroids, self.scores, self.topk_idx, self.d_gate,
                             self.expert_offsets, self.perm_token, self.row_of, self.du_router,
                             self.grads["centroids"], self.ws_bwd)

    def input_grad(self, d_out):
        B.moe_input_grad(self.shape, d_out, self.du_router, self.da_all, self.row_of, self.du)

    def backward(self, d_out: torch.Tensor) -> torch.Tensor:
        """Gradients of the last forward_train for the output gradient d_out [T, d]: returns du [T, d] fp32 and
        fills self.grads (centroids, expert gate/up and down weights, fp32)."""
        d_out = d_out.contiguous()
        self.combine_backward(d_out)
        self.ffn_backward()
        self.route_backward()
        self.input_grad(d_out)
        return self.du

    def outputs(self) -> LayerOutputs:
        return LayerOutputs(self.topk_idx, self.topk_gate, self.expert_load, self.expert_offsets, self.perm_token,
                            self.row_of, self.y_routed, self.y_shared if self.cfg.n_shared else None, self.out,
                            self.scores, getattr(self, "u_q", None), getattr(self, "u_scale", None))
