"""ctypes binding of libmoe.so (include/moe.h), same names as the C ABI.

Argument marshalling only: torch tensors are passed as device pointers, the
stream is torch's current stream, and tensor sizes are checked against the
shape before the call (the C side cannot see sizes). Every step runs in the
HIP library; if it is not built this module raises at import of the library.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

MOE_OK, MOE_E_INVALID, MOE_E_UNSUPPORTED, MOE_E_WORKSPACE, MOE_E_HIP = range(5)
MOE_F32, MOE_BF16, MOE_F8E4M3, MOE_F8E4M3_POW2, MOE_F4E2M1, MOE_BF16_TILED = 0, 1, 2, 3, 4, 5
MOE_ROWS_DIRECT, MOE_ROWS_GATHER, MOE_ROWS_SEGMENT = 0, 1, 2

_STATUS = {1: "MOE_E_INVALID", 2: "MOE_E_UNSUPPORTED", 3: "MOE_E_WORKSPACE", 4: "MOE_E_HIP"}


class MoEError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


class moe_shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("T", "d", "n_routed", "n_groups", "topk_groups", "group_topn", "topk", "n_shared", "inter",
                 "batch_invariant")]

    @classmethod
    def of(cls, cfg) -> "moe_shape":
        return cls(cfg.T, cfg.d, cfg.n_routed, cfg.n_groups, cfg.topk_groups, cfg.group_topn, cfg.topk,
                   cfg.n_shared, cfg.inter, int(getattr(cfg, "batch_invariant", 0)))


_lib = None
_lock = threading.Lock()
_P = ctypes.c_void_p
_I = ctypes.c_int32
_S = ctypes.POINTER(moe_shape)

_SIGS = {
    "moe_route": [_S, _I, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "moe_permute": [_S, _I, _P, _P, _P, _P, _P, _P, _I, _P, _I, _P, ctypes.c_size_t, _P],
    "moe_permute_noalloc": [_S, _I, _P, _P, _P, _P, _P, _P, _I, _P, _I, _P],
    "moe_permute_noalloc_max_scratch": [],
    "moe_grouped_ffn": [_S, _I, _I, _I, _P, _I, _P, _P, _P, _I, _P, _P, _P, _P, _I, _P, _P, ctypes.c_size_t, _P],
    "moe_ffn_gate_up": [_S, _I, _I, _I, _P, _I, _P, _P, _P, _I, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "moe_ffn_down": [_S, _I, _I, _I, _P, _P, _P, _P, _P, _I, _P, _P, ctypes.c_size_t, _P],
    "moe_combine": [_S, _I, _P, _P, _P, _P, _P, _P, _P],
    "moe_balance_stats": [_S, _P, _P, _I, ctypes.c_float, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "moe_bias_update": [_S, _P, ctypes.c_float, _P, _P],
    "moe_quantize_weights": [_I, _I, _I, _I, _P, _P, _P, _P],
    "moe_quantize_weights_mxfp4": [_I, _I, _I, _I, _P, _P, _P, _P],
    "moe_tile_weights_bf16": [_I, _I, _I, _I, _P, _P, _P],
    "moe_ffn_gate_up_cache": [_S, _I, _I, _I, _P, _I, _P, _P, _I, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "moe_combine_backward": [_S, _I, _P, _P, _P, _P, _I, _P, _P, _P],
    "moe_route_backward": [_S, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "moe_transpose_weights_bf16": [_I, _I, _I, _P, _P, _P],
    "moe_ffn_backward_workspace_bytes": [_S, _I],
    "moe_ffn_backward": [_S, _I, _I, _I, _P, _I, _P, _P, _I, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "moe_input_grad": [_S, _P, _P, _P, _P, _P, _P],
    "moe_transpose_bf16": [_I, _I, _I, _P, _P, _P],
    "moe_ffn_gate_up_cache_fp8": [_S, _I, _I, _P, _I, _P, _P, _P, _I, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "moe_ffn_backward_fp8_workspace_bytes": [_S, _I, _I],
    "moe_ffn_backward_fp8": [_S, _I, _I, _P, _I, _P, _P, _P, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                             ctypes.c_size_t, _P],
    "moe_workspace_bytes": [_S, _I],
    "moe_last_error": [],
    "moe_version": [],
}


def lib() -> ctypes.CDLL:
    """Load libmoe.so (once). Raises if the library has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise ImportError(f"{LIB_PATH} is not built; run `python -m mixture_experts_layer_gate_amd.build`")
            L = ctypes.CDLL(LIB_PATH)
            for name, args in _SIGS.items():
                f = getattr(L, name)
                f.argtypes = args
                f.restype = ctypes.c_size_t if name.endswith(("_bytes", "_max_scratch")) else ctypes.c_int
            L.moe_workspace_bytes.restype = ctypes.c_size_t
            L.moe_last_error.restype = ctypes.c_char_p
            L.moe_version.restype = ctypes.c_char_p
            _lib = L
    return _lib


# MOE_SYNC_DEBUG=1: wait for the device after every call, so an asynchronous kernel error surfaces at the
# call that caused it
_SYNC_DEBUG = os.environ.get("MOE_SYNC_DEBUG") == "1"


def _check(status: int):
    if status != MOE_OK:
        raise MoEError(status, lib().moe_last_error().decode())
    if _SYNC_DEBUG:
        torch.cuda.synchronize()


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libmoe must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype in (torch.float8_e4m3fn, torch.uint8):
        return MOE_F8E4M3
    raise TypeError(f"unsupported dtype {t.dtype}")


def _need(t: Optional[torch.Tensor], numel: int, name: str):
    if t is not None and t.numel() < numel:
        raise ValueError(f"{name} has {t.numel()} elements, needs {numel}")


def _nbytes(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def moe_workspace_bytes(shape: moe_shape, gemm: int) -> int:
    return int(lib().moe_workspace_bytes(ctypes.byref(shape), gemm))


def moe_route(shape: moe_shape, u, centroids, bias, topk_idx, topk_gate, expert_load, scores=None,
              workspace=None, stream=None):
    T, d, N, K = shape.T, shape.d, shape.n_routed, shape.topk
    _need(u, T * d, "u"); _need(centroids, N * d, "centroids"); _need(bias, N, "bias")
    _need(topk_idx, T * K, "topk_idx"); _need(topk_gate, T * K, "topk_gate"); _need(expert_load, N, "expert_load")
    _need(scores, T * N, "scores")
    _check(lib().moe_route(ctypes.byref(shape), _dt(u), _ptr(u), _ptr(centroids), _ptr(bias), _ptr(topk_idx),
                           _ptr(topk_gate), _ptr(expert_load), _ptr(scores), _ptr(workspace), _nbytes(workspace),
                           _stream(stream)))


def moe_permute(shape: moe_shape, topk_idx, u, expert_offsets, perm_token, row_of, a=None, a_dtype=None,
                a_scale=None, gather=1, workspace=None, stream=None):
    T, d, N, K = shape.T, shape.d, shape.n_routed, shape.topk
    _need(topk_idx, T * K, "topk_idx"); _need(expert_offsets, N + 1, "expert_offsets")
    _need(perm_token, T * K, "perm_token"); _need(row_of, T * K, "row_of")
    act = _dt(u) if u is not None else MOE_BF16
    if a is not None:
        rows = T * K if gather else T
        _need(u, T * d, "u"); _need(a, rows * d, "a")
        if a_dtype is None:
            a_dtype = _dt(a)
        if a_dtype in (MOE_F8E4M3, MOE_F8E4M3_POW2):
            _need(a_scale, rows * (d // 128), "a_scale")
    _check(lib().moe_permute(ctypes.byref(shape), act, _ptr(topk_idx), _ptr(u), _ptr(expert_offsets),
                             _ptr(perm_token), _ptr(row_of), _ptr(a), a_dtype if a_dtype is not None else act,
                             _ptr(a_scale), int(gather), _ptr(workspace), _nbytes(workspace), _stream(stream)))


def moe_permute_noalloc(shape: moe_shape, topk_idx, u, expert_offsets, perm_token, row_of, a=None, a_dtype=None,
                        a_scale=None, gather=1, stream=None):
    """moe_permute on the library's static scratch: no workspace, nothing allocated."""
    T, d, N, K = shape.T, shape.d, shape.n_routed, shape.topk
    _need(topk_idx, T * K, "topk_idx"); _need(expert_offsets, N + 1, "expert_offsets")
    _need(perm_token, T * K, "perm_token"); _need(row_of, T * K, "row_of")
    act = _dt(u) if u is not None else MOE_BF16
    if a is not None:
        rows = T * K if gather else T
        _need(u, T * d, "u"); _need(a, rows * d, "a")
        if a_dtype is None:
            a_dtype = _dt(a)
        if a_dtype in (MOE_F8E4M3, MOE_F8E4M3_POW2):
            _need(a_scale, rows * (d // 128), "a_scale")
    _check(lib().moe_permute_noalloc(ctypes.byref(shape), act, _ptr(topk_idx), _ptr(u), _ptr(expert_offsets),
                                     _ptr(perm_token), _ptr(row_of), _ptr(a), a_dtype if a_dtype is not None else act,
                                     _ptr(a_scale), int(gather), _stream(stream)))


def _wscale_count(w: int, rows: int, cols: int) -> int:
    """Weight-scale entries of one [rows, cols] matrix: fp32 per 128x128 block, or E8M0 bytes per 1x32 (MXFP4,
    rows padded to whole 256-row tiles)."""
    return mx_rows(rows) * cols // 32 if w == MOE_F4E2M1 else (rows // 128) * (cols // 128)


def mx_rows(rows: int) -> int:
    """Rows of a matrix in the tiled E4M3 / MXFP4 weight layouts: whole 256-row tiles."""
    return -(-rows // 256) * 256


def moe_grouped_ffn(shape: moe_shape, w: int, n_experts: int, n_rows: int, expert_offsets, mode: int, row_src,
                    a, a_scale, a_rows: int, w_gate_up, w_gu_scale, w_down, w_d_scale, y, workspace=None,
                    stream=None):
    d, I = shape.d, shape.inter
    wdiv = 2 if w == MOE_F4E2M1 else 1            # MXFP4: two codes per byte
    _need(expert_offsets, n_experts + 1, "expert_offsets"); _need(a, a_rows * d, "a")
    _need(w_gate_up, n_experts * 2 * I * d // wdiv, "w_gate_up")
    _need(w_down, n_experts * (mx_rows(d) if w in (MOE_F8E4M3, MOE_F4E2M1, MOE_BF16_TILED) else d) * I // wdiv,
          "w_down")
    _need(y, n_rows * d, "y")
    if mode == MOE_ROWS_GATHER:
        _need(row_src, n_rows, "row_src")
    if w in (MOE_F8E4M3, MOE_F4E2M1):
        _need(a_scale, a_rows * (d // 128), "a_scale")
        _need(w_gu_scale, n_experts * _wscale_count(w, 2 * I, d), "w_gu_scale")
        _need(w_d_scale, n_experts * _wscale_count(w, d, I), "w_d_scale")
    _check(lib().moe_grouped_ffn(ctypes.byref(shape), w, n_experts, n_rows, _ptr(expert_offsets), mode,
                                 _ptr(row_src), _ptr(a), _ptr(a_scale), a_rows, _ptr(w_gate_up), _ptr(w_gu_scale),
                                 _ptr(w_down), _ptr(w_d_scale), _dt(y), _ptr(y), _ptr(workspace),
                                 _nbytes(workspace), _stream(stream)))


def moe_ffn_gate_up(shape: moe_shape, w: int, n_experts: int, n_rows: int, expert_offsets, mode: int, row_src,
                    a, a_scale, a_rows: int, w_gate_up, w_gu_scale, h, h_scale=None, workspace=None, stream=None):
    d, I = shape.d, shape.inter
    wdiv = 2 if w == MOE_F4E2M1 else 1
    _need(expert_offsets, n_experts + 1, "expert_offsets"); _need(a, a_rows * d, "a")
    _need(w_gate_up, n_experts * 2 * I * d // wdiv, "w_gate_up"); _need(h, n_rows * I, "h")
    if mode == MOE_ROWS_GATHER:
        _need(row_src, n_rows, "row_src")
    if w in (MOE_F8E4M3, MOE_F4E2M1):
        _need(a_scale, a_rows * (d // 128), "a_scale")
        _need(w_gu_scale, n_experts * _wscale_count(w, 2 * I, d), "w_gu_scale")
        _need(h_scale, n_rows * (I // 128), "h_scale")
    _check(lib().moe_ffn_gate_up(ctypes.byref(shape), w, n_experts, n_rows, _ptr(expert_offsets), mode,
                                 _ptr(row_src), _ptr(a), _ptr(a_scale), a_rows, _ptr(w_gate_up), _ptr(w_gu_scale),
                                 _ptr(h), _ptr(h_scale), _ptr(workspace), _nbytes(workspace), _stream(stream)))


def moe_ffn_down(shape: moe_shape, w: int, n_experts: int, n_rows: int, expert_offsets, h, h_scale, w_down,
                 w_d_scale, y, workspace=None, stream=None):
    d, I = shape.d, shape.inter
    wdiv = 2 if w == MOE_F4E2M1 else 1
    _need(expert_offsets, n_experts + 1, "expert_offsets"); _need(h, n_rows * I, "h")
    _need(w_down, n_experts * (mx_rows(d) if w in (MOE_F8E4M3, MOE_F4E2M1, MOE_BF16_TILED) else d) * I // wdiv,
          "w_down")
    _need(y, n_rows * d, "y")
    if w in (MOE_F8E4M3, MOE_F4E2M1):
        _need(h_scale, n_rows * (I // 128), "h_scale")
        _need(w_d_scale, n_experts * _wscale_count(w, d, I), "w_d_scale")
    _check(lib().moe_ffn_down(ctypes.byref(shape), w, n_experts, n_rows, _ptr(expert_offsets), _ptr(h),
                              _ptr(h_scale), _ptr(w_down), _ptr(w_d_scale), _dt(y), _ptr(y), _ptr(workspace),
                              _nbytes(workspace), _stream(stream)))


def moe_balance_stats(shape: moe_shape, scores, topk_idx, seq_len: int, alpha: float, f, P, loss, workspace,
                      stream=None):
    T, N, K = shape.T, shape.n_routed, shape.topk
    n_seq = -(-T // seq_len)
    _need(scores, T * N, "scores"); _need(topk_idx, T * K, "topk_idx")
    _need(f, n_seq * N, "f"); _need(P, n_seq * N, "P"); _need(loss, n_seq, "loss")
    _check(lib().moe_balance_stats(ctypes.byref(shape), _ptr(scores), _ptr(topk_idx), seq_len, ctypes.c_float(alpha),
                                   _ptr(f), _ptr(P), _ptr(loss), _ptr(workspace), _nbytes(workspace),
                                   _stream(stream)))


def moe_combine(shape: moe_shape, u, y_routed, row_of, topk_gate, y_shared, out, stream=None):
    T, d, K, Ns = shape.T, shape.d, shape.topk, shape.n_shared
    _need(u, T * d, "u"); _need(y_routed, T * K * d, "y_routed"); _need(row_of, T * K, "row_of")
    _need(topk_gate, T * K, "topk_gate"); _need(out, T * d, "out")
    if Ns:
        _need(y_shared, Ns * T * d, "y_shared")
    _check(lib().moe_combine(ctypes.byref(shape), _dt(u), _ptr(u), _ptr(y_routed), _ptr(row_of), _ptr(topk_gate),
                             _ptr(y_shared), _ptr(out), _stream(stream)))


def moe_bias_update(shape: moe_shape, expert_load, gamma: float, bias, stream=None):
    _need(expert_load, shape.n_routed, "expert_load"); _need(bias, shape.n_routed, "bias")
    _check(lib().moe_bias_update(ctypes.byref(shape), _ptr(expert_load), float(gamma), _ptr(bias),
                                 _stream(stream)))


def moe_quantize_weights(w, codes, scale, gate_up: bool, stream=None):
    """w [n, rows, cols] bf16 -> E4M3 codes in the tiled layout (n * ceil(rows/256)*256 * cols bytes) and fp32
    block scales [n, rows/128, cols/128] (gate_up: rows = 2I, gate rows then up rows)."""
    n, rows, cols = w.shape
    _need(codes, n * mx_rows(rows) * cols, "codes"); _need(scale, n * (rows // 128) * (cols // 128), "scale")
    _check(lib().moe_quantize_weights(n, rows, cols, int(gate_up), _ptr(w), _ptr(codes), _ptr(scale),
                                      _stream(stream)))


def moe_quantize_weights_mxfp4(w, codes, scales, gate_up: bool, stream=None):
    """w [n, rows, cols] bf16 -> MXFP4 in the tiled layout: codes n * ceil(rows/256)*256 * cols/2 bytes, scales
    n * ceil(rows/256)*256 * cols/32 bytes (gate_up: rows = 2I, gate rows then up rows)."""
    n, rows, cols = w.shape
    _need(codes, n * mx_rows(rows) * cols // 2, "codes"); _need(scales, n * mx_rows(rows) * (cols // 32), "scales")
    _check(lib().moe_quantize_weights_mxfp4(n, rows, cols, int(gate_up), _ptr(w), _ptr(codes), _ptr(scales),
                                            _stream(stream)))


def moe_tile_weights_bf16(w, out, gate_up: bool, stream=None):
    """w [n, rows, cols] bf16 -> out: the tiled layout of MOE_BF16_TILED (n * ceil(rows/256)*256 * cols bf16)."""
    n, rows, cols = w.shape
    _need(out, n * mx_rows(rows) * cols, "out")
    _check(lib().moe_tile_weights_bf16(n, rows, cols, int(gate_up), _ptr(w), _ptr(out), _stream(stream)))


# ---------------------------------------------------------------- backward

def moe_ffn_gate_up_cache(shape: moe_shape, w: int, n_experts: int, n_rows: int, expert_offsets, mode: int, row_src,
                          a, a_rows: int, w_gate_up, h, gu_cache, workspace=None, stream=None):
    d, I = shape.d, shape.inter
    _need(expert_offsets, n_experts + 1, "expert_offsets"); _need(a, a_rows * d, "a")
    _need(h, n_rows * I, "h"); _need(gu_cache, n_rows * 2 * I, "gu_cache")
    if mode == MOE_ROWS_GATHER:
        _need(row_src, n_rows, "row_src")
    _check(lib().moe_ffn_gate_up_cache(ctypes.byref(shape), w, n_experts, n_rows, _ptr(expert_offsets), mode,
                                       _ptr(row_src), _ptr(a), a_rows, _ptr(w_gate_up), _ptr(h), _ptr(gu_cache),
                                       _ptr(workspace), _nbytes(workspace), _stream(stream)))


def moe_combine_backward(shape: moe_shape, d_out, y_routed, row_of, topk_gate, dy, d_gate, stream=None):
    T, d, K = shape.T, shape.d, shape.topk
    _need(d_out, T * d, "d_out"); _need(y_routed, T * K * d, "y_routed"); _need(row_of, T * K, "row_of")
    _need(topk_gate, T * K, "topk_gate"); _need(dy, (T * K + shape.n_shared * T) * d, "dy")
    _need(d_gate, T * K, "d_gate")
    _check(lib().moe_combine_backward(ctypes.byref(shape), _dt(d_out), _ptr(d_out), _ptr(y_routed), _ptr(row_of),
                                      _ptr(topk_gate), _dt(dy), _ptr(dy), _ptr(d_gate), _stream(stream)))


def moe_route_backward(shape: moe_shape, u, centroids, scores, topk_idx, d_gate, expert_offsets, perm_token, row_of,
                       du_router, d_centroids, workspace, stream=None):
    T, d, N, K = shape.T, shape.d, shape.n_routed, shape.topk
    _need(u, T * d, "u"); _need(centroids, N * d, "centroids"); _need(scores, T * N, "scores")
    _need(du_router, T * d, "du_router"); _need(d_centroids, N * d, "d_centroids")
    _check(lib().moe_route_backward(ctypes.byref(shape), _dt(u), _ptr(u), _ptr(centroids), _ptr(scores),
                                    _ptr(topk_idx), _ptr(d_gate), _ptr(expert_offsets), _ptr(perm_token),
                                    _ptr(row_of), _ptr(du_router), _ptr(d_centroids), _ptr(workspace),
                                    _nbytes(workspace), _stream(stream)))


def moe_transpose_weights_bf16(w, out, stream=None):
    """w [n, rows, cols] bf16 -> out: W^T [n, cols, rows] in the tiled layout (n * ceil(cols/256)*256 * rows)."""
    n, rows, cols = w.shape
    _need(out, n * mx_rows(cols) * rows, "out")
    _check(lib().moe_transpose_weights_bf16(n, rows, cols, _ptr(w), _ptr(out), _stream(stream)))


def moe_ffn_backward_workspace_bytes(shape: moe_shape, n_rows: int) -> int:
    return int(lib().moe_ffn_backward_workspace_bytes(ctypes.byref(shape), n_rows))


def moe_ffn_backward(shape: moe_shape, n_experts: int, n_rows: int, expert_offsets, mode: int, row_src, a,
                     a_rows: int, gu_cache, w_gate_up_t, w_down_t, dy, da, dw_gate_up, dw_down, workspace,
                     stream=None):
    d, I = shape.d, shape.inter
    _need(expert_offsets, n_experts + 1, "expert_offsets"); _need(a, a_rows * d, "a")
    _need(gu_cache, n_rows * 2 * I, "gu_cache"); _need(dy, n_rows * d, "dy"); _need(da, n_rows * d, "da")
    _need(w_gate_up_t, n_experts * mx_rows(d) * 2 * I, "w_gate_up_t")
    _need(w_down_t, n_experts * mx_rows(I) * d, "w_down_t")
    _need(dw_gate_up, n_experts * 2 * I * d, "dw_gate_up"); _need(dw_down, n_experts * d * I, "dw_down")
    if mode == MOE_ROWS_GATHER:
        _need(row_src, n_rows, "row_src")
    _check(lib().moe_ffn_backward(ctypes.byref(shape), MOE_BF16_TILED, n_experts, n_rows, _ptr(expert_offsets), mode,
                                  _ptr(row_src), _ptr(a), a_rows, _ptr(gu_cache), _ptr(w_gate_up_t), _ptr(w_down_t),
                                  _ptr(dy), _ptr(da), _ptr(dw_gate_up), _ptr(dw_down), _ptr(workspace),
                                  _nbytes(workspace), _stream(stream)))


def moe_input_grad(shape: moe_shape, d_out, du_router, da, row_of, du, stream=None):
    T, d = shape.T, shape.d
    _need(d_out, T * d, "d_out"); _need(du, T * d, "du")
    _need(da, (T * shape.topk + shape.n_shared * T) * d, "da")
    _check(lib().moe_input_grad(ctypes.byref(shape), _ptr(d_out), _ptr(du_router), _ptr(da), _ptr(row_of), _ptr(du),
                                _stream(stream)))


# ---------------------------------------------------------------- FP8 backward

def moe_transpose_bf16(w, out, stream=None):
    """w [n, rows, cols] bf16 -> out [n, cols, rows] (row-major)."""
    n, rows, cols = w.shape
    _need(out, n * rows * cols, "out")
    _check(lib().moe_transpose_bf16(n, rows, cols, _ptr(w), _ptr(out), _stream(stream)))


def moe_ffn_gate_up_cache_fp8(shape: moe_shape, n_experts: int, n_rows: int, expert_offsets, mode: int, row_src,
                              a_codes, a_scale, a_rows: int, w_gate_up, w_gu_scale, h_codes, h_scale, gu_codes,
                              gu_scale, workspace=None, stream=None):
    d, I = shape.d, shape.inter
    _need(expert_offsets, n_experts + 1, "expert_offsets"); _need(a_codes, a_rows * d, "a_codes")
    _need(a_scale, a_rows * (d // 128), "a_scale"); _need(h_codes, n_rows * I, "h_codes")
    _need(h_scale, n_rows * (I // 128), "h_scale"); _need(gu_codes, n_rows * 2 * I, "gu_codes")
    _need(gu_scale, n_rows * (2 * I // 128), "gu_scale")
    _need(w_gate_up, n_experts * mx_rows(2 * I) * d, "w_gate_up")
    if mode == MOE_ROWS_GATHER:
        _need(row_src, n_rows, "row_src")
    _check(lib().moe_ffn_gate_up_cache_fp8(ctypes.byref(shape), n_experts, n_rows, _ptr(expert_offsets), mode,
                                           _ptr(row_src), _ptr(a_codes), _ptr(a_scale), a_rows, _ptr(w_gate_up),
                                           _ptr(w_gu_scale), _ptr(h_codes), _ptr(h_scale), _ptr(gu_codes),
                                           _ptr(gu_scale), _ptr(workspace), _nbytes(workspace), _stream(stream)))


def moe_ffn_backward_fp8_workspace_bytes(shape: moe_shape, n_rows: int, n_experts: int) -> int:
    return int(lib().moe_ffn_backward_fp8_workspace_bytes(ctypes.byref(shape), n_rows, n_experts))


def moe_ffn_backward_fp8(shape: moe_shape, n_experts: int, n_rows: int, expert_offsets, mode: int, row_src, a_codes,
                         a_scale, a_rows: int, gu_codes, gu_scale, w_gate_up_t, w_gate_up_t_scale, w_down_t,
                         w_down_t_scale, dy, da, dw_gate_up, dw_down, workspace, stream=None):
    d, I = shape.d, shape.inter
    _need(expert_offsets, n_experts + 1, "expert_offsets"); _need(a_codes, a_rows * d, "a_codes")
    _need(a_scale, a_rows * (d // 128), "a_scale"); _need(gu_codes, n_rows * 2 * I, "gu_codes")
    _need(gu_scale, n_rows * (2 * I // 128), "gu_scale")
    _need(w_gate_up_t, n_experts * mx_rows(d) * 2 * I, "w_gate_up_t")
    _need(w_gate_up_t_scale, n_experts * (d // 128) * (2 * I // 128), "w_gate_up_t_scale")
    _need(w_down_t, n_experts * mx_rows(I) * d, "w_down_t")
    _need(w_down_t_scale, n_experts * (I // 128) * (d // 128), "w_down_t_scale")
    _need(dy, n_rows * d, "dy"); _need(da, n_rows * d, "da")
    _need(dw_gate_up, n_experts * 2 * I * d, "dw_gate_up"); _need(dw_down, n_experts * d * I, "dw_down")
    if mode == MOE_ROWS_GATHER:
        _need(row_src, n_rows, "row_src")
    _check(lib().moe_ffn_backward_fp8(ctypes.byref(shape), n_experts, n_rows, _ptr(expert_offsets), mode,
                                      _ptr(row_src), _ptr(a_codes), _ptr(a_scale), a_rows, _ptr(gu_codes),
                                      _ptr(gu_scale), _ptr(w_gate_up_t), _ptr(w_gate_up_t_scale), _ptr(w_down_t),
                                      _ptr(w_down_t_scale), _ptr(dy), _ptr(da), _ptr(dw_gate_up), _ptr(dw_down),
                                      _ptr(workspace), _nbytes(workspace), _stream(stream)))
