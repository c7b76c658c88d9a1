"""The C ABI loads, exports every call declared in include/moe.h, and rejects
bad arguments on the host before any HIP call (runs without a GPU)."""
import ctypes
import os
import re

import pytest

from mixture_experts_layer_gate_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    txt = open(os.path.join(ROOT, "include", "moe.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert {"moe_route", "moe_permute", "moe_grouped_ffn", "moe_combine", "moe_bias_update"} <= set(names)
    L = B.lib()
    for n in names:
        assert hasattr(L, n), n
    assert L.moe_version().startswith(b"moe-gfx950")


def _shape(**kw):
    base = dict(T=64, d=256, n_routed=16, n_groups=4, topk_groups=2, group_topn=2, topk=2, n_shared=1, inter=128,
                batch_invariant=0)
    base.update(kw)
    return B.moe_shape(*[base[k] for k, _ in B.moe_shape._fields_])


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


def _route(shape, **ptrs):
    p = dict(u=FAKE, c=FAKE, b=FAKE, i=FAKE, g=FAKE, l=FAKE, s=FAKE)
    p.update(ptrs)
    L = B.lib()
    st = L.moe_route(ctypes.byref(shape), B.MOE_BF16, p["u"], p["c"], p["b"], p["i"], p["g"], p["l"], p["s"],
                     None, 0, None)
    return st, L.moe_last_error().decode()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(T=0), B.MOE_E_INVALID, "non-positive"),
    (dict(batch_invariant=2), B.MOE_E_INVALID, "batch_invariant"),
    (dict(n_routed=15), B.MOE_E_INVALID, "multiple of n_groups"),
    (dict(topk_groups=5), B.MOE_E_INVALID, "topk_groups"),
    (dict(topk=9), B.MOE_E_INVALID, "topk"),
    (dict(group_topn=5), B.MOE_E_INVALID, "group_topn"),
    (dict(d=200), B.MOE_E_UNSUPPORTED, "multiple of 128"),
    (dict(inter=100), B.MOE_E_UNSUPPORTED, "multiple of 128"),
    (dict(n_routed=2048, n_groups=2048 // 4, topk_groups=2), B.MOE_E_UNSUPPORTED, ""),
    (dict(topk=17, n_routed=64, n_groups=1, topk_groups=1), B.MOE_E_UNSUPPORTED, "topk"),
])
def test_route_rejects_bad_shapes(kw, status, needle):
    st, msg = _route(_shape(**kw))
    assert st == status, msg
    assert needle in msg


def test_route_rejects_null_and_missing_workspace():
    st, msg = _route(_shape(), u=None)
    assert st == B.MOE_E_INVALID and "NULL" in msg
    st, msg = _route(_shape(), s=None)   # no scores buffer and no workspace
    assert st == B.MOE_E_WORKSPACE and "workspace" in msg
    st, msg = _route(_shape())           # scores given: the K-slice partial sums still need the workspace
    assert st == B.MOE_E_WORKSPACE and "workspace" in msg


def test_balance_stats_validation():
    L = B.lib()
    sh = _shape()
    call = lambda seq, ws, nb: L.moe_balance_stats(ctypes.byref(sh), FAKE, FAKE, seq, ctypes.c_float(1e-4), FAKE, FAKE,
                                                    FAKE, ws, nb, None)
    assert call(0, FAKE, 1 << 20) == B.MOE_E_INVALID
    assert call(16, None, 0) == B.MOE_E_WORKSPACE
    assert L.moe_balance_stats(ctypes.byref(sh), None, FAKE, 16, ctypes.c_float(1e-4), FAKE, FAKE, FAKE, FAKE, 1 << 20,
                               None) == B.MOE_E_INVALID
    assert B.moe_workspace_bytes(sh, B.MOE_BF16) >= 64 * 16 * 8     # seq_len = 1: one chunk per token


def test_ffn_phases_need_queue_workspace():
    """The split FFN calls take their work-queue counters from the caller's workspace (no allocation)."""
    L = B.lib()
    sh = _shape()
    for ws, nb in ((None, 0), (FAKE, 64)):
        assert L.moe_ffn_gate_up(ctypes.byref(sh), B.MOE_BF16, 4, 10, FAKE, B.MOE_ROWS_DIRECT, None, FAKE, None, 10,
                                 FAKE, None, FAKE, None, ws, nb, None) == B.MOE_E_WORKSPACE
        assert b"workspace" in L.moe_last_error()
        assert L.moe_ffn_down(ctypes.byref(sh), B.MOE_BF16, 4, 10, FAKE, FAKE, None, FAKE, None, B.MOE_BF16, FAKE,
                              ws, nb, None) == B.MOE_E_WORKSPACE


def test_grouped_ffn_validation():
    L = B.lib()
    sh = _shape()
    args = lambda **o: [ctypes.byref(sh), o.get("w", B.MOE_BF16), o.get("ne", 4), o.get("nr", 10), FAKE,
                        o.get("mode", B.MOE_ROWS_GATHER), o.get("rs", FAKE), FAKE, o.get("asc", None),
                        o.get("ar", 10), FAKE, o.get("gs", None), FAKE, o.get("ds", None), o.get("ydt", B.MOE_BF16),
                        FAKE, None, o.get("ws", 0), None]
    assert L.moe_grouped_ffn(*args(rs=None)) == B.MOE_E_INVALID
    assert L.moe_grouped_ffn(*args(mode=7)) == B.MOE_E_INVALID
    assert L.moe_grouped_ffn(*args(ydt=B.MOE_F32)) == B.MOE_E_INVALID
    assert L.moe_grouped_ffn(*args(w=B.MOE_F8E4M3)) == B.MOE_E_INVALID     # missing scales
    assert L.moe_grouped_ffn(*args(w=B.MOE_F8E4M3_POW2, asc=FAKE, gs=FAKE, ds=FAKE)) == B.MOE_E_INVALID
    assert L.moe_grouped_ffn(*args(w=B.MOE_F4E2M1)) == B.MOE_E_INVALID       # MXFP4 needs its scales too
    assert L.moe_grouped_ffn(*args(w=B.MOE_F4E2M1, asc=FAKE, gs=FAKE, ds=FAKE)) == B.MOE_E_WORKSPACE
    assert L.moe_grouped_ffn(*args()) == B.MOE_E_WORKSPACE
    assert b"workspace" in L.moe_last_error()


def test_grouped_ffn_refuses_32_bit_offset_overflow():
    """The expert GEMM kernels address rows through 32-bit byte offsets: shapes whose gathered activations, H or
    one expert's weights would pass 4 GiB are refused before any launch (the router splits its token range
    instead)."""
    L = B.lib()
    sh = _shape(d=7168, inter=2048)

    def call(w, nr, ar, shape=sh):
        scales = FAKE if w in (B.MOE_F8E4M3, B.MOE_F4E2M1) else None
        return L.moe_grouped_ffn(ctypes.byref(shape), w, 4, nr, FAKE, B.MOE_ROWS_GATHER, FAKE, FAKE, scales, ar, FAKE,
                                 scales, FAKE, scales, B.MOE_BF16, FAKE, FAKE, 1 << 40, None)

    for w in (B.MOE_BF16, B.MOE_BF16_TILED):
        assert call(w, 1000, 299_594) == B.MOE_E_UNSUPPORTED           # a_rows * d * 2 >= 2^32
        assert b"a_rows" in L.moe_last_error()
        assert call(w, 1 << 20, 1000) == B.MOE_E_UNSUPPORTED           # n_rows * inter * 2 >= 2^32
        assert call(w, 1000, 299_000, _shape(d=7168, inter=150016)) == B.MOE_E_UNSUPPORTED   # 2 I d * 2 >= 2^32
    for w in (B.MOE_F8E4M3, B.MOE_F4E2M1):
        assert call(w, 1000, 599_187) == B.MOE_E_UNSUPPORTED           # a_rows * d >= 2^32
        assert call(w, 1 << 21, 1000) == B.MOE_E_UNSUPPORTED           # n_rows * inter >= 2^32


def test_grouped_ffn_expert_count_limits():
    """At most 4096 experts per grouped call, 2048 on the bf16 and MXFP4 paths (their schedule table shares
    the LDS with the ring): refused before any launch."""
    L = B.lib()
    sh = _shape(d=256, inter=128)

    def call(w, ne):
        scales = FAKE if w in (B.MOE_F8E4M3, B.MOE_F4E2M1) else None
        return L.moe_grouped_ffn(ctypes.byref(sh), w, ne, 64, FAKE, B.MOE_ROWS_GATHER, FAKE, FAKE, scales, 64, FAKE,
                                 scales, FAKE, scales, B.MOE_BF16, FAKE, FAKE, 1 << 40, None)

    for w in (B.MOE_BF16, B.MOE_BF16_TILED, B.MOE_F4E2M1):
        assert call(w, 2049) == B.MOE_E_UNSUPPORTED
        assert b"2048" in L.moe_last_error()
    for w in (B.MOE_F32, B.MOE_F8E4M3):
        assert call(w, 4097) == B.MOE_E_UNSUPPORTED


def test_permute_combine_bias_validation():
    L = B.lib()
    sh = _shape()
    assert L.moe_permute(ctypes.byref(sh), B.MOE_BF16, None, FAKE, FAKE, FAKE, FAKE, None, B.MOE_BF16, None, 1,
                         None, 0, None) == B.MOE_E_INVALID
    # gather=0 without quantisation is refused
    assert L.moe_permute(ctypes.byref(sh), B.MOE_BF16, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, B.MOE_BF16, None, 0,
                         FAKE, 1 << 20, None) == B.MOE_E_INVALID
    assert L.moe_permute(ctypes.byref(sh), B.MOE_BF16, FAKE, FAKE, FAKE, FAKE, FAKE, None, B.MOE_BF16, None, 1,
                         FAKE, 16, None) == B.MOE_E_WORKSPACE
    # power-of-two fp8 output needs its scales; an unknown a_dtype is refused; E4M3_POW2 is no weight dtype
    assert L.moe_permute(ctypes.byref(sh), B.MOE_BF16, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, B.MOE_F8E4M3_POW2, None,
                         0, FAKE, 1 << 20, None) == B.MOE_E_INVALID
    assert L.moe_permute(ctypes.byref(sh), B.MOE_BF16, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, FAKE, 0,
                         FAKE, 1 << 20, None) == B.MOE_E_INVALID
    assert L.moe_combine(ctypes.byref(sh), B.MOE_BF16, FAKE, FAKE, FAKE, FAKE, None, FAKE, None) == B.MOE_E_INVALID
    assert L.moe_bias_update(ctypes.byref(sh), FAKE, ctypes.c_float(-1.0), FAKE, None) == B.MOE_E_INVALID
    assert L.moe_quantize_weights(1, 100, 128, 0, FAKE, FAKE, FAKE, None) == B.MOE_E_UNSUPPORTED
    assert L.moe_quantize_weights(1, 384, 128, 1, FAKE, FAKE, FAKE, None) == B.MOE_E_UNSUPPORTED     # 2I % 256
    assert L.moe_quantize_weights(1, 256, 128, 2, FAKE, FAKE, FAKE, None) == B.MOE_E_INVALID
    assert L.moe_quantize_weights_mxfp4(1, 100, 96, 0, FAKE, FAKE, FAKE, None) == B.MOE_E_UNSUPPORTED   # K % 128
    assert L.moe_quantize_weights_mxfp4(1, 384, 128, 1, FAKE, FAKE, FAKE, None) == B.MOE_E_UNSUPPORTED  # 2I % 256
    assert L.moe_quantize_weights_mxfp4(1, 100, 128, 2, FAKE, FAKE, FAKE, None) == B.MOE_E_INVALID
    assert L.moe_quantize_weights_mxfp4(1, 100, 128, 0, FAKE, None, FAKE, None) == B.MOE_E_INVALID
    assert L.moe_quantize_weights_mxfp4(0, 100, 128, 0, FAKE, FAKE, FAKE, None) == B.MOE_E_INVALID


def test_workspace_size_covers_each_call():
    sh = _shape(T=8192, d=7168, n_routed=256, n_groups=8, topk_groups=4, topk=8, inter=2048)
    n = B.moe_workspace_bytes(sh, B.MOE_BF16)
    assert n >= 8192 * 8 * 2048 * 2         # H for the routed rows in bf16
    assert n >= 8192 * 256 * 4              # the router scores
    n8 = B.moe_workspace_bytes(sh, B.MOE_F8E4M3)
    assert 8192 * 8 * 2048 <= n8 < n
    assert B.moe_workspace_bytes(_shape(T=-1), B.MOE_BF16) == 0


def test_backward_validation():
    L = B.lib()
    sh = _shape()
    P = lambda: [FAKE] * 3
    # the SwiGLU-input cache is a bf16-weight feature
    assert L.moe_ffn_gate_up_cache(ctypes.byref(sh), B.MOE_F8E4M3, 4, 10, FAKE, B.MOE_ROWS_GATHER, FAKE, FAKE, 10,
                                   FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == B.MOE_E_INVALID
    assert L.moe_ffn_gate_up_cache(ctypes.byref(sh), B.MOE_BF16, 4, 10, FAKE, B.MOE_ROWS_GATHER, FAKE, FAKE, 10,
                                   FAKE, FAKE, None, FAKE, 1 << 20, None) == B.MOE_E_INVALID
    assert L.moe_ffn_gate_up_cache(ctypes.byref(sh), B.MOE_BF16, 4, 10, FAKE, B.MOE_ROWS_GATHER, FAKE, FAKE, 10,
                                   FAKE, FAKE, FAKE, FAKE, 16, None) == B.MOE_E_WORKSPACE
    assert L.moe_combine_backward(ctypes.byref(sh), B.MOE_F32, *P(), FAKE, B.MOE_BF16, FAKE, FAKE, None) == B.MOE_E_INVALID
    assert L.moe_combine_backward(ctypes.byref(sh), B.MOE_BF16, *P(), FAKE, B.MOE_BF16, None, FAKE, None) == B.MOE_E_INVALID
    assert L.moe_combine_backward(ctypes.byref(sh), B.MOE_BF16, *P(), FAKE, B.MOE_F8E4M3, FAKE, FAKE, None) == B.MOE_E_INVALID
    assert L.moe_route_backward(ctypes.byref(sh), B.MOE_BF16, *P(), *P(), *P(), FAKE, FAKE, 64 * 2 * 4 - 4,
                                None) == B.MOE_E_WORKSPACE
    assert L.moe_route_backward(ctypes.byref(sh), B.MOE_F8E4M3, *P(), *P(), *P(), FAKE, FAKE, 1 << 20,
                                None) == B.MOE_E_INVALID
    assert L.moe_transpose_weights_bf16(1, 100, 128, FAKE, ctypes.c_void_p(32), None) == B.MOE_E_UNSUPPORTED
    assert L.moe_transpose_weights_bf16(1, 128, 128, FAKE, FAKE, None) == B.MOE_E_INVALID        # in place
    assert L.moe_transpose_weights_bf16(0, 128, 128, FAKE, ctypes.c_void_p(32), None) == B.MOE_E_INVALID
    need = B.moe_ffn_backward_workspace_bytes(sh, 10)
    assert need >= 10 * 128 * 2 * 4
    args = lambda w=B.MOE_BF16_TILED, ws=need, dy=FAKE: [ctypes.byref(sh), w, 4, 10, FAKE, B.MOE_ROWS_GATHER, FAKE,
                                                       FAKE, 10, FAKE, FAKE, FAKE, dy, FAKE, FAKE, FAKE, FAKE, ws, None]
    assert L.moe_ffn_backward(*args(w=B.MOE_BF16)) == B.MOE_E_INVALID          # needs the transposed tiled weights
    assert L.moe_ffn_backward(*args(dy=None)) == B.MOE_E_INVALID
    assert L.moe_ffn_backward(*args(ws=need - 1)) == B.MOE_E_WORKSPACE
    assert b"workspace" in L.moe_last_error()
    assert L.moe_input_grad(ctypes.byref(sh), FAKE, None, None, FAKE, FAKE, None) == B.MOE_E_INVALID


def test_backward_fp8_validation():
    L = B.lib()
    sh = _shape()
    assert L.moe_transpose_bf16(1, 100, 128, FAKE, ctypes.c_void_p(32), None) == B.MOE_E_UNSUPPORTED
    assert L.moe_transpose_bf16(1, 128, 128, FAKE, FAKE, None) == B.MOE_E_INVALID
    gu = lambda **o: [ctypes.byref(sh), 4, 10, FAKE, B.MOE_ROWS_GATHER, FAKE, FAKE, FAKE, 10, FAKE, FAKE, FAKE, FAKE,
                      o.get("gq", FAKE), FAKE, FAKE, o.get("ws", 1 << 20), None]
    assert L.moe_ffn_gate_up_cache_fp8(*gu(gq=None)) == B.MOE_E_INVALID
    assert L.moe_ffn_gate_up_cache_fp8(*gu(ws=16)) == B.MOE_E_WORKSPACE
    need = B.moe_ffn_backward_fp8_workspace_bytes(sh, 10, 4)
    assert need >= 10 * 256 + 10 * 128 * 4 * 3
    bw = lambda **o: [ctypes.byref(o.get("sh", sh)), 4, 10, FAKE, B.MOE_ROWS_GATHER, FAKE, FAKE, FAKE, 10, FAKE, FAKE,
                      FAKE, FAKE, FAKE, FAKE, o.get("dy", FAKE), FAKE, FAKE, FAKE, FAKE, o.get("ws", need), None]
    assert L.moe_ffn_backward_fp8(*bw(dy=None)) == B.MOE_E_INVALID
    assert L.moe_ffn_backward_fp8(*bw(ws=need - 1)) == B.MOE_E_WORKSPACE
    wide = _shape(inter=5248)                                 # 2I > 10240
    assert L.moe_ffn_backward_fp8(*bw(sh=wide, ws=1 << 40)) == B.MOE_E_UNSUPPORTED


def test_peak_probe_library_is_separate():
    """The benchmark's peak probes live in libmoe_probe.so, outside the product library, and reject bad
    arguments before any launch."""
    import os
    L = B.lib()
    for name in ("moe_probe_mfma", "moe_probe_copy", "moe_probe_read", "probe_mfma"):
        assert not hasattr(L, name), name
    P = ctypes.CDLL(os.path.join(os.path.dirname(B.LIB_PATH), "libmoe_probe.so"))
    P.probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    P.probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    P.probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    assert P.probe_mfma(0, 0, FAKE, FAKE, None) == -1
    assert P.probe_copy(FAKE, FAKE, 1 << 20, None) == -1          # in place
    assert P.probe_copy(FAKE, ctypes.c_void_p(0x2000), 24, None) == -1
    assert P.probe_read(FAKE, 24, FAKE, None) == -1


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """With no built library every call raises: there is no CPU fallback."""
    from moe_inputs import get_config
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "libmoe.so"))
    monkeypatch.setattr(B, "_lib", None)
    with pytest.raises(ImportError, match="not built"):
        B.lib()
    with pytest.raises(ImportError, match="not built"):
        B.moe_workspace_bytes(B.moe_shape.of(get_config("c1")), 2)
