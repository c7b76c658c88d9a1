"""Pins of the oracle's FFN, fp8 codec/quantisation and combine (CPU only).

* P6: the permuted layer equals a dense all-experts computation masked by the
  gates (eq. (12) of "DeepSeek_V3_Report: Annotation").
* P10: the E4M3 codec against torch's float8_e4m3fn (a library routine) and
  the format's fixed points.
* P12: 6*d*I FLOPs per token-expert pair and 6hd/3h = 2d = 6144 for the
  V4-Pro expert width ("DeepSeek V3 / V4 Infra", V4 fine-grained EP section).
* P13: SwiGLU against torch's textbook SiLU.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle.e4m3 import e4m3_decode, e4m3_encode
from moe_inputs import get_config, generate, MoEConfig


# ---------------------------------------------------------------- P10 codec

def test_p10_decode_all_codes_match_library():
    codes = np.arange(256, dtype=np.uint8)
    mine = e4m3_decode(codes)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], lib[~nan])
    assert mine[0x7E] == 448.0 and mine[0x01] == 2.0 ** -9 and mine[0x08] == 2.0 ** -6 and mine[0x38] == 1.0
    assert np.isnan(mine[0x7F]) and np.isnan(mine[0xFF])


def test_p10_encode_matches_library_rne_in_range():
    rng = np.random.default_rng(0)
    grid = e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (grid[:-1] + grid[1:]) / 2                       # exact ties
    vals = np.concatenate([grid, mids, rng.uniform(0, 448, 20000), rng.uniform(0, 0.02, 20000)])
    vals = np.concatenate([vals, -vals]).astype(np.float32)
    lib = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3_encode(vals), lib)


def test_p10_quantum_encoder_matches_nearest_search():
    from oracle.e4m3 import e4m3_encode_nearest
    rng = np.random.default_rng(12)
    grid = e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (grid[:-1] + grid[1:]) / 2
    eps = np.nextafter(mids, np.inf) - mids
    vals = np.concatenate([grid, mids, mids + eps, mids - eps, rng.uniform(0, 500, 200000),
                           np.exp(rng.uniform(np.log(1e-5), np.log(600), 200000)), [0.0, 448.0, 464.0, 480.0, 1e9]])
    vals = np.concatenate([vals, -vals]).astype(np.float32)
    assert np.array_equal(e4m3_encode(vals), e4m3_encode_nearest(vals))


def test_p10_saturation_and_roundtrip_error():
    assert e4m3_encode(np.float32(1e6)) == 0x7E and e4m3_encode(np.float32(-500.0)) == 0xFE
    x = np.random.default_rng(1).uniform(2.0 ** -6, 448, 100000)
    rel = np.abs(e4m3_decode(e4m3_encode(x)) - x) / x
    assert rel.max() <= 2.0 ** -4


# ------------------------------------------------------------ quantisation

def test_quantize_tiles_fixed_points():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 384)).astype(np.float32)
    x[3] = 0.0
    codes, scale = oracle.quantize_tiles(x)
    assert scale.shape == (5, 3) and codes.dtype == np.uint8
    assert np.all(codes[3] == 0) and np.all(scale[3] == 1.0)
    for r in (0, 1, 2, 4):
        for j in range(3):
            tile = x[r, 128 * j:128 * (j + 1)]
            c = codes[r, 128 * j:128 * (j + 1)]
            m = np.argmax(np.abs(tile))
            assert c[m] & 0x7F == 0x7E                        # amax lands on +-448
    dq = oracle.dequantize_tiles(codes, scale)
    big = np.abs(x) > np.repeat(scale, 128, axis=1) * 2.0 ** -6 * 1.01
    assert np.all(np.abs(dq - x)[big] <= np.abs(x)[big] * 2.0 ** -4 * 1.0001)


def test_quantize_tiles_exact_for_representable_inputs():
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 0x7E, (4, 256)).astype(np.uint8)
    codes |= (rng.integers(0, 2, codes.shape) << 7).astype(np.uint8)
    codes[:, 5] = 0x7E
    codes[:, 200] = 0xFE
    x = (e4m3_decode(codes) * 2.0 ** -5).astype(np.float32)
    q, s = oracle.quantize_tiles(x)
    assert np.all(s == np.float32(2.0 ** -5))
    assert np.array_equal(e4m3_decode(q), e4m3_decode(codes))


def test_quantize_blocks_layout():
    rng = np.random.default_rng(4)
    w = rng.standard_normal((256, 384)).astype(np.float32)
    mag = np.array([[1, 8, 64], [512, 4096, 0.125]], np.float32)
    w *= np.repeat(np.repeat(mag, 128, axis=0), 128, axis=1)
    codes, scale = oracle.quantize_blocks(w)
    assert scale.shape == (2, 3)
    dq = oracle.dequantize_blocks(codes, scale)
    assert np.max(np.abs(dq - w) / np.abs(w).max()) < 2.0 ** -4
    for i in range(2):
        for j in range(3):
            blk = np.abs(w[128 * i:128 * (i + 1), 128 * j:128 * (j + 1)])
            assert np.isclose(scale[i, j] * 448.0, blk.max(), rtol=1e-6)


# ------------------------------------------------------------- SwiGLU, fp8 FFN

def test_p13_swiglu_matches_textbook():
    rng = np.random.default_rng(5)
    a = rng.standard_normal((17, 64))
    wgu = rng.standard_normal((2 * 48, 64)) * 0.1
    wd = rng.standard_normal((64, 48)) * 0.1
    ta, tg, tu, td = (torch.from_numpy(v) for v in (a, wgu[:48], wgu[48:], wd))
    ref = (F.silu(ta @ tg.T) * (ta @ tu.T)) @ td.T
    np.testing.assert_allclose(oracle.swiglu_ffn(a, wgu, wd), ref.numpy(), rtol=1e-12, atol=1e-14)


def _representable(rng, shape, exp2):
    c = rng.integers(0, 0x7E, shape).astype(np.uint8)
    c |= (rng.integers(0, 2, shape) << 7).astype(np.uint8)
    return c


def test_fp8_ffn_reduces_to_exact_on_representable_operands():
    """Representable a and W: gate/up are exact; the down projection sees quantised h."""
    rng = np.random.default_rng(6)
    n, d, I = 9, 256, 128
    ac = _representable(rng, (n, d), 0)
    ac[:, 0] = 0x7E
    ac[:, 130] = 0x7E
    a = (e4m3_decode(ac) * 2.0 ** -6).astype(np.float32)
    wc = _representable(rng, (2 * I, d), 0)
    wc[0:128:1, 0] = 0x7E  # each 128x128 block gets a 448 entry
    for bi in range(2):
        for bj in range(2):
            wc[128 * bi, 128 * bj] = 0x7E
    wgu = (e4m3_decode(wc) * 2.0 ** -12).astype(np.float32)
    wd = (np.eye(d, I) * 448.0 * 2.0 ** -12).astype(np.float32)  # scaled identity, amax 448*2^-12: exact
    gq, gs = oracle.quantize_blocks(wgu)
    dq_, ds_ = oracle.quantize_blocks(wd)
    y, aux = oracle.ffn_fp8(a, gq, gs, dq_, ds_, return_h=True)
    ta, tw = torch.from_numpy(a.astype(np.float64)), torch.from_numpy(wgu.astype(np.float64))
    h_exact = (F.silu(ta @ tw[:I].T) * (ta @ tw[I:].T)).to(torch.float32).numpy()
    np.testing.assert_allclose(aux["h32"], h_exact, rtol=2.0 ** -22, atol=0)
    hq = oracle.dequantize_tiles(*oracle.quantize_tiles(aux["h32"]))
    np.testing.assert_array_equal(y[:, :I], hq * (448.0 * 2.0 ** -12))
    assert np.all(y[:, I:] == 0)


def test_fp8_ffn_error_is_e4m3_sized():
    rng = np.random.default_rng(7)
    n, d, I = 32, 512, 256
    a = rng.standard_normal((n, d)).astype(np.float32)
    wgu = (rng.standard_normal((2 * I, d)) * 0.02).astype(np.float32)
    wd = (rng.standard_normal((d, I)) * 0.02).astype(np.float32)
    exact = oracle.swiglu_ffn(a, wgu, wd)
    y8 = oracle.expert_ffn(a, wgu, wd, "fp8")
    rel = np.linalg.norm(y8 - exact) / np.linalg.norm(exact)
    assert 1e-3 < rel < 0.08


# ------------------------------------------------------------- P6 dense check

def _dense_layer(cfg, inp, r, gemm):
    """u + sum_s FFN_s(u) + sum_i g'_i FFN_i(u), every expert on every token (torch fp64)."""
    u = inp["u"].to(torch.float64)
    T = u.shape[0]
    gp = torch.zeros((T, cfg.n_routed), dtype=torch.float64)
    gp.scatter_(1, torch.from_numpy(r["idx"]), torch.from_numpy(r["gate"]))

    def ffn(wg, wd):
        if gemm == "fp8":
            return torch.from_numpy(oracle.expert_ffn(u.numpy(), wg, wd, "fp8"))
        wg64, wd64 = wg.to(torch.float64), wd.to(torch.float64)
        I = wg64.shape[0] // 2
        return (F.silu(u @ wg64[:I].T) * (u @ wg64[I:].T)) @ wd64.T

    out = u.clone()
    for s in range(cfg.n_shared):
        out += ffn(inp["s_gate_up"][s], inp["s_down"][s])
    for i in range(cfg.n_routed):
        out += gp[:, i:i + 1] * ffn(inp["w_gate_up"][i], inp["w_down"][i])
    return out.numpy()


@pytest.mark.parametrize("gemm", ["f32", "fp8"])
def test_p6_layer_equals_dense_masked_sum_c1(gemm):
    cfg = get_config("c1", gemm=gemm)
    inp = generate(cfg, "cpu")
    res = oracle.layer_forward(cfg, inp)
    dense = _dense_layer(cfg, inp, res["route"], gemm)
    np.testing.assert_allclose(res["out"], dense, rtol=1e-10, atol=1e-12)
    # the FFN part is not negligible next to the residual
    ffn_part = res["out"] - inp["u"].double().numpy()
    assert np.linalg.norm(ffn_part) > 1e-3 * np.linalg.norm(res["out"])


def test_p6_layer_equals_dense_masked_sum_c2_small():
    cfg = get_config("c2", T=64, n_routed=16, n_groups=4, topk_groups=3, topk=6, d=256, inter=128)
    inp = generate(cfg, "cpu")
    res = oracle.layer_forward(cfg, inp)
    dense = _dense_layer(cfg, inp, res["route"], "bf16")
    np.testing.assert_allclose(res["out"], dense, rtol=1e-10, atol=1e-12)


def test_p12_flop_accounting():
    cfg = get_config("c3")
    assert cfg.ffn_flops() == 6 * 7168 * 2048 * 8192 * (8 + 1)
    # V4-Pro: 6hd FLOPs against 3h bytes per pair is 2d with d = 3072
    h, d = 7168, 3072
    assert (6 * h * d) / (3 * h) == 2 * d == 6144


# ---------------------------------------------------------------- power-of-two activation scales

def test_pow2_tile_scales():
    """Scales are powers of two, the smallest with every |x| / s <= 448; codes are the plain E4M3 encode of
    x / s; when amax / 448 is itself a power of two the fp32-scale quantiser gives the same codes."""
    rng = np.random.default_rng(12)
    x = (rng.standard_normal((64, 512)) * 10.0 ** rng.integers(-3, 4, (64, 1))).astype(np.float32)
    x[3] = 0.0
    codes, scale = oracle.quantize_tiles(x, pow2=True)
    m, _ = np.frexp(scale.astype(np.float64))
    assert np.all(m == 0.5)                                          # powers of two
    amax = np.abs(x).reshape(64, 4, 128).max(axis=2)
    v = (amax / np.float32(448)).astype(np.float32)
    nz = amax > 0
    assert np.all(v[nz] <= scale[nz]) and np.all(scale[nz] / 2 < v[nz])   # the smallest such power
    assert np.all(scale[~nz] == 1) and np.all(codes[3] == 0)
    xs = (x.reshape(64, 4, 128) / scale[:, :, None]).reshape(64, 512).astype(np.float32)
    assert np.array_equal(codes, e4m3_encode(xs))
    deq = oracle.dequantize_tiles(codes, scale)
    assert np.all(np.abs(deq - x) <= np.abs(x) * 2.0 ** -4 + scale.repeat(128, axis=1) * 2.0 ** -10)
    # amax = 448 * 2^k: both quantisers agree
    y = rng.standard_normal((8, 128)).astype(np.float32)
    y[:, 0] = np.float32(448.0 * 2.0 ** -5)
    y[:, 1:] = np.clip(y[:, 1:], -448.0 * 2.0 ** -5, 448.0 * 2.0 ** -5)
    c1, s1 = oracle.quantize_tiles(y, pow2=True)
    c2, s2 = oracle.quantize_tiles(y)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)
