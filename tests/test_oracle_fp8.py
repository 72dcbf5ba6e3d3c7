"""Pins of the oracle's per-group FP8 for the FFN (N2): the power-of-two
group exponent against brute force, the group codes against torch's
float8_e4m3fn rounding, the row and block layouts, the GEMM against numpy's
fp64 matmul of values decoded by torch, add & RMS norm against numpy, and
SiLU against closed forms and torch."""
import math

import numpy as np
import pytest
import torch

import workloads as W


def _e_brute(amax):
    if amax == 0:
        return -127
    for e in range(-127, 200):
        if amax <= 448.0 * 2.0 ** e:
            return e
    raise AssertionError


def test_e8m0_exponent_brute_force(orc):
    rng = np.random.default_rng(1)
    vals = [448.0, 449.0, 224.0, 224.0000001, 223.99, 1.0, 1.75, 1.7500001, 0.875, 3e38, 1e-30, 1e-45,
            np.nextafter(448.0, 1e9), np.nextafter(448.0, 0)]
    vals += list(np.exp(rng.uniform(-80, 80, 400)))
    vals += [448.0 * 2.0 ** k for k in range(-130, 120, 7)]
    for a in vals:
        assert orc.e8m0_exponent(a) == max(-127, _e_brute(a)), a
    assert orc.e8m0_exponent(0.0) == -127
    assert orc.e8m0_value(127) == 1.0 and orc.e8m0_value(130) == 8.0 and orc.e8m0_value(0) == 2.0 ** -127


def _torch_e4m3(x):
    """RNE to float8_e4m3fn by torch's cast (inputs within +-448)"""
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _decode(codes):
    return torch.from_numpy(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def test_quantize_group_pow2(orc):
    rng = np.random.default_rng(2)
    for trial in range(300):
        scale = math.exp(rng.uniform(-30, 30))
        x = rng.standard_normal(128) * scale
        if trial % 7 == 0:
            x[rng.integers(128)] *= 50                     # an outlier sets the scale
        x = x.astype(np.float32).astype(np.float64)        # so that x / 2^e is exact in float32
        codes, sc = orc.fp8_quantize_pow2(x)
        e = sc - 127
        assert e == orc.e8m0_exponent(np.abs(x).max())
        q = np.ldexp(x, -e)
        assert np.abs(q).max() <= 448.0
        # torch's float8 cast of x / 2^e (exact in float32 here) gives the same codes
        assert np.array_equal(codes, _torch_e4m3(q)), trial
        # the group max lands in the top binade of the grid: [224, 448]
        assert 224.0 <= np.abs(_decode(codes)).max() <= 448.0
    codes, sc = orc.fp8_quantize_pow2(np.zeros(128))
    assert sc == 0 and not codes.any()


def test_quant_rows_layout(orc):
    rng = np.random.default_rng(3)
    M, K = 5, 384
    x = (rng.standard_normal((M, K)) * 3).astype(np.float32)
    x[2, 128:256] = 0.0
    codes, scales = orc.fp8_quant_rows(x, orc.F32)
    assert scales.shape == (3, 5)
    for m in range(M):
        for g in range(3):
            c, s = orc.fp8_quantize_pow2(x[m, g * 128:(g + 1) * 128].astype(np.float64))
            assert np.array_equal(codes[m, g * 128:(g + 1) * 128], c) and scales[g, m] == s
    assert scales[1, 2] == 0 and not codes[2, 128:256].any()
    # bf16 bits read as their values, float64 rows as themselves
    xb = torch.from_numpy(x).bfloat16()
    cb, sb = orc.fp8_quant_rows(W.as_numpy_bits(xb), orc.BF16)
    cd, sd = orc.fp8_quant_rows(xb.double().numpy(), orc.F64)
    assert np.array_equal(cb, cd) and np.array_equal(sb, sd)


def test_quant_weight_blocks(orc):
    rng = np.random.default_rng(4)
    N, K = 256, 384
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    w[128:, 256:] *= 1000.0
    codes, scales = orc.fp8_quant_weight(w, orc.F32)
    assert scales.shape == (2, 3)
    for bn in range(2):
        for bk in range(3):
            blk = w[bn * 128:(bn + 1) * 128, bk * 128:(bk + 1) * 128].astype(np.float64)
            e = orc.e8m0_exponent(np.abs(blk).max())
            assert scales[bn, bk] == e + 127
            assert np.array_equal(codes[bn * 128:(bn + 1) * 128, bk * 128:(bk + 1) * 128],
                                  _torch_e4m3(np.ldexp(blk, -e)))
    assert scales[1, 2] > scales[0, 0] + 8


def test_fp8_gemm_vs_numpy(orc):
    rng = np.random.default_rng(5)
    M, N, K = 37, 256, 512
    a = (rng.standard_normal((M, K)) * 2).astype(np.float32)
    b = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    ca, sa = orc.fp8_quant_rows(a, orc.F32)
    cb, sb = orc.fp8_quant_weight(b, orc.F32)
    ad = _decode(ca) * np.repeat(2.0 ** (sa.T.astype(np.float64) - 127), 128, axis=1)
    bd = _decode(cb) * np.kron(2.0 ** (sb.astype(np.float64) - 127), np.ones((128, 128)))
    ref = ad @ bd.T
    c = orc.fp8_gemm(ca, sa, cb, sb)
    assert np.allclose(c, ref, rtol=1e-12, atol=1e-12)
    # the quantised product approximates the float product within the fp8 steps
    exact = a.astype(np.float64) @ b.astype(np.float64).T
    assert np.abs(c - exact).max() <= 0.06 * np.abs(exact).max()
    rows = np.array([36, 0, 17])
    assert np.array_equal(orc.fp8_gemm(ca, sa, cb, sb, rows=rows), c[rows])
    # a one-hot A row picks one dequantised row of B
    ca1 = np.zeros_like(ca)
    ca1[3, 200] = 0x38                                     # 1.0
    sa1 = np.full_like(sa, 127)
    c1 = orc.fp8_gemm(ca1, sa1, cb, sb)
    assert np.array_equal(c1[3], bd[:, 200]) and not np.delete(c1, 3, axis=0).any()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_addnorm_vs_numpy(orc, dtype):
    rng = np.random.default_rng(6)
    M, K = 9, 512
    x = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32))
    r = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32))
    g = torch.from_numpy((1 + 0.1 * rng.standard_normal(K)).astype(np.float32))
    dt = orc.F32 if dtype == "f32" else orc.BF16
    if dtype == "bf16":
        x, r, g = x.bfloat16(), r.bfloat16(), g.bfloat16()
    res_out, y = orc.addnorm(W.as_numpy_bits(x), W.as_numpy_bits(r), W.as_numpy_bits(g), 1e-6, dt)
    s = (x.float() + r.float()).to(x.dtype)                # torch's add in fp32, rounded to the stream dtype
    assert np.array_equal(res_out, W.as_numpy_bits(s))
    sd = s.double().numpy()
    ref = sd / np.sqrt((sd ** 2).mean(axis=1, keepdims=True) + 1e-6) * g.double().numpy()
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)
    # a constant row normalises to gamma * sign (up to eps)
    c = np.full((1, K), 3.0, np.float32)
    _, yc = orc.addnorm(c, None, np.ones(K, np.float32), 0.0, orc.F32)
    assert np.allclose(yc, 1.0, rtol=0, atol=1e-15)


def test_silu_and_swiglu(orc):
    assert orc.silu(0.0) == 0.0
    assert orc.silu(40.0) == pytest.approx(40.0, rel=1e-15)
    assert abs(orc.silu(-40.0)) < 1e-15
    assert orc.silu(1.0) == pytest.approx(1.0 / (1.0 + math.e ** -1.0), rel=1e-15)
    rng = np.random.default_rng(7)
    gg, uu = rng.standard_normal(1000) * 4, rng.standard_normal(1000)
    y = orc.swiglu(gg, uu)
    ref = torch.nn.functional.silu(torch.from_numpy(gg)).numpy() * uu
    assert np.allclose(y, ref, rtol=1e-13, atol=1e-15)
