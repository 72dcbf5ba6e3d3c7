"""Pins of the oracle's vocab statistics: closed forms (uniform, one-hot,
two-way tie), a 50-digit mpmath evaluation, and torch/scipy library routines
(log_softmax, scipy.stats.entropy) on random rows."""
import math

import mpmath
import numpy as np
import pytest
import scipy.special
import scipy.stats
import torch

import workloads as W


def _bf16_bits(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("V", [2, 512, 50257, 126464])
def test_uniform_row(orc, V):
    x = np.full((1, V), 0.37, dtype=np.float32)
    am, mp, en = orc.vocab_stats(x, orc.F32)
    assert am[0] == 0
    assert mp[0] == 1.0 / V                 # the sum of V ones is exact
    # a sequential fp64 sum of V terms carries at most V unit roundoffs
    assert abs(en[0] - math.log(V)) <= V * 2.0 ** -52 * math.log(V)


def test_one_hot_and_gap(orc):
    V = 1000
    x = np.full((3, V), -np.inf, dtype=np.float32)
    x[0, 417] = 3.0
    x[1, :] = -2000.0
    x[1, 9] = 0.0                       # gap of 2000: every other p underflows
    x[2, 0] = 5.0
    am, mp, en = orc.vocab_stats(x, orc.F32)
    assert list(am) == [417, 9, 0]
    assert np.all(mp == 1.0)
    assert np.all(en == 0.0)


def test_two_way_tie(orc):
    V = 300
    x = np.full((2, V), -np.inf, dtype=np.float32)
    x[0, [250, 17]] = 1.5
    x[1, [5, 6]] = -7.25
    am, mp, en = orc.vocab_stats(x, orc.F32)
    assert list(am) == [17, 5]
    assert np.all(mp == 0.5)
    assert np.allclose(en, math.log(2.0), rtol=0, atol=1e-15)


def test_ties_lowest_index_among_finite(orc):
    rng = np.random.default_rng(5)
    x = rng.standard_normal((50, 777)).astype(np.float32)
    for r in range(50):
        i, j = sorted(rng.choice(777, 2, replace=False))
        x[r, i] = x[r, j] = 9.0
        am, _, _ = orc.vocab_stats(x[r:r + 1], orc.F32)
        assert am[0] == i


def test_mpmath_50_digits(orc):
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((3, 64)) * 3).astype(np.float32)
    am, mp, en = orc.vocab_stats(x, orc.F32)
    mpmath.mp.dps = 50
    for r in range(3):
        xs = [mpmath.mpf(float(v)) for v in x[r]]
        z = mpmath.fsum(mpmath.exp(v) for v in xs)
        ps = [mpmath.exp(v) / z for v in xs]
        H = -mpmath.fsum(p * mpmath.log(p) for p in ps)
        assert abs(float(H) - en[r]) <= 1e-13
        assert abs(float(max(ps)) - mp[r]) <= 1e-15
        assert am[r] == int(np.argmax(x[r]))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_library_cross_check(orc, dtype):
    rng = np.random.default_rng(13)
    V = 5003
    x = (rng.standard_normal((40, V)) * rng.uniform(0.5, 4, (40, 1))).astype(np.float32)
    x[::3, rng.integers(0, V, 14)] += 8.0
    if dtype == "bf16":
        bits = _bf16_bits(x)
        xv = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double()
        am, mp, en = orc.vocab_stats(bits, orc.BF16)
    else:
        xv = torch.from_numpy(x).double()
        am, mp, en = orc.vocab_stats(x, orc.F32)
    lsm = torch.log_softmax(xv, dim=-1)
    p = lsm.exp()
    ref_H = -(p * lsm).sum(-1).numpy()
    assert np.allclose(en, ref_H, rtol=1e-12, atol=1e-12)
    assert np.allclose(mp, p.max(-1).values.numpy(), rtol=1e-12, atol=0)
    assert np.array_equal(am, torch.argmax(xv, dim=-1).numpy())
    sp = scipy.stats.entropy(scipy.special.softmax(xv.numpy(), axis=-1), axis=-1)
    assert np.allclose(en, sp, rtol=1e-11, atol=1e-12)


def test_row_stride_padding_ignored(orc):
    rng = np.random.default_rng(17)
    V, S = 1001, 1008
    x = rng.standard_normal((6, S)).astype(np.float32)
    x[:, V:] = 1e30                      # padding beyond V must not be read
    am, mp, en = orc.vocab_stats(x, orc.F32, V=V)
    am2, mp2, en2 = orc.vocab_stats(np.ascontiguousarray(x[:, :V]), orc.F32)
    assert np.array_equal(am, am2) and np.array_equal(mp, mp2) and np.array_equal(en, en2)
    rows = np.array([4, 0, 4])
    am3, mp3, en3 = orc.vocab_stats(x, orc.F32, V=V, rows=rows)
    assert np.array_equal(am3, am2[rows]) and np.array_equal(en3, en2[rows])


def test_workload_generator_ties_are_exact(orc):
    import dataclasses
    cfg = dataclasses.replace(W.CONFIGS["vocab"], V=4096, V_stride=4096)
    x = W.logits(cfg, rows=2048)                       # the recipe at a small size
    bits = W.as_numpy_bits(x)
    am, mp, en = orc.vocab_stats(bits, orc.BF16, V=4096)
    # rows whose two largest logits are equal must report the lower index
    xv = x.float().numpy()
    top2 = np.sort(xv, axis=1)[:, -2:]
    tie_rows = np.flatnonzero(top2[:, 0] == top2[:, 1])
    assert tie_rows.size > 0
    for r in tie_rows:
        assert am[r] == np.flatnonzero(xv[r] == xv[r].max())[0]
