"""Pins of the oracle's number formats (bfloat16 decode, OCP e4m3fn decode,
encode and per-group quantize) against the OCP table, torch's own dtype
conversions and a brute-force nearest-grid search."""
import json
import os

import numpy as np
import pytest
import torch

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_bf16_decode_all_patterns(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().double().numpy()
    got = orc.bf16_value(bits)
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite], ref[finite])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(np.isinf(got), np.isinf(ref))


def test_e4m3_decode_ocp_table(orc):
    g = json.load(open(os.path.join(GOLD, "e4m3_ocp_values.json")))
    for code, val in g["codes"].items():
        v = orc.e4m3_value(np.array([int(code, 16)], dtype=np.uint8))[0]
        assert v == val and np.signbit(v) == np.signbit(val), code
    for code in g["nan_codes"]:
        assert np.isnan(orc.e4m3_value(np.array([int(code, 16)], dtype=np.uint8))[0])


def test_e4m3_decode_matches_torch(orc):
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = orc.e4m3_value(codes)
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.array_equal(np.isnan(got), np.isnan(ref))


def _grid():
    codes = np.arange(256, dtype=np.uint8)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    keep = (codes < 0x7F)        # non-negative finite codes
    return codes[keep], vals[keep]


def _nearest_even(x):
    """brute force: nearest non-negative grid value, ties to the even code"""
    codes, vals = _grid()
    a = np.abs(x.astype(np.float64))
    out = np.zeros(x.shape, dtype=np.uint8)
    for i, ai in enumerate(a.ravel()):
        if ai > 448.0:
            c = 0x7E
        else:
            dist = np.abs(vals - ai)
            best = np.flatnonzero(dist == dist.min())
            c = codes[best[0]] if len(best) == 1 else [cc for cc in codes[best] if cc % 2 == 0][0]
        out.ravel()[i] = c | (0x80 if np.signbit(x.ravel()[i]) else 0)
    return out


def test_e4m3_encode_brute_force(orc):
    rng = np.random.default_rng(7)
    _, vals = _grid()
    mids = (vals[1:] + vals[:-1]) / 2          # every rounding midpoint (ties)
    xs = np.concatenate([
        vals, mids, np.nextafter(mids.astype(np.float32), np.float32(0)),
        np.nextafter(mids.astype(np.float32), np.float32(1000)),
        rng.uniform(0, 460, 3000), np.exp(rng.uniform(np.log(1e-5), np.log(448), 3000)),
        [448.0, 448.5, 463.9, 464.0, 500.0, 1e30, np.inf, 0.0, 1e-40],
    ]).astype(np.float32)
    xs = np.concatenate([xs, -xs])
    got = orc.e4m3_encode(xs)
    ref = _nearest_even(xs)
    bad = np.flatnonzero(got != ref)
    assert bad.size == 0, (xs[bad[:5]], got[bad[:5]], ref[bad[:5]])


def test_e4m3_encode_matches_torch_in_range(orc):
    rng = np.random.default_rng(11)
    xs = (rng.standard_normal(20000) * rng.choice([1e-3, 0.1, 1, 30, 150], 20000)).astype(np.float32)
    xs = np.clip(xs, -448, 448)
    ref = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = orc.e4m3_encode(xs)
    assert np.array_equal(got, ref)


def test_e4m3_quantize_group(orc):
    rng = np.random.default_rng(3)
    for trial in range(20):
        x = (rng.standard_normal(128) * 10 ** rng.uniform(-3, 2)).astype(np.float32)
        codes, scale = orc.e4m3_quantize_group(x)
        amax = np.max(np.abs(x))
        assert scale == np.float32(amax) / np.float32(448.0)
        # the largest-magnitude element lands on the largest code
        i = int(np.argmax(np.abs(x)))
        assert codes[i] & 0x7F == 0x7E
        # each code is the nearest grid point of x / scale (float32 divide)
        q = (x / np.float32(scale)).astype(np.float32)
        assert np.array_equal(codes, _nearest_even(q))
        # dequantized error within half a grid step (relative 1/16 for normals)
        deq = orc.e4m3_value(codes) * scale
        assert np.all(np.abs(deq - x) <= np.maximum(np.abs(x) / 16 * (1 + 1e-6), scale * 2.0 ** -10) + 1e-30)
    codes, scale = orc.e4m3_quantize_group(np.zeros(128, dtype=np.float32))
    assert scale == 0.0 and not codes.any()
