"""Pins of the oracle's FACache merge (N1): the memoized state of the
unchanged keys, continued over the changed block keys, equals attention over
all keys (the lossless claim); an empty memo reduces to plain attention; an
empty key list returns the memo; merges chain (associativity); a two-key
closed form; and the unchanged/changed key maps partition the positions."""
import numpy as np
import pytest
import torch

import workloads as W

from test_oracle_attention import _cache


def _bits(t):
    return W.as_numpy_bits(t)


def _queries(orc, B, Hq, n, d, qdt, seed, std=0.5):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, Hq, n, d, generator=g) * std
    return _bits(q.to(torch.float32 if qdt == orc.F32 else torch.bfloat16))


def _memo(orc, ck, cv, ks, vs, dt, q, qdt, keys):
    """the fill: attention of the queries over the unchanged keys, stored as
    float32 (O = O~/l, lse = m + ln l)"""
    o, lse = orc.block_attention(ck, cv, ks, vs, dt, q, qdt, key_idx=keys)
    return o.astype(np.float32), lse.astype(np.float32)


CASES = [
    # dtype, d, B, L, Hkv, Hq, b
    ("f32", 16, 1, 64, 4, 4, 8),
    ("bf16", 64, 2, 70, 2, 6, 16),
    ("e4m3", 128, 2, 48, 1, 2, 8),
]


@pytest.mark.parametrize("dtype,d,B,L,Hkv,Hq,b", CASES)
def test_facache_lossless(orc, dtype, d, B, L, Hkv, Hq, b):
    """memo over the unchanged keys + the block keys == all L keys"""
    dt = {"f32": orc.F32, "bf16": orc.BF16, "e4m3": orc.E4M3}[dtype]
    qdt = orc.F32 if dt == orc.F32 else orc.BF16
    ck, cv, ks, vs, _, _ = _cache(orc, B, L, Hkv, d, dt, seed=21)
    rng = np.random.default_rng(22)
    start = rng.integers(0, L - b + 1, size=B)
    un, blk = orc.facache_key_maps(L, b, start)
    q = _queries(orc, B, Hq, L - b, d, qdt, seed=23)      # the unchanged queries
    mo, ml = _memo(orc, ck, cv, ks, vs, dt, q, qdt, un)
    out, lse = orc.facache_merge(ck, cv, ks, vs, dt, q, qdt, mo, ml, key_idx=blk)
    ref, ref_lse = orc.block_attention(ck, cv, ks, vs, dt, q, qdt)
    # the memo is float32: relative 2^-24 on O, absolute |lse| 2^-24 on lse
    assert np.abs(out - ref).max() <= 1e-6 * max(1.0, np.abs(ref).max())
    assert np.abs(lse - ref_lse).max() <= 1e-6 * max(1.0, np.abs(ref_lse).max())
    # a wrong merge (memo dropped, or the block keys counted twice) is far off
    dropped, _ = orc.block_attention(ck, cv, ks, vs, dt, q, qdt, key_idx=blk)
    assert np.abs(dropped - ref).max() > 1e-3


def test_facache_padding_in_block_keys(orc):
    B, L, H, d, b = 2, 40, 2, 16, 6
    ck, cv, _, _, _, _ = _cache(orc, B, L, H, d, orc.F32, seed=24)
    un, blk = orc.facache_key_maps(L, b, [3, 30])
    q = _queries(orc, B, H, L - b, d, orc.F32, seed=25)
    mo, ml = _memo(orc, ck, cv, None, None, orc.F32, q, orc.F32, un)
    padded = np.concatenate([blk[:, :2], -np.ones((B, 3), np.int32), blk[:, 2:]], axis=1)
    a, la = orc.facache_merge(ck, cv, None, None, orc.F32, q, orc.F32, mo, ml, key_idx=blk)
    c, lc = orc.facache_merge(ck, cv, None, None, orc.F32, q, orc.F32, mo, ml, key_idx=padded)
    assert np.allclose(a, c, rtol=0, atol=1e-15) and np.allclose(la, lc, rtol=0, atol=1e-15)


def test_facache_empty_memo_is_attention(orc):
    B, L, H, d, b = 1, 33, 2, 16, 7
    ck, cv, _, _, _, _ = _cache(orc, B, L, H, d, orc.F32, seed=26)
    _, blk = orc.facache_key_maps(L, b, [11])
    q = _queries(orc, B, H, 5, d, orc.F32, seed=27)
    mo = np.full((B, H, 5, d), np.nan, np.float32)          # ignored with lse = -inf
    ml = np.full((B, H, 5), -np.inf, np.float32)
    out, lse = orc.facache_merge(ck, cv, None, None, orc.F32, q, orc.F32, mo, ml, key_idx=blk)
    ref, ref_lse = orc.block_attention(ck, cv, None, None, orc.F32, q, orc.F32, key_idx=blk)
    assert np.allclose(out, ref, rtol=1e-13, atol=1e-15)
    assert np.allclose(lse, ref_lse, rtol=1e-13, atol=1e-15)
    # and with no keys either: zero output, lse = -inf
    none = -np.ones((B, 3), np.int32)
    out, lse = orc.facache_merge(ck, cv, None, None, orc.F32, q, orc.F32, mo, ml, key_idx=none)
    assert not out.any() and np.all(lse == -np.inf)


def test_facache_no_changed_keys_returns_memo(orc):
    B, L, H, d = 2, 20, 1, 16
    ck, cv, _, _, _, _ = _cache(orc, B, L, H, d, orc.F32, seed=28)
    rng = np.random.default_rng(29)
    mo = rng.standard_normal((B, H, 4, d)).astype(np.float32)
    ml = rng.standard_normal((B, H, 4)).astype(np.float32) * 5
    q = _queries(orc, B, H, 4, d, orc.F32, seed=30)
    out, lse = orc.facache_merge(ck, cv, None, None, orc.F32, q, orc.F32, mo, ml,
                                 key_idx=-np.ones((B, 4), np.int32))
    assert np.array_equal(out, mo.astype(np.float64)) and np.array_equal(lse, ml.astype(np.float64))


def test_facache_merges_chain(orc):
    """three disjoint key sets folded in one after another == all at once"""
    B, L, Hkv, Hq, d = 1, 60, 2, 4, 64
    ck, cv, _, _, _, _ = _cache(orc, B, L, Hkv, d, orc.BF16, seed=31)
    q = _queries(orc, B, Hq, 9, d, orc.BF16, seed=32)
    perm = np.random.default_rng(33).permutation(L).astype(np.int32)
    a, b_, c = np.sort(perm[:25]), np.sort(perm[25:47]), np.sort(perm[47:])
    mo, ml = _memo(orc, ck, cv, None, None, orc.BF16, q, orc.BF16, a[None])
    o2, l2 = orc.facache_merge(ck, cv, None, None, orc.BF16, q, orc.BF16, mo, ml, key_idx=b_[None])
    o3, l3 = orc.facache_merge(ck, cv, None, None, orc.BF16, q, orc.BF16, o2.astype(np.float32),
                               l2.astype(np.float32), key_idx=c[None])
    ref, ref_lse = orc.block_attention(ck, cv, None, None, orc.BF16, q, orc.BF16)
    assert np.abs(o3 - ref).max() <= 2e-6 and np.abs(l3 - ref_lse).max() <= 2e-6
    # the order of the sets does not matter either
    mo, ml = _memo(orc, ck, cv, None, None, orc.BF16, q, orc.BF16, c[None])
    o2, l2 = orc.facache_merge(ck, cv, None, None, orc.BF16, q, orc.BF16, mo, ml,
                               key_idx=np.concatenate([b_, a])[None])
    assert np.abs(o2 - ref).max() <= 2e-6 and np.abs(l2 - ref_lse).max() <= 2e-6


def test_facache_two_key_closed_form(orc):
    """one memoized key (score s1, value v1) plus one block key (s2, v2):
    out = sigmoid(s1 - s2) v1 + sigmoid(s2 - s1) v2, lse = logaddexp(s1, s2)"""
    d = 16
    ck = np.zeros((1, 1, 2, d), np.float32)
    cv = np.zeros((1, 1, 2, d), np.float32)
    ck[0, 0, 0, 0], ck[0, 0, 1, 0] = 1.5, -0.5
    cv[0, 0, 0, :], cv[0, 0, 1, :] = 2.0, -1.0
    q = np.zeros((1, 1, 1, d), np.float32)
    q[0, 0, 0, 0] = 4.0                                   # s = 4 k0 / 4 with scale 1/sqrt(16)
    s1, s2 = 1.5, -0.5
    mo, ml = _memo(orc, ck, cv, None, None, orc.F32, q, orc.F32, np.array([[0]], np.int32))
    assert np.allclose(mo, 2.0) and ml[0, 0, 0] == np.float32(s1)
    out, lse = orc.facache_merge(ck, cv, None, None, orc.F32, q, orc.F32, mo, ml,
                                 key_idx=np.array([[1]], np.int32))
    w1 = 1.0 / (1.0 + np.exp(s2 - s1))
    assert np.allclose(out, w1 * 2.0 + (1 - w1) * -1.0, rtol=0, atol=1e-14)
    assert np.isclose(lse[0, 0, 0], np.logaddexp(s1, s2), rtol=0, atol=1e-14)


def test_facache_key_maps_partition(orc):
    L, b = 50, 8
    for o in (0, 17, 42):
        un, blk = orc.facache_key_maps(L, b, [o])
        assert list(blk[0]) == list(range(o, o + b))
        assert sorted(list(un[0]) + list(blk[0])) == list(range(L))
        assert not set(un[0]) & set(blk[0])
    with pytest.raises(ValueError):
        orc.facache_key_maps(L, b, [43])


def test_facache_head_subset(orc):
    B, L, Hkv, Hq, d, b = 2, 30, 1, 3, 16, 4
    ck, cv, _, _, _, _ = _cache(orc, B, L, Hkv, d, orc.F32, seed=34)
    un, blk = orc.facache_key_maps(L, b, [0, 26])
    q = _queries(orc, B, Hq, L - b, d, orc.F32, seed=35)
    mo, ml = _memo(orc, ck, cv, None, None, orc.F32, q, orc.F32, un)
    full, lf = orc.facache_merge(ck, cv, None, None, orc.F32, q, orc.F32, mo, ml, key_idx=blk)
    heads = np.array([[1, 2], [0, 0]], np.int32)
    part, lp = orc.facache_merge(ck, cv, None, None, orc.F32, q, orc.F32, mo, ml, key_idx=blk,
                                 heads=heads)
    assert np.array_equal(part[0], full[1, 2]) and np.array_equal(part[1], full[0, 0])
    assert np.array_equal(lp[0], lf[1, 2]) and np.array_equal(lp[1], lf[0, 0])
