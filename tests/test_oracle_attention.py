"""Pins of the oracle's scatter (A1), sink+rolling key map (A2) and block
attention (A3): the lossless invariant, closed forms (Q = 0, V = 1, planted
key), key-permutation invariance, and numpy's matmul/softmax in fp64."""
import json
import os

import numpy as np
import pytest
import torch

import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _bits(t):
    return W.as_numpy_bits(t)


def _decode(orc, arr, dtype, scale=None):
    """storage -> float64 by library routines (torch dtype views)"""
    if dtype == orc.F32:
        return arr.astype(np.float64)
    if dtype == orc.BF16:
        return torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16).double().numpy()
    v = torch.from_numpy(arr).view(torch.float8_e4m3fn).double().numpy()
    d = arr.shape[-1]
    s = np.repeat(scale.astype(np.float64), 128, axis=-1).reshape(arr.shape)
    return v * s


def _cache(orc, B, L, Hkv, d, dtype, seed, std=0.3):
    g = torch.Generator().manual_seed(seed)
    src = orc.F32 if dtype == orc.F32 else orc.BF16
    tdt = torch.float32 if src == orc.F32 else torch.bfloat16
    k = (torch.randn(B, L, Hkv, d, generator=g) * std).to(tdt)
    v = (torch.randn(B, L, Hkv, d, generator=g) * std).to(tdt)
    esz = {orc.F32: np.float32, orc.BF16: np.uint16, orc.E4M3: np.uint8}[dtype]
    ck = np.zeros((B, Hkv, L, d), dtype=esz)
    cv = np.zeros_like(ck)
    ks = np.zeros((B, Hkv, L, d // 128), dtype=np.float32) if dtype == orc.E4M3 else None
    vs = np.zeros_like(ks) if ks is not None else None
    pos = np.tile(np.arange(L, dtype=np.int32), (B, 1))
    orc.scatter_kv(ck, cv, ks, vs, dtype, _bits(k), _bits(v), src, pos)
    return ck, cv, ks, vs, k, v


def _numpy_attention(q64, k64, v64, Hq, scale, key_idx=None):
    B, Hkv, L, d = k64.shape
    g = Hq // Hkv
    out = np.zeros(q64.shape)
    lse = np.zeros(q64.shape[:3])
    for b in range(B):
        keys = np.arange(L) if key_idx is None else key_idx[b]
        for h in range(Hq):
            K = k64[b, h // g, keys]
            Vv = v64[b, h // g, keys]
            s = (q64[b, h] @ K.T) * scale
            m = s.max(-1, keepdims=True)
            p = np.exp(s - m)
            z = p.sum(-1, keepdims=True)
            out[b, h] = (p / z) @ Vv
            lse[b, h] = (m + np.log(z))[:, 0]
    return out, lse


# ---- A1 -----------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_scatter_lossless(orc, dtype):
    dt = {"f32": orc.F32, "bf16": orc.BF16}[dtype]
    B, L, H, d, n = 3, 50, 2, 16, 7
    ck, cv, _, _, k_all, v_all = _cache(orc, B, L, H, d, dt, seed=1)
    before_k, before_v = ck.copy(), cv.copy()
    g = torch.Generator().manual_seed(2)
    pos = torch.stack([torch.randperm(L, generator=g)[:n] for _ in range(B)]).int().numpy()
    tdt = torch.float32 if dt == orc.F32 else torch.bfloat16
    kn = torch.randn(B, n, H, d, generator=g).to(tdt)
    vn = torch.randn(B, n, H, d, generator=g).to(tdt)
    orc.scatter_kv(ck, cv, None, None, dt, _bits(kn), _bits(vn), dt, pos)
    # a full recompute would assemble: unchanged rows + the fresh rows
    ref_k, ref_v = before_k.copy(), before_v.copy()
    knb, vnb = _bits(kn), _bits(vn)
    for b in range(B):
        for j in range(n):
            ref_k[b, :, pos[b, j]] = knb[b, j]
            ref_v[b, :, pos[b, j]] = vnb[b, j]
    assert np.array_equal(ck, ref_k) and np.array_equal(cv, ref_v)
    # the cache of the full rows equals the rows in cache layout
    assert np.array_equal(before_k, np.ascontiguousarray(_bits(k_all).transpose(0, 2, 1, 3)))


def test_scatter_e4m3_groups(orc):
    B, L, H, d = 2, 9, 3, 256
    ck, cv, ks, vs, k_all, _ = _cache(orc, B, L, H, d, orc.E4M3, seed=4)
    kf = k_all.float().numpy().transpose(0, 2, 1, 3)       # [B, H, L, d]
    for b in range(B):
        for h in range(H):
            for p in range(L):
                for gi in range(d // 128):
                    x = np.ascontiguousarray(kf[b, h, p, gi * 128:(gi + 1) * 128])
                    codes, s = orc.e4m3_quantize_group(x)
                    assert ks[b, h, p, gi] == s
                    assert np.array_equal(ck[b, h, p, gi * 128:(gi + 1) * 128], codes)
    deq = _decode(orc, ck, orc.E4M3, ks)
    assert np.all(np.abs(deq - kf) <= np.abs(kf) / 16 * (1 + 1e-6) + ks.max() * 2.0 ** -9)


def test_scatter_rejects_bad_positions(orc):
    ck = np.zeros((1, 1, 4, 16), dtype=np.float32)
    with pytest.raises(ValueError):
        orc.scatter_kv(ck, ck.copy(), None, None, orc.F32, np.zeros((1, 1, 1, 16), np.float32),
                       np.zeros((1, 1, 1, 16), np.float32), orc.F32, np.array([[4]], np.int32))
    assert not ck.any()


# ---- A2 -----------------------------------------------------------------------

def test_check_positions(orc):
    """the position check against a set-based count (valid entries minus
    distinct valid entries) on random lists with planted repeats, padding and
    out-of-range entries, and its closed forms"""
    rng = np.random.default_rng(17)
    for trial in range(300):
        B, L, n = int(rng.integers(1, 4)), int(rng.integers(1, 40)), int(rng.integers(0, 30))
        pos = rng.integers(-3, L + 3, (B, n)).astype(np.int32)
        if n and trial % 3 == 0:
            pos[:, -1] = pos[:, 0]                       # a planted repeat
        bad, dup = orc.check_positions(L, pos)
        for b in range(B):
            row = pos[b].tolist()
            valid = [p for p in row if 0 <= p < L]
            assert bad[b] == sum(1 for p in row if p != -1 and not 0 <= p < L), trial
            assert dup[b] == len(valid) - len(set(valid)), trial
    assert [x.tolist() for x in orc.check_positions(8, np.arange(8, dtype=np.int32)[None])] == [[0], [0]]
    assert [x.tolist() for x in orc.check_positions(8, np.full((1, 5), 3, np.int32))] == [[0], [4]]
    assert [x.tolist() for x in orc.check_positions(8, np.full((1, 5), -1, np.int32))] == [[0], [0]]
    assert [x.tolist() for x in orc.check_positions(8, np.array([[8, -2, 7, 7]], np.int32))] == [[2], [1]]


def test_sink_rolling_page_example(orc):
    g = json.load(open(os.path.join(GOLD, "sinks_rolling_example.json")))
    C, S, R = g["total_cache_C"], g["sinks_S"], g["rolling_R"]
    assert C - S == R
    prev_rolling = None
    for end in range(1, 30):
        keys = orc.sink_rolling_keys(S, R, end)
        assert len(keys) <= C
        assert list(keys[:min(S, end)]) == list(range(min(S, end)))      # sinks first, untouched
        rolling = list(keys[min(S, end):])
        assert rolling == list(range(max(S, end - R), end))              # newest R, oldest first
        if end > S:
            assert 1 <= len(rolling) <= R
        if prev_rolling is not None and len(prev_rolling) == R:
            assert rolling[:-1] == prev_rolling[1:]                      # one in, oldest out
        prev_rolling = rolling
    assert g["rolling_length_logged"] == [R - 1, R]


def test_sink_rolling_degenerate_and_long(orc):
    assert list(orc.sink_rolling_keys(4, 100, 50)) == list(range(50))   # R >= end - S: all keys
    keys = orc.sink_rolling_keys(4, 8188, 32768)
    assert len(keys) == 8192
    assert list(keys[:4]) == [0, 1, 2, 3] and keys[4] == 24580 and keys[-1] == 32767
    assert list(orc.sink_rolling_keys(0, 5, 3)) == [0, 1, 2]


# ---- A3 -----------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16", "e4m3"])
def test_attention_vs_numpy(orc, dtype):
    dt = {"f32": orc.F32, "bf16": orc.BF16, "e4m3": orc.E4M3}[dtype]
    d = 128 if dt == orc.E4M3 else 32
    B, L, Hkv, Hq, b = 2, 70, 2, 6, 5
    ck, cv, ks, vs, _, _ = _cache(orc, B, L, Hkv, d, dt, seed=6)
    g = torch.Generator().manual_seed(7)
    qdt = orc.F32 if dt == orc.F32 else orc.BF16
    q = (torch.randn(B, Hq, b, d, generator=g) * 0.5).to(torch.float32 if qdt == orc.F32 else torch.bfloat16)
    qb = _bits(q)
    key_idx = np.stack([np.sort(np.random.default_rng(8 + i).choice(L, 40, replace=False))
                        for i in range(B)]).astype(np.int32)
    for kid in (None, key_idx):
        out, lse = orc.block_attention(ck, cv, ks, vs, dt, qb, qdt, key_idx=kid)
        ref, ref_lse = _numpy_attention(_decode(orc, qb, qdt), _decode(orc, ck, dt, ks),
                                        _decode(orc, cv, dt, vs), Hq, 1 / np.sqrt(d), kid)
        assert np.allclose(out, ref, rtol=1e-11, atol=1e-13)
        assert np.allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


def test_attention_closed_forms(orc):
    B, L, H, d, b = 1, 33, 2, 16, 3
    ck, cv, _, _, _, _ = _cache(orc, B, L, H, d, orc.F32, seed=9)
    kid = np.array([[0, 5, 6, 7, 30, 31, 32]], dtype=np.int32)
    # Q = 0: every key weighs the same, the output is the mean of the values
    q0 = np.zeros((B, H, b, d), dtype=np.float32)
    out, lse = orc.block_attention(ck, cv, None, None, orc.F32, q0, orc.F32, key_idx=kid)
    for h in range(H):
        mean_v = cv[0, h, kid[0]].astype(np.float64).mean(0)
        assert np.allclose(out[0, h], mean_v[None], rtol=0, atol=1e-15)
    assert np.allclose(lse, np.log(7.0), atol=1e-15)
    # V = 1: the weights of each row sum to one
    ones = np.ones_like(cv)
    rng = np.random.default_rng(10)
    q = rng.standard_normal((B, H, b, d)).astype(np.float32)
    out, _ = orc.block_attention(ck, ones, None, None, orc.F32, q, orc.F32)
    assert np.allclose(out, 1.0, rtol=0, atol=1e-14)
    # a planted key aligned with the query takes all the weight
    ck2 = ck.copy()
    ck2[0, 1, 17] = q[0, 1, 2] * 200.0
    out, _ = orc.block_attention(ck2, cv, None, None, orc.F32, q, orc.F32)
    assert np.allclose(out[0, 1, 2], cv[0, 1, 17], rtol=0, atol=1e-12)


def test_attention_key_permutation_and_scale(orc):
    B, L, H, d, b = 2, 40, 1, 16, 4
    ck, cv, _, _, _, _ = _cache(orc, B, L, H, d, orc.F32, seed=11)
    q = np.random.default_rng(12).standard_normal((B, H, b, d)).astype(np.float32)
    kid = np.tile(np.arange(L, dtype=np.int32), (B, 1))
    perm = np.stack([np.random.default_rng(13 + i).permutation(L) for i in range(B)]).astype(np.int32)
    a, la = orc.block_attention(ck, cv, None, None, orc.F32, q, orc.F32)
    b1, lb = orc.block_attention(ck, cv, None, None, orc.F32, q, orc.F32, key_idx=kid)
    c, lc = orc.block_attention(ck, cv, None, None, orc.F32, q, orc.F32, key_idx=perm)
    assert np.array_equal(a, b1) and np.array_equal(la, lb)
    assert np.allclose(a, c, rtol=1e-13, atol=1e-15) and np.allclose(la, lc, rtol=1e-14)
    e, le = orc.block_attention(ck, cv, None, None, orc.F32, q, orc.F32, scale=0.25)
    assert np.array_equal(e, a) and np.array_equal(le, la)      # 1/sqrt(16) explicitly
    f, _ = orc.block_attention(ck, cv, None, None, orc.F32, q, orc.F32, scale=0.5)
    assert not np.allclose(f, a)


def test_attention_lossless_after_scatter(orc):
    """attention over the cache after scattering fresh rows equals attention
    over freshly assembled K/V (what a full recompute would see)"""
    B, L, H, d, n = 2, 48, 3, 32, 8
    ck, cv, _, _, k_all, v_all = _cache(orc, B, L, H, d, orc.BF16, seed=14)
    g = torch.Generator().manual_seed(15)
    pos = np.tile(np.arange(16, 16 + n, dtype=np.int32), (B, 1))
    kn = (torch.randn(B, n, H, d, generator=g) * 0.3).bfloat16()
    vn = (torch.randn(B, n, H, d, generator=g) * 0.3).bfloat16()
    orc.scatter_kv(ck, cv, None, None, orc.BF16, _bits(kn), _bits(vn), orc.BF16, pos)
    fk, fv = k_all.clone(), v_all.clone()
    fk[:, 16:16 + n] = kn
    fv[:, 16:16 + n] = vn
    full_k = np.ascontiguousarray(_bits(fk).transpose(0, 2, 1, 3))
    full_v = np.ascontiguousarray(_bits(fv).transpose(0, 2, 1, 3))
    q = _bits((torch.randn(B, H, n, d, generator=g) * 0.3).bfloat16())
    a, la = orc.block_attention(ck, cv, None, None, orc.BF16, q, orc.BF16)
    b1, lb = orc.block_attention(full_k, full_v, None, None, orc.BF16, q, orc.BF16)
    assert np.array_equal(a, b1) and np.array_equal(la, lb)


def test_attention_head_subset(orc):
    B, L, Hkv, Hq, d, b = 2, 20, 2, 4, 16, 3
    ck, cv, _, _, _, _ = _cache(orc, B, L, Hkv, d, orc.F32, seed=16)
    q = np.random.default_rng(17).standard_normal((B, Hq, b, d)).astype(np.float32)
    full, lf = orc.block_attention(ck, cv, None, None, orc.F32, q, orc.F32)
    heads = np.array([[1, 3], [0, 0], [1, 2]], dtype=np.int32)
    sub, ls = orc.block_attention(ck, cv, None, None, orc.F32, q, orc.F32, heads=heads)
    for i, (bb, hh) in enumerate(heads):
        assert np.array_equal(sub[i], full[bb, hh]) and np.array_equal(ls[i], lf[bb, hh])


def test_padding_entries(orc):
    """-1 in a position list or key map is padding: it is skipped"""
    B, L, H, d = 2, 30, 2, 16
    ck, cv, _, _, _, _ = _cache(orc, B, L, H, d, orc.F32, seed=18)
    q = np.random.default_rng(19).standard_normal((B, H, 3, d)).astype(np.float32)
    kid = np.array([[3, 4, 5, 9, 10], [0, 1, 2, 28, 29]], dtype=np.int32)
    padded = np.array([[3, -1, 4, 5, 9, -1, 10], [-1, 0, 1, 2, 28, 29, -1]], dtype=np.int32)
    a, la = orc.block_attention(ck, cv, None, None, orc.F32, q, orc.F32, key_idx=kid)
    b1, lb = orc.block_attention(ck, cv, None, None, orc.F32, q, orc.F32, key_idx=padded)
    assert np.allclose(a, b1, rtol=1e-14, atol=1e-15) and np.allclose(la, lb, rtol=1e-14)
    empty = np.full((B, 4), -1, dtype=np.int32)
    e, le = orc.block_attention(ck, cv, None, None, orc.F32, q, orc.F32, key_idx=empty)
    assert np.all(e == 0) and np.all(np.isneginf(le))
    # scatter: a -1 row writes nothing
    before = ck.copy()
    kn = np.ones((B, 2, H, d), np.float32)
    orc.scatter_kv(ck, cv, None, None, orc.F32, kn, kn, orc.F32, np.array([[-1, 7], [-1, -1]], np.int32))
    changed = np.argwhere(np.any(ck != before, axis=-1))
    assert changed.tolist() == [[0, 0, 7], [0, 1, 7]]
