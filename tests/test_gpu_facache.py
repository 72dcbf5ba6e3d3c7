"""GPU parity of the FACache calls against the fp64 oracle.

dllm_facache_maps is compared bit for bit.  dllm_facache_merge is held to
the attention bars (max-abs 2e-2 bf16 / 6e-2 e4m3, normalised 1e-2, lse
1e-3; the float32 path 1e-4 normalised) on the same seeded memo, queries and
cache bytes as the oracle, over ragged query counts, GQA, e4m3, padding in
the key list, empty memo rows, key splits and sharp queries; and the
lossless property: the memo filled on the GPU over the unchanged keys, then
merged with the block keys, matches the oracle's attention over all L keys.
"""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import attn_errors, bits, cache_np, need_gpu, new_cache, say

pytestmark = pytest.mark.gpu

ABS = {W.F32: 2e-2, W.BF16: 2e-2, W.E4M3: 6e-2}
NORM = {W.F32: 1e-4, W.BF16: 1e-2, W.E4M3: 1e-2}


def _fill(D, B, Hkv, L, d, dtype, seed, std):
    cache = new_cache(D, B, Hkv, L, d, dtype)
    g = torch.Generator().manual_seed(seed)
    src = torch.float32 if dtype == W.F32 else torch.bfloat16
    k = (torch.randn((B, L, Hkv, d), generator=g) * std).to(src).cuda()
    v = (torch.randn((B, L, Hkv, d), generator=g) * std).to(src).cuda()
    pos = torch.arange(L, dtype=torch.int32, device="cuda").repeat(B, 1)
    D.dllm_scatter_kv(cache, k, v, pos)
    return cache


def _compare(cache, out, lse, ref, ref_lse, label):
    e_abs, e_norm = attn_errors(out, ref)
    assert e_abs <= ABS[cache.dtype], (label, e_abs)
    assert e_norm <= NORM[cache.dtype], (label, e_norm, e_abs)
    l_got = lse.cpu().numpy()
    assert np.array_equal(np.isneginf(l_got), np.isneginf(ref_lse)), label
    fin = np.isfinite(ref_lse)
    assert np.all(np.abs(l_got[fin] - ref_lse[fin]) <= 1e-3), (label, np.abs(l_got[fin] - ref_lse[fin]).max())


def _merge_check(orc, D, cache, q, memo_o, memo_lse, key_idx, label, heads=None, out_dtype=None):
    B, Hq, n_q, d = q.shape
    say("facache merge", label, "B", B, "Hq", Hq, "n_q", n_q, "d", d, "L", cache.desc.L,
        "n_keys", None if key_idx is None else key_idx.shape[1],
        "ws", D.dllm_facache_merge_workspace(cache, W.F32 if q.dtype == torch.float32 else W.BF16,
                                             Hq, n_q, key_idx.shape[1] if key_idx is not None else cache.desc.L))
    lse = torch.empty((B, Hq, n_q), dtype=torch.float32, device="cuda")
    out = D.dllm_facache_merge(cache, q, memo_o, memo_lse, key_idx=key_idx, lse=lse, out_dtype=out_dtype)
    torch.cuda.synchronize()
    ck, cv, ks, vs = cache_np(cache)
    qdt = W.F32 if q.dtype == torch.float32 else W.BF16
    kid = key_idx.cpu().numpy() if key_idx is not None else None
    mo, ml = memo_o.cpu().numpy(), memo_lse.cpu().numpy()
    if heads is not None:
        ref, ref_lse = orc.facache_merge(ck, cv, ks, vs, cache.dtype, bits(q), qdt, mo, ml, key_idx=kid,
                                         heads=heads)
        out = torch.stack([out[b_, h_] for b_, h_ in heads])
        lse = torch.stack([lse[b_, h_] for b_, h_ in heads])
    else:
        ref, ref_lse = orc.facache_merge(ck, cv, ks, vs, cache.dtype, bits(q), qdt, mo, ml, key_idx=kid)
    _compare(cache, out, lse, ref, ref_lse, label)
    return out


def test_facache_maps_gpu(orc):
    D = need_gpu()
    L, b = 700, 32
    starts = np.array([0, 13, 334, 668, 5], dtype=np.int32)
    say("facache maps", "L", L, "b", b)
    un, blk = D.dllm_facache_maps(L, b, torch.from_numpy(starts).cuda())
    torch.cuda.synchronize()
    ru, rb = orc.facache_key_maps(L, b, starts)
    assert np.array_equal(un.cpu().numpy(), ru) and np.array_equal(blk.cpu().numpy(), rb)
    # starts outside [0, L - b] are clamped
    un, blk = D.dllm_facache_maps(L, b, torch.tensor([-4, 900], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    ru, rb = orc.facache_key_maps(L, b, [0, L - b])
    assert np.array_equal(un.cpu().numpy(), ru) and np.array_equal(blk.cpu().numpy(), rb)


CASES = [
    # label, dtype, d, B, Hkv, Hq, L, b
    ("f32 d16", W.F32, 16, 1, 4, 4, 64, 8),
    ("bf16 d64 gqa ragged", W.BF16, 64, 2, 2, 6, 300, 32),
    ("bf16 d128", W.BF16, 128, 2, 2, 2, 200, 32),
    ("bf16 d128 few rows", W.BF16, 128, 1, 1, 1, 40, 35),
    ("e4m3 d128 gqa", W.E4M3, 128, 2, 2, 8, 700, 64),
]


@pytest.mark.parametrize("label,dtype,d,B,Hkv,Hq,L,b", CASES)
def test_facache_merge_parity(orc, label, dtype, d, B, Hkv, Hq, L, b):
    D = need_gpu()
    std = 1 / np.sqrt(d)
    cache = _fill(D, B, Hkv, L, d, dtype, seed=L + d, std=std)
    rng = np.random.default_rng(L)
    starts = torch.from_numpy(rng.integers(0, L - b + 1, size=B).astype(np.int32)).cuda()
    un, blk = D.dllm_facache_maps(L, b, starts)
    n_q = L - b
    qdt = torch.float32 if dtype == W.F32 else torch.bfloat16
    g = torch.Generator().manual_seed(b + Hq)
    q = (torch.randn((B, Hq, n_q, d), generator=g) * std).to(qdt).cuda()
    mo, ml = W.memo_state(B, Hq, n_q, d, seed=L + 1, o_std=std, lse_mean=np.log(n_q),
                          empty_frac=0.05, device="cuda")
    _merge_check(orc, D, cache, q, mo, ml, blk, label)
    # sharp queries: block scores far above the memo's lse (the memo rescaled away)
    _merge_check(orc, D, cache, q, mo, ml - 30.0, blk, label + " memo low")
    _merge_check(orc, D, cache, (q.float() * 12 / std).to(qdt), mo, ml, blk, label + " sharp")
    # a key list with padding
    kid = blk.clone()
    kid[:, ::5] = -1
    _merge_check(orc, D, cache, q, mo, ml, kid, label + " padded keys", out_dtype=torch.float32)


def test_facache_merge_key_splits(orc):
    """one sequence, a long list of changed keys: the keys are split over
    workgroups, the memo enters split 0 only"""
    D = need_gpu()
    B, Hkv, Hq, L, d = 1, 1, 2, 3000, 128
    cache = _fill(D, B, Hkv, L, d, W.BF16, seed=5, std=1 / np.sqrt(d))
    n_q = 40
    assert D.dllm_facache_merge_workspace(cache, W.BF16, Hq, n_q, 2000) > 0
    q = (torch.randn((B, Hq, n_q, d), generator=torch.Generator().manual_seed(6)) / np.sqrt(d)).bfloat16().cuda()
    mo, ml = W.memo_state(B, Hq, n_q, d, seed=7, o_std=0.1, lse_mean=np.log(1000.0), empty_frac=0.1,
                          device="cuda")
    kid = torch.arange(500, 2500, dtype=torch.int32, device="cuda")[None]
    _merge_check(orc, D, cache, q, mo, ml, kid, "split bf16")
    _merge_check(orc, D, cache, q, mo, ml, kid, "split f32 out", out_dtype=torch.float32)


def test_facache_merge_degenerate(orc):
    D = need_gpu()
    B, H, L, d = 1, 2, 96, 128
    cache = _fill(D, B, H, L, d, W.BF16, seed=8, std=0.1)
    n_q = 1
    q = (torch.randn((B, H, n_q, d)) * 0.1).bfloat16().cuda()
    mo, ml = W.memo_state(B, H, n_q, d, seed=9, o_std=0.1, lse_mean=2.0, device="cuda")
    kid = torch.arange(40, 72, dtype=torch.int32, device="cuda")[None]
    _merge_check(orc, D, cache, q, mo, ml, kid, "one query")
    # no changed key at all: out is the memo, lse the memo's
    none = torch.full((B, 32), -1, dtype=torch.int32, device="cuda")
    lse = torch.empty((B, H, n_q), device="cuda")
    out = D.dllm_facache_merge(cache, q, mo, ml, key_idx=none, lse=lse, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.allclose(out, mo, rtol=1e-6, atol=0) and torch.allclose(lse, ml, rtol=1e-6, atol=1e-6)
    # every memo row empty: plain attention over the changed keys
    empty = torch.full_like(ml, float("-inf"))
    nanmo = torch.full_like(mo, float("nan"))
    out = _merge_check(orc, D, cache, q, nanmo, empty, kid, "empty memo", out_dtype=torch.float32)
    assert torch.isfinite(out).all()
    # both: out = 0, lse = -inf
    out = D.dllm_facache_merge(cache, q, nanmo, empty, key_idx=none, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))


@pytest.mark.parametrize("dtype,d,Hkv,Hq,L,b", [(W.BF16, 64, 2, 4, 400, 32), (W.E4M3, 128, 1, 4, 300, 64),
                                               (W.F32, 16, 2, 2, 64, 8)])
def test_facache_lossless_gpu(orc, dtype, d, Hkv, Hq, L, b):
    """GPU fill over the unchanged keys + GPU merge of the block keys ==
    the oracle's attention over all L keys"""
    D = need_gpu()
    B = 2
    std = 1 / np.sqrt(d)
    cache = _fill(D, B, Hkv, L, d, dtype, seed=11 + L, std=std)
    starts = torch.tensor([0, (L - b) // 2], dtype=torch.int32, device="cuda")
    un, blk = D.dllm_facache_maps(L, b, starts)
    qdt = torch.float32 if dtype == W.F32 else torch.bfloat16
    for sharp in (1.0, 12 / std):
        q = (torch.randn((B, Hq, L - b, d), generator=torch.Generator().manual_seed(12)) * std * sharp).to(qdt).cuda()
        say("facache lossless", dtype, d, "sharp", sharp)
        memo_lse = torch.empty((B, Hq, L - b), device="cuda")
        memo_o = D.dllm_block_attention(cache, q, key_idx=un, out_dtype=torch.float32, lse=memo_lse)
        lse = torch.empty_like(memo_lse)
        out = D.dllm_facache_merge(cache, q, memo_o, memo_lse, key_idx=blk, lse=lse)
        torch.cuda.synchronize()
        ck, cv, ks, vs = cache_np(cache)
        ref, ref_lse = orc.block_attention(ck, cv, ks, vs, dtype, bits(q),
                                           W.F32 if dtype == W.F32 else W.BF16)
        _compare(cache, out, lse, ref, ref_lse, f"lossless {dtype} sharp {sharp}")


def test_facache_llada_full_sampled(orc):
    """the LLaDA-shaped step at full size: 16 x 32 heads x 2016 queries
    outside the 32-position block, d 128, bf16 cache"""
    D = need_gpu()
    cfg = W.CONFIGS["llada"]
    cache = new_cache(D, cfg.B, cfg.Hkv, cfg.L, cfg.d, W.BF16)
    k, v = W.kv_rows(cfg, device="cuda")
    D.dllm_scatter_kv(cache, k, v, torch.arange(cfg.L, dtype=torch.int32, device="cuda").repeat(cfg.B, 1))
    pos = W.block_positions(cfg, "cuda")
    kn, vn = W.kv_rows(cfg, device="cuda", which="fresh")
    D.dllm_scatter_kv(cache, kn, vn, pos)
    un, blk = D.dllm_facache_maps(cfg.L, cfg.b, pos[:, 0].contiguous())
    q = W.outside_queries(cfg, device="cuda")
    n_q = cfg.L - cfg.b
    rng = np.random.default_rng(4)
    heads = np.stack([rng.integers(0, cfg.B, 12), rng.integers(0, cfg.Hq, 12)], 1).astype(np.int32)
    # a seeded memo, the same for both sides
    mo, ml = W.memo_state(cfg.B, cfg.Hq, n_q, cfg.d, seed=13, o_std=cfg.qkv_std,
                          lse_mean=np.log(n_q), empty_frac=0.01, device="cuda")
    _merge_check(orc, D, cache, q, mo, ml, blk, "llada merge", heads=heads)
    # lossless at full size: GPU fill + merge vs all-key attention, sampled heads
    say("facache llada lossless")
    memo_lse = torch.empty((cfg.B, cfg.Hq, n_q), device="cuda")
    memo_o = D.dllm_block_attention(cache, q, key_idx=un, out_dtype=torch.float32, lse=memo_lse)
    lse = torch.empty_like(memo_lse)
    out = D.dllm_facache_merge(cache, q, memo_o, memo_lse, key_idx=blk, lse=lse)
    torch.cuda.synchronize()
    ck, cv, ks, vs = cache_np(cache)
    hs = heads[:6]
    ref, ref_lse = orc.block_attention(ck, cv, ks, vs, W.BF16, bits(q), W.BF16, heads=hs)
    _compare(cache, torch.stack([out[b_, h_] for b_, h_ in hs]),
             torch.stack([lse[b_, h_] for b_, h_ in hs]), ref, ref_lse, "llada lossless")


def test_facache_deterministic():
    D = need_gpu()
    B, H, L, d, b = 2, 4, 300, 128, 32
    cache = _fill(D, B, H, L, d, W.BF16, seed=14, std=0.1)
    un, blk = D.dllm_facache_maps(L, b, torch.tensor([10, 200], dtype=torch.int32, device="cuda"))
    q = (torch.randn((B, H, L - b, d)) * 0.1).bfloat16().cuda()
    mo, ml = W.memo_state(B, H, L - b, d, seed=15, o_std=0.1, lse_mean=5.0, device="cuda")
    say("facache determinism")
    a = D.dllm_facache_merge(cache, q, mo, ml, key_idx=blk).clone()
    c = D.dllm_facache_merge(cache, q, mo, ml, key_idx=blk)
    assert torch.equal(a, c)
