"""GPU parity of dllm_scatter_attention: the cache and the output equal, bit
for bit, what dllm_scatter_kv then dllm_block_attention leave, whether the
per-wave attention kernel writes the block's rows itself (bf16 cache and rows,
no key map, one 32-row group per KV head) or the two kernels run in sequence;
and the output is checked against the oracle's scatter and attention on the
same bytes, to the attention bars."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import attn_errors, bits, cache_np, need_gpu, new_cache, say

pytestmark = pytest.mark.gpu


def _case(D, B, Hkv, Hq, L, d, b, n, dtype, seed, with_map=False, bad=False):
    """two identical caches, the block's fresh rows and positions, queries"""
    g = torch.Generator().manual_seed(seed)
    src = torch.float32 if dtype == W.F32 else torch.bfloat16
    caches = []
    k = (torch.randn((B, L, Hkv, d), generator=g) / np.sqrt(d)).to(src).cuda()
    v = (torch.randn((B, L, Hkv, d), generator=g) / np.sqrt(d)).to(src).cuda()
    for _ in range(2):
        c = new_cache(D, B, Hkv, L, d, dtype)
        D.dllm_scatter_kv(c, k, v, torch.arange(L, dtype=torch.int32, device="cuda").repeat(B, 1))
        caches.append(c)
    kn = (torch.randn((B, n, Hkv, d), generator=g) / np.sqrt(d)).to(src).cuda()
    vn = (torch.randn((B, n, Hkv, d), generator=g) / np.sqrt(d)).to(src).cuda()
    rng = np.random.default_rng(seed)
    pos = np.stack([rng.choice(L, n, replace=False) for _ in range(B)]).astype(np.int32)
    if bad:
        pos[0, 0] = -1                 # padding
        pos[-1, -1] = L + 5            # out of range: skipped and counted
    q = (torch.randn((B, Hq, b, d), generator=g) / np.sqrt(d)).to(torch.bfloat16).cuda()
    kid = None
    if with_map:
        kid = torch.from_numpy(np.stack([np.sort(rng.choice(L, min(L, 300), replace=False))
                                         for _ in range(B)]).astype(np.int32)).cuda()
    return caches, kn, vn, torch.from_numpy(pos).cuda(), q, kid


@pytest.mark.parametrize("B,Hkv,Hq,L,d,b,n,dtype,with_map,bad", [
    (2, 3, 3, 1000, 64, 32, 32, W.BF16, False, False),    # one kernel: the gpt2 layout
    (2, 2, 2, 700, 128, 32, 32, W.BF16, False, True),     # one kernel, padding and a bad position
    (1, 1, 1, 4096, 64, 32, 40, W.BF16, False, False),    # one kernel with key splits and the merge pass
    (2, 2, 2, 700, 128, 32, 32, W.BF16, True, False),     # key map: the two kernels in sequence
    (2, 1, 4, 600, 128, 64, 64, W.BF16, False, False),    # grouped rows: the two kernels in sequence
    (1, 2, 2, 300, 128, 32, 16, W.E4M3, False, False),    # e4m3: quantising scatter, then attention
    (2, 2, 8, 700, 128, 64, 64, W.E4M3, True, True),      # e4m3, grouped rows, key map, padding and a bad position
    (2, 1, 1, 500, 128, 48, 48, W.E4M3, True, False),     # the same with 2-wave workgroups, rows past the last
])
def test_scatter_attention_equals_two_calls(orc, B, Hkv, Hq, L, d, b, n, dtype, with_map, bad):
    D = need_gpu()
    say("scatter_attention", B, Hkv, Hq, L, d, b, n, dtype, "map" if with_map else "", "bad" if bad else "")
    (c1, c2), kn, vn, pos, q, kid = _case(D, B, Hkv, Hq, L, d, b, n, dtype, seed=L + d + n,
                                          with_map=with_map, bad=bad)
    bad1 = torch.zeros(1, dtype=torch.int32, device="cuda")
    bad2 = torch.zeros(1, dtype=torch.int32, device="cuda")
    n_keys = kid.shape[1] if kid is not None else L
    ws = D.dllm_block_attention_workspace(c1, W.BF16, Hq, b, n_keys)
    ws1 = torch.zeros(max(ws, 16), dtype=torch.uint8, device="cuda")
    ws2 = torch.zeros(max(ws, 16), dtype=torch.uint8, device="cuda")
    lse1 = torch.empty((B, Hq, b), dtype=torch.float32, device="cuda")
    lse2 = torch.empty_like(lse1)
    D.dllm_scatter_kv(c1, kn, vn, pos, bad_count=bad1)
    o1 = D.dllm_block_attention(c1, q, key_idx=kid, lse=lse1, workspace=ws1)
    o2 = D.dllm_scatter_attention(c2, kn, vn, pos, q, key_idx=kid, lse=lse2, workspace=ws2, bad_count=bad2)
    torch.cuda.synchronize()
    assert torch.equal(c1.k.view(torch.uint8), c2.k.view(torch.uint8))
    assert torch.equal(c1.v.view(torch.uint8), c2.v.view(torch.uint8))
    if dtype == W.E4M3:
        assert torch.equal(c1.k_scale, c2.k_scale) and torch.equal(c1.v_scale, c2.v_scale)
    assert torch.equal(o1, o2)
    assert torch.equal(lse1, lse2)
    assert int(bad1.item()) == int(bad2.item()) == (1 if bad else 0)
    # the oracle: the scatter on the cache as it was, then the attention
    ck, cv, ks, vs = cache_np(c2)
    ref, _ = orc.block_attention(ck, cv, ks, vs, dtype, bits(q), W.BF16,
                                 key_idx=kid.cpu().numpy() if kid is not None else None)
    e_abs, e_norm = attn_errors(o2, ref)
    assert e_abs <= (6e-2 if dtype == W.E4M3 else 2e-2) and e_norm <= 1e-2, (e_abs, e_norm)


def test_scatter_attention_e4m3_sink_map_splits(orc):
    """the long-context form at a small size: e4m3 cache, sinks + a rolling
    window of 8188 keys ending at the sequence's end, 8 key splits, the block
    at the newest positions (in the last split's keys) with padding, an
    out-of-range position and two rows outside the map: bit for bit as the
    scatter then the attention"""
    D = need_gpu()
    B, Hkv, Hq, L, d, b, n = 1, 1, 4, 9000, 128, 64, 64
    (c1, c2), kn, vn, _, q, _ = _case(D, B, Hkv, Hq, L, d, b, n, W.E4M3, seed=9000)
    pos = torch.arange(L - n, L, dtype=torch.int32, device="cuda").view(1, n).clone()
    pos[0, 3] = -1                      # padding
    pos[0, 7] = L + 1                   # out of range: skipped and counted
    pos[0, 10] = 100                    # outside the map (between the sinks and the window)
    pos[0, 11] = 2                      # a sink
    kid = torch.empty((B, 4 + 8188), dtype=torch.int32, device="cuda")
    D.dllm_sink_rolling_map(L, 4, 8188, torch.tensor([L], dtype=torch.int32, device="cuda"), kid)
    say("scatter_attention e4m3 sink map splits")
    ws = D.dllm_block_attention_workspace(c1, W.BF16, Hq, b, kid.shape[1])
    assert ws > 0                       # key splits
    bad1 = torch.zeros(1, dtype=torch.int32, device="cuda")
    bad2 = torch.zeros(1, dtype=torch.int32, device="cuda")
    D.dllm_scatter_kv(c1, kn, vn, pos, bad_count=bad1)
    o1 = D.dllm_block_attention(c1, q, key_idx=kid)
    o2 = D.dllm_scatter_attention(c2, kn, vn, pos, q, key_idx=kid, bad_count=bad2)
    torch.cuda.synchronize()
    assert torch.equal(c1.k.view(torch.uint8), c2.k.view(torch.uint8))
    assert torch.equal(c1.v.view(torch.uint8), c2.v.view(torch.uint8))
    assert torch.equal(c1.k_scale, c2.k_scale) and torch.equal(c1.v_scale, c2.v_scale)
    assert torch.equal(o1, o2)
    assert int(bad1.item()) == int(bad2.item()) == 1
    ck, cv, ks, vs = cache_np(c2)
    ref, _ = orc.block_attention(ck, cv, ks, vs, W.E4M3, bits(q), W.BF16, key_idx=kid.cpu().numpy())
    e_abs, e_norm = attn_errors(o2, ref)
    assert e_abs <= 6e-2 and e_norm <= 1e-2, (e_abs, e_norm)


def test_scatter_attention_rows_land_where_the_oracle_puts_them(orc):
    """the one-kernel path writes the cache exactly as the oracle's scatter"""
    D = need_gpu()
    B, Hkv, Hq, L, d, b, n = 2, 2, 2, 1024, 64, 32, 32
    (c1, _), kn, vn, pos, q, _ = _case(D, B, Hkv, Hq, L, d, b, n, W.BF16, seed=7)
    ck0, cv0, _, _ = cache_np(c1)
    D.dllm_scatter_attention(c1, kn, vn, pos, q)
    torch.cuda.synchronize()
    ck, cv = ck0.copy(), cv0.copy()
    orc.scatter_kv(ck, cv, None, None, W.BF16, bits(kn), bits(vn), W.BF16, pos.cpu().numpy())
    got_k, got_v, _, _ = cache_np(c1)
    assert np.array_equal(got_k, ck) and np.array_equal(got_v, cv)


@pytest.mark.parametrize("name,n_heads", [("gpt2", None), ("llada", 24), ("longctx", 10)])
def test_scatter_attention_full_size(orc, name, n_heads):
    """the call as the bench step makes it, at the workload's full size: the
    block's rows land in the cache (bf16: the fresh bytes themselves; e4m3:
    the oracle's quantisation of them), and the output matches the oracle on
    the cache the call leaves (every head at the gpt2 size, sampled heads at
    the others)"""
    D = need_gpu()
    cfg = W.CONFIGS[name]
    say("scatter_attention full", name)
    cache = new_cache(D, cfg.B, cfg.Hkv, cfg.L, cfg.d, cfg.kv_dtype)
    k, v = W.kv_rows(cfg, device="cuda")
    D.dllm_scatter_kv(cache, k, v, torch.arange(cfg.L, dtype=torch.int32, device="cuda").repeat(cfg.B, 1))
    del k, v
    kn, vn = W.kv_rows(cfg, device="cuda", which="fresh")
    pos = W.block_positions(cfg, "cuda")
    kid = None
    if cfg.sinks:
        end = (pos[:, -1] + 1).contiguous()
        kid = torch.empty((cfg.B, cfg.sinks + cfg.rolling), dtype=torch.int32, device="cuda")
        D.dllm_sink_rolling_map(cfg.L, cfg.sinks, cfg.rolling, end, kid)
    q = W.queries(cfg, device="cuda")
    lse = torch.empty((cfg.B, cfg.Hq, cfg.b), dtype=torch.float32, device="cuda")
    out = D.dllm_scatter_attention(cache, kn, vn, pos, q, key_idx=kid, lse=lse)
    torch.cuda.synchronize()
    p = pos.long()
    bi = torch.arange(cfg.B, device="cuda")[:, None]
    got_k = cache.k[bi, :, p].cpu()                    # [B, b, Hkv, d]
    got_v = cache.v[bi, :, p].cpu()
    if cfg.kv_dtype == W.BF16:
        assert torch.equal(got_k.view(torch.int16), kn.cpu().view(torch.int16))
        assert torch.equal(got_v.view(torch.int16), vn.cpu().view(torch.int16))
    else:
        for src, got, sc in ((kn, got_k, cache.k_scale), (vn, got_v, cache.v_scale)):
            # a few rows quantised by the oracle, codes and scale
            for j, h in ((0, 0), (cfg.b - 1, cfg.Hkv - 1), (cfg.b // 2, 1)):
                x = orc.bf16_value(bits(src)[-1, j, h])
                codes, scale = orc.e4m3_quantize_group(x)
                assert np.array_equal(got[-1, j, h].numpy(), codes), (j, h)
                assert float(sc[-1, h, int(pos[-1, j]), 0]) == scale, (j, h)
    ck, cv, ks, vs = cache_np(cache)
    kid_np = kid.cpu().numpy() if kid is not None else None
    if n_heads is None:
        ref, ref_lse = orc.block_attention(ck, cv, ks, vs, cfg.kv_dtype, bits(q), W.BF16, key_idx=kid_np)
        out_s, lse_s = out, lse
    else:
        rng = np.random.default_rng(5)
        heads = np.stack([rng.integers(0, cfg.B, n_heads), rng.integers(0, cfg.Hq, n_heads)], 1).astype(np.int32)
        ref, ref_lse = orc.block_attention(ck, cv, ks, vs, cfg.kv_dtype, bits(q), W.BF16, key_idx=kid_np,
                                           heads=heads)
        out_s = torch.stack([out[b_, h_] for b_, h_ in heads])
        lse_s = torch.stack([lse[b_, h_] for b_, h_ in heads])
    e_abs, e_norm = attn_errors(out_s, ref)
    bar = 6e-2 if cfg.kv_dtype == W.E4M3 else 2e-2
    assert e_abs <= bar and e_norm <= 1e-2, (name, e_abs, e_norm)
    assert np.all(np.abs(lse_s.cpu().numpy() - ref_lse) <= 1e-3), name
