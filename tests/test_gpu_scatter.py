"""GPU parity of dllm_cache_init, dllm_scatter_kv and dllm_sink_rolling_map
against the oracle: bit-exact cache bytes and scales, bit-exact key maps."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import bits, cache_np, need_gpu, new_cache, say

pytestmark = pytest.mark.gpu


def _rows(shape, dt, seed, std=0.5):
    g = torch.Generator().manual_seed(seed)
    tdt = torch.float32 if dt == W.F32 else torch.bfloat16
    return (torch.randn(shape, generator=g) * std).to(tdt)


@pytest.mark.parametrize("dtype,src,d", [(W.F32, W.F32, 16), (W.BF16, W.BF16, 64), (W.BF16, W.BF16, 128),
                                         (W.E4M3, W.BF16, 128), (W.E4M3, W.F32, 256)])
def test_scatter_bitwise(orc, dtype, src, d):
    D = need_gpu()
    B, H, L, n = 3, 2, 97, 13
    say("scatter", dtype, src, d)
    cache = new_cache(D, B, H, L, d, dtype)
    ck, cv, ks, vs = cache_np(cache)
    assert not ck.any() and not cv.any()                      # init zero-fills
    for step in range(3):
        g = torch.Generator().manual_seed(100 + step)
        pos = torch.stack([torch.randperm(L, generator=g)[:n] for _ in range(B)]).int()
        pos[1, 3] = -1                                        # padding
        kn, vn = _rows((B, n, H, d), src, 10 + step), _rows((B, n, H, d), src, 20 + step)
        bad = torch.zeros(1, dtype=torch.int32, device="cuda")
        D.dllm_scatter_kv(cache, kn.cuda(), vn.cuda(), pos.cuda(), bad)
        orc.scatter_kv(ck, cv, ks, vs, dtype, bits(kn), bits(vn), src, pos.numpy())
        torch.cuda.synchronize()
        gk, gv, gks, gvs = cache_np(cache)
        assert np.array_equal(gk, ck) and np.array_equal(gv, cv), step
        if dtype == W.E4M3:
            assert np.array_equal(gks.view(np.uint32), ks.view(np.uint32))
            assert np.array_equal(gvs.view(np.uint32), vs.view(np.uint32))
        assert bad.item() == 0


def test_scatter_bad_positions_counted():
    D = need_gpu()
    say("scatter bad positions")
    cache = new_cache(D, 2, 1, 10, 64, W.BF16)
    pos = torch.tensor([[3, 10, -1], [-2, 4, 9]], dtype=torch.int32, device="cuda")
    kn = torch.ones((2, 3, 1, 64), dtype=torch.bfloat16, device="cuda")
    bad = torch.zeros(1, dtype=torch.int32, device="cuda")
    D.dllm_scatter_kv(cache, kn, kn, pos, bad)
    torch.cuda.synchronize()
    assert bad.item() == 2                                   # 10 (== L) and -2
    written = torch.nonzero(cache.k.float().abs().sum(-1)).tolist()
    assert written == [[0, 0, 3], [1, 0, 4], [1, 0, 9]]


def test_e4m3_encoder_every_code_and_midpoint(orc):
    """rows whose amax is exactly 448 have scale 1, so x/scale = x: the rest of
    the row then walks every e4m3 grid value, every midpoint and its float
    neighbours, zeros, subnormal-range values and values above 448"""
    D = need_gpu()
    codes = np.arange(0x7F, dtype=np.uint8)
    grid = orc.e4m3_value(codes).astype(np.float32)
    mids = ((grid[1:].astype(np.float64) + grid[:-1]) / 2).astype(np.float32)
    vals = np.concatenate([grid, mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(500)),
                           np.float32([0.0, -0.0, 1e-12, 2.0 ** -10, 3 * 2.0 ** -11, 447.99, 448.0])])
    vals = np.concatenate([vals, -vals])
    per = 127
    nrows = -(-len(vals) // per)
    x = np.zeros((nrows, 128), np.float32)
    x[:, 0] = 448.0
    flat = np.zeros(nrows * per, np.float32)
    flat[:len(vals)] = vals
    x[:, 1:] = flat.reshape(nrows, per)
    say("e4m3 encoder sweep", nrows, "rows")
    cache = new_cache(D, 1, 1, nrows, 128, W.E4M3)
    kn = torch.from_numpy(x).reshape(1, nrows, 1, 128)
    pos = torch.arange(nrows, dtype=torch.int32).reshape(1, nrows)
    D.dllm_scatter_kv(cache, kn.cuda(), kn.cuda(), pos.cuda())
    torch.cuda.synchronize()
    gk, _, gks, _ = cache_np(cache)
    assert np.all(gks == 1.0)
    ref = orc.e4m3_encode(x)
    assert np.array_equal(gk[0, 0], ref)
    # a zero row: scale 0 and zero codes; a tiny row: scale in the float32 subnormal range
    z = torch.zeros((1, 2, 1, 128))
    z[0, 1, 0, :] = torch.linspace(-1e-39, 1e-39, 128)
    cache2 = new_cache(D, 1, 1, 2, 128, W.E4M3)
    D.dllm_scatter_kv(cache2, z.cuda(), z.cuda(), torch.tensor([[0, 1]], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    gk2, _, gks2, _ = cache_np(cache2)
    c0, s0 = orc.e4m3_quantize_group(z[0, 0, 0].numpy())
    c1, s1 = orc.e4m3_quantize_group(z[0, 1, 0].numpy())
    assert gks2[0, 0, 0, 0] == s0 == 0.0 and not gk2[0, 0, 0].any()
    assert gks2[0, 0, 1, 0] == s1 and np.array_equal(gk2[0, 0, 1], c1)


def test_scatter_longctx_fill_sampled(orc):
    """full e4m3 cache of the long-context workload (4 x 8 x 32768 x 128):
    every row quantised on the GPU; a sample of rows checked bit for bit"""
    D = need_gpu()
    cfg = W.CONFIGS["longctx"]
    say("longctx full fill")
    cache = new_cache(D, cfg.B, cfg.Hkv, cfg.L, cfg.d, W.E4M3)
    k, v = W.kv_rows(cfg, device="cuda", which="cache")
    pos = torch.arange(cfg.L, dtype=torch.int32, device="cuda").repeat(cfg.B, 1)
    D.dllm_scatter_kv(cache, k, v, pos)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    for _ in range(64):
        b, h, p = rng.integers(cfg.B), rng.integers(cfg.Hkv), rng.integers(cfg.L)
        for src, dst, sc in ((k, cache.k, cache.k_scale), (v, cache.v, cache.v_scale)):
            x = src[b, p, h].float().cpu().numpy()
            codes, s = orc.e4m3_quantize_group(x)
            assert sc[b, h, p, 0].item() == s
            assert np.array_equal(dst[b, h, p].cpu().numpy(), codes)


def test_sink_rolling_map_bitwise(orc):
    D = need_gpu()
    for (L, S, R, ends) in [(32768, 4, 8188, [32768, 8192, 8191, 100, 3, 0]),
                            (20, 3, 4, [0, 2, 3, 5, 7, 8, 20]), (64, 0, 10, [64, 5])]:
        say("sink map", L, S, R, ends)
        end = torch.tensor(ends, dtype=torch.int32, device="cuda")
        out = torch.full((len(ends), S + R + 3), 77, dtype=torch.int32, device="cuda")
        D.dllm_sink_rolling_map(L, S, R, end, out)
        got = out.cpu().numpy()
        for i, e in enumerate(ends):
            ref = orc.sink_rolling_keys(S, R, e)
            row = np.full(S + R + 3, -1, np.int32)
            row[:len(ref)] = ref
            assert np.array_equal(got[i], row), (L, S, R, e)


@pytest.mark.parametrize("B,L,n", [(3, 97, 40), (2, 131072, 5000), (4, 1024, 0), (1, 64, 64)])
def test_check_positions_gpu(orc, B, L, n):
    """the debug check of position lists, bit-exact counts against the
    oracle: random lists with planted repeats, padding and bad entries, a
    maximum-length sequence, an empty list and a full permutation"""
    D = need_gpu()
    rng = np.random.default_rng(L + n)
    if n == L:
        pos = np.stack([rng.permutation(L) for _ in range(B)]).astype(np.int32)
    else:
        pos = rng.integers(-2, L + 2, (B, n)).astype(np.int32)
        if n:
            pos[0, n // 2:] = pos[0, :n - n // 2]            # half the first row repeats
            pos[-1, ::5] = -1
    say("check_positions", B, L, n)
    bad, dup = D.dllm_check_positions(L, torch.from_numpy(pos).cuda())
    torch.cuda.synchronize()
    obad, odup = orc.check_positions(L, pos)
    assert np.array_equal(bad.cpu().numpy(), obad) and np.array_equal(dup.cpu().numpy(), odup)
    if n == L:
        assert not obad.any() and not odup.any()
