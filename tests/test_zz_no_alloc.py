"""dllm_scatter_attention_noalloc, the allocation-free variant of
dllm_scatter_attention, against that entry point: two calls in a row on
the same GPU (the second with a smaller input, both with key splits, so both
use the library's scratch), each compared bit for bit with
dllm_scatter_attention on identical caches and inputs (output, lse and the
cache afterwards); and a call without key splits."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import bits, need_gpu, new_cache, say

pytestmark = pytest.mark.gpu


def _pair(D, B, Hkv, Hq, L, d, b, n, dtype, seed, with_map):
    g = torch.Generator().manual_seed(seed)
    src = torch.bfloat16
    k = (torch.randn((B, L, Hkv, d), generator=g) / np.sqrt(d)).to(src).cuda()
    v = (torch.randn((B, L, Hkv, d), generator=g) / np.sqrt(d)).to(src).cuda()
    caches = []
    for _ in range(2):
        c = new_cache(D, B, Hkv, L, d, dtype)
        D.dllm_scatter_kv(c, k, v, torch.arange(L, dtype=torch.int32, device="cuda").repeat(B, 1))
        caches.append(c)
    kn = (torch.randn((B, n, Hkv, d), generator=g) / np.sqrt(d)).to(src).cuda()
    vn = (torch.randn((B, n, Hkv, d), generator=g) / np.sqrt(d)).to(src).cuda()
    rng = np.random.default_rng(seed)
    pos = torch.from_numpy(np.stack([rng.choice(L, n, replace=False) for _ in range(B)]).astype(np.int32)).cuda()
    q = (torch.randn((B, Hq, b, d), generator=g) / np.sqrt(d)).to(torch.bfloat16).cuda()
    kid = None
    if with_map:
        kid = torch.empty((B, 4 + 8188), dtype=torch.int32, device="cuda")
        D.dllm_sink_rolling_map(L, 4, 8188, torch.full((B,), L, dtype=torch.int32, device="cuda"), kid)
    return caches, kn, vn, pos, q, kid


def _compare(D, shape, seed, with_map, expect_split):
    B, Hkv, Hq, L, d, b, n, dtype = shape
    (c1, c2), kn, vn, pos, q, kid = _pair(D, B, Hkv, Hq, L, d, b, n, dtype, seed, with_map)
    n_keys = kid.shape[1] if kid is not None else L
    ws_need = D.dllm_block_attention_workspace(c1, W.BF16, Hq, b, n_keys)
    assert (ws_need > 0) == expect_split and ws_need <= D.NOALLOC_SCRATCH_BYTES
    ws = torch.zeros(max(ws_need, 16), dtype=torch.uint8, device="cuda")
    o1 = torch.empty_like(q)
    o2 = torch.full_like(q, float("nan"))
    l1 = torch.empty((B, Hq, b), dtype=torch.float32, device="cuda")
    l2 = torch.full_like(l1, float("nan"))
    say("no-alloc scatter_attention", shape, "map" if with_map else "", "split" if expect_split else "")
    D.dllm_scatter_attention(c1, kn, vn, pos, q, key_idx=kid, out=o1, lse=l1, workspace=ws)
    D.dllm_scatter_attention_noalloc(c2, kn, vn, pos, q, o2, key_idx=kid, lse=l2)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))
    assert np.array_equal(bits(c1.k), bits(c2.k)) and np.array_equal(bits(c1.v), bits(c2.v))
    if dtype == W.E4M3:
        assert torch.equal(c1.k_scale, c2.k_scale) and torch.equal(c1.v_scale, c2.v_scale)


def test_noalloc_matches_scatter_attention_twice():
    D = need_gpu()
    # the long-context layout (e4m3, sink + rolling map, grouped rows, 8 key
    # splits), then a smaller one-sequence bf16 call whose keys are split too
    _compare(D, (2, 2, 8, 9000, 128, 64, 64, W.E4M3), seed=5, with_map=True, expect_split=True)
    _compare(D, (1, 1, 1, 4096, 64, 32, 40, W.BF16), seed=6, with_map=False, expect_split=True)


def test_noalloc_without_split():
    D = need_gpu()
    _compare(D, (2, 3, 3, 1000, 64, 32, 32, W.BF16), seed=7, with_map=False, expect_split=False)
