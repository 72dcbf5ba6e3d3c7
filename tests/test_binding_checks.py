"""The Python binding checks every tensor's shape and dtype against the call
before a pointer reaches the library, so a mis-shaped argument raises on the
host instead of letting a kernel read or write past a buffer.  These run on
the CPU: every case below raises before any device pointer is taken."""
import pytest
import torch

import cached_denoising_amd as D


def _cache(dtype=D.BF16, B=2, L=16, H=2, d=64):
    desc = D._KVCache(B=B, L=L, n_kv_heads=H, d_head=d, dtype=dtype)
    return D.Cache(desc, None, None, None, None)


def _raises(match, fn, *a, **k):
    with pytest.raises(D.DllmError, match=match):
        fn(*a, **k)


def test_scatter_arguments():
    c = _cache()
    kn = torch.zeros((2, 4, 2, 64), dtype=torch.bfloat16)
    pos = torch.zeros((2, 4), dtype=torch.int32)
    _raises("pos: dtype", D.dllm_scatter_kv, c, kn, kn, pos.long())
    _raises("pos: shape", D.dllm_scatter_kv, c, kn, kn, pos[:1])
    _raises("k_new: shape", D.dllm_scatter_kv, c, kn.transpose(1, 2), kn, pos)
    _raises("k_new: dtype", D.dllm_scatter_kv, c, kn.float(), kn.float(), pos)
    _raises("v_new: shape", D.dllm_scatter_kv, c, kn, kn[:, :3], pos)
    _raises("bad_count: dtype", D.dllm_scatter_kv, c, kn, kn, pos, bad_count=torch.zeros(1, dtype=torch.int64))
    _raises("bad_count must hold", D.dllm_scatter_kv, c, kn, kn, pos, bad_count=torch.zeros(0, dtype=torch.int32))
    # an e4m3 cache takes float32 or bfloat16 rows
    e = _cache(D.E4M3, d=128)
    _raises("k_new: dtype", D.dllm_scatter_kv, e, torch.zeros((2, 4, 2, 128), dtype=torch.float16),
            torch.zeros((2, 4, 2, 128), dtype=torch.float16), pos)
    # a well-formed call on host tensors stops only at the device check
    _raises("GPU tensor", D.dllm_scatter_kv, c, kn, kn, pos)


def test_attention_arguments():
    c = _cache()
    q = torch.zeros((2, 4, 8, 64), dtype=torch.bfloat16)
    _raises("q: shape", D.dllm_block_attention, c, q[:1])
    _raises("q: shape", D.dllm_block_attention, c, torch.zeros((2, 4, 8, 32), dtype=torch.bfloat16))
    _raises("multiple of 2 KV heads", D.dllm_block_attention, c, torch.zeros((2, 3, 8, 64), dtype=torch.bfloat16))
    _raises("q: dtype", D.dllm_block_attention, c, q.half())
    _raises("key_idx: dtype", D.dllm_block_attention, c, q, key_idx=torch.zeros((2, 5), dtype=torch.int64))
    _raises("key_idx: shape", D.dllm_block_attention, c, q, key_idx=torch.zeros((3, 5), dtype=torch.int32))
    _raises("out: shape", D.dllm_block_attention, c, q, out=torch.zeros((2, 4, 7, 64), dtype=torch.bfloat16))
    _raises("out: dtype", D.dllm_block_attention, c, q, out=torch.zeros((2, 4, 8, 64), dtype=torch.float16))
    _raises("lse: dtype", D.dllm_block_attention, c, q, out=torch.zeros_like(q),
            lse=torch.zeros((2, 4, 8), dtype=torch.bfloat16))
    _raises("lse: shape", D.dllm_block_attention, c, q, out=torch.zeros_like(q),
            lse=torch.zeros((2, 4, 9), dtype=torch.float32))
    kn = torch.zeros((2, 4, 2, 64), dtype=torch.bfloat16)
    pos = torch.zeros((2, 4), dtype=torch.int32)
    _raises("k_new: shape", D.dllm_scatter_attention, c, kn[:, :, :1], kn, pos, q, out=torch.zeros_like(q))
    _raises("out: shape", D.dllm_scatter_attention, c, kn, kn, pos, q, out=q[:, :, :4])
    mo = torch.zeros((2, 4, 8, 64))
    ml = torch.zeros((2, 4, 8))
    _raises("memo", D.dllm_facache_merge, c, q, mo[:, :2], ml)
    _raises("out: shape", D.dllm_facache_merge, c, q, mo, ml, out=torch.zeros((2, 4, 8, 32), dtype=torch.bfloat16))
    _raises("key_idx: dtype", D.dllm_facache_merge, c, q, mo, ml, key_idx=torch.zeros((2, 4), dtype=torch.int16))


def test_map_arguments():
    _raises("end: shape", D.dllm_sink_rolling_map, 16, 2, 4, torch.zeros(3, dtype=torch.int32),
            torch.zeros((2, 6), dtype=torch.int32))
    _raises("key_idx: dtype", D.dllm_sink_rolling_map, 16, 2, 4, torch.zeros(2, dtype=torch.int32),
            torch.zeros((2, 6), dtype=torch.int64))
    _raises("start: dtype", D.dllm_facache_maps, 16, 4, torch.zeros(2, dtype=torch.int64))
    _raises("block length", D.dllm_facache_maps, 16, 16, torch.zeros(2, dtype=torch.int32))
    _raises("unchanged_idx: shape", D.dllm_facache_maps, 16, 4, torch.zeros(2, dtype=torch.int32),
            torch.zeros((2, 11), dtype=torch.int32), torch.zeros((2, 4), dtype=torch.int32))
    _raises("pos: dtype", D.dllm_check_positions, 16, torch.zeros((2, 4), dtype=torch.int64))
    _raises("bad: shape", D.dllm_check_positions, 16, torch.zeros((2, 4), dtype=torch.int32),
            bad=torch.zeros(3, dtype=torch.int32))


def test_vocab_and_fp8_arguments():
    x = torch.zeros((4, 100), dtype=torch.bfloat16)
    _raises("logits: dtype", D.dllm_vocab_stats, x.half())
    _raises("V = 101", D.dllm_vocab_stats, x, V=101)
    _raises("argmax: dtype", D.dllm_vocab_stats, x, argmax=torch.zeros(4, dtype=torch.int64))
    _raises("maxprob: shape", D.dllm_vocab_stats, x, maxprob=torch.zeros(3))
    a = torch.zeros((64, 256), dtype=torch.uint8)
    w = torch.zeros((256, 256), dtype=torch.uint8)
    sa = torch.zeros((2, 64), dtype=torch.uint8)
    sw = torch.zeros((2, 2), dtype=torch.uint8)
    _raises("a_scale: shape", D.dllm_fp8_gemm, a, sa[:1], w, sw)
    _raises("w_scale: shape", D.dllm_fp8_gemm, a, sa, w, sw[:1])
    _raises("disagree", D.dllm_fp8_gemm, a, sa, w[:, :128], sw)
    _raises("out: dtype", D.dllm_fp8_gemm, a, sa, w, sw, out=torch.zeros((64, 256)))
    _raises("out_codes: shape", D.dllm_fp8_gemm_swiglu, a, sa, w, sw, out_codes=torch.zeros((64, 256), dtype=torch.uint8))
    _raises("codes: shape", D.dllm_fp8_quant_rows, torch.zeros((8, 256)), codes=torch.zeros((8, 128), dtype=torch.uint8))
    _raises("gamma: shape", D.dllm_fp8_addnorm_quant, torch.zeros((8, 256)), None, torch.zeros(128))
    _raises("scales: shape", D.dllm_fp8_quant_weight, torch.zeros((128, 256)),
            scales=torch.zeros((2, 2), dtype=torch.uint8))


def test_stability_arguments():
    st = D.StabilityState.__new__(D.StabilityState)
    st.B, st.L, st.D = 2, 8, 3
    am = torch.zeros((2, 8), dtype=torch.int32)
    mp = torch.zeros((2, 8))
    kw = dict(K=3, tau=0.9, R=1, V=10)
    _raises("argmax: dtype", D.dllm_stability_mask, st, 0, None, am.long(), mp, mp, **kw)
    _raises("maxprob: 15 elements", D.dllm_stability_mask, st, 0, None, am, mp.view(-1)[:15], mp, **kw)
    _raises("pos: shape", D.dllm_stability_mask, st, 0, torch.zeros((3, 2), dtype=torch.int32), am, mp, mp, **kw)
    _raises("pos: dtype", D.dllm_stability_mask, st, 0, torch.zeros((2, 2), dtype=torch.int64), am, mp, mp, **kw)
    _raises("evicted: shape", D.dllm_evict_by_confidence, st, torch.zeros(2, dtype=torch.int32), None,
            torch.zeros(3, dtype=torch.int32))
