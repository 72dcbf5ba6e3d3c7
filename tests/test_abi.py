"""The C-ABI library loads, exports every entry point include/dllm.h declares,
and its host-side argument checks answer without a GPU (no compute call)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dllm.h")


def declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dllm_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def dl():
    import cached_denoising_amd as D
    return D


def test_header_declares_the_boundary():
    names = declared()
    for n in ["dllm_cache_init", "dllm_scatter_kv", "dllm_block_attention", "dllm_scatter_attention",
              "dllm_vocab_stats",
              "dllm_stability_mask", "dllm_sink_rolling_map", "dllm_stability_reset",
              "dllm_block_attention_workspace", "dllm_vocab_stats_workspace", "dllm_status_str",
              "dllm_facache_maps", "dllm_facache_merge", "dllm_facache_merge_workspace",
              "dllm_evict_by_confidence", "dllm_cache_quotas", "dllm_refresh_interval",
              "dllm_self_verify", "dllm_parallel_width", "dllm_confidence_decay",
              "dllm_check_positions"]:
        assert n in names


def test_library_exports_every_declared_symbol(dl):
    lib = ctypes.CDLL(dl.LIB_PATH)
    missing = [n for n in declared() if not hasattr(lib, n)]
    assert not missing
    # the binding wraps exactly these
    assert sorted(dl.EXPORTS) == declared()


def test_status_strings_and_version(dl):
    assert dl.dllm_status_str(0) == "ok"
    assert "workspace" in dl.dllm_status_str(-7)
    assert dl.dllm_version() >= 100


def test_host_validation_without_gpu(dl):
    L = dl.lib()
    desc = dl._KVCache()
    # null storage, bad dtype, misaligned row size: rejected before any HIP call
    assert L.dllm_cache_init(ctypes.byref(desc), 1, 8, 1, 16, 1, None, None, None, None, None) == -1
    assert L.dllm_cache_init(ctypes.byref(desc), 1, 8, 1, 16, 7, 16, 16, None, None, None) == -2
    assert L.dllm_cache_init(ctypes.byref(desc), 1, 8, 1, 24, 2, 16, 16, 16, 16, None) in (-3, -4)
    assert L.dllm_cache_init(None, 1, 8, 1, 16, 0, 16, 16, None, None, None) == -1
    # one (sequence, KV head)'s rows must span less than 4 GiB: 2^24 bf16 rows of 128 do not
    assert L.dllm_cache_init(ctypes.byref(desc), 1, 1 << 24, 1, 128, 1, 16, 16, None, None, None) == -5
    assert L.dllm_vocab_stats(None, 1, 4, 10, 5, None, None, None, None, 0, None) == -3   # stride < V
    assert L.dllm_vocab_stats(None, 5, 4, 10, 10, None, None, None, None, 0, None) == -2  # dtype
    assert L.dllm_vocab_stats(None, 1, 0, 10, 10, None, None, None, None, 0, None) == 0   # N = 0: no-op
    prm = dl._StabParams(K=3, D=2, R=1, tau=0.9, vocab=10)                                  # D < K
    assert L.dllm_stability_mask(1, 4, 0, None, None, 4, 16, 16, 16, 16, 16, 16, 16, 16, 16,
                                 ctypes.byref(prm), 16, 16, 16, 16, 16, None) == -1
    prm = dl._StabParams(K=3, D=3, R=1, tau=0.9, vocab=10, refresh_every=-1)                # bad schedule
    assert L.dllm_stability_mask(1, 4, 0, None, None, 4, 16, 16, 16, 16, 16, 16, 16, 16, 16,
                                 ctypes.byref(prm), 16, 16, 16, 16, 16, None) == -1
    prm = dl._StabParams(K=3, D=3, R=1, tau=0.9, vocab=10, alpha=0.7, beta=0.3)               # no decay table
    assert L.dllm_stability_mask(1, 4, 0, None, None, 4, 16, 16, 16, 16, 16, 16, 16, 16, 16,
                                 ctypes.byref(prm), 16, 16, 16, 16, 16, None) == -1
    prm = dl._StabParams(K=3, D=3, R=1, tau=0.9, vocab=10, alpha=0.7, beta=0.3, decay=16, n_decay=0)
    assert L.dllm_stability_mask(1, 4, 0, None, None, 4, 16, 16, 16, 16, 16, 16, 16, 16, 16,
                                 ctypes.byref(prm), 16, 16, 16, 16, 16, None) == -1
    prm = dl._StabParams(K=3, D=3, R=1, tau=0.9, vocab=10, alpha=0.7, beta=0.3, decay=20, n_decay=8)
    assert L.dllm_stability_mask(1, 4, 0, None, None, 4, 16, 16, 16, 16, 16, 16, 16, 16, 16,
                                 ctypes.byref(prm), 16, 16, 16, 16, 16, None) == -4          # misaligned table
    # position check: shapes and limits before any launch
    assert L.dllm_check_positions(0, 8, 16, 2, 16, 16, None) == -3
    assert L.dllm_check_positions(1, 1 << 18, 16, 2, 16, 16, None) == -5
    assert L.dllm_check_positions(1, 8, None, 2, 16, 16, None) == -1
    assert L.dllm_check_positions(1, 8, 16, 2, None, 16, None) == -1
    # eviction: shapes and limits before any launch
    assert L.dllm_evict_by_confidence(1, 0, 16, 16, None, 0, 16, 16, 16, 16, None, None) == -3
    assert L.dllm_evict_by_confidence(1, 8, 16, 16, None, 5, 16, 16, 16, 16, None, None) == -3
    assert L.dllm_evict_by_confidence(1, 8, 16, 16, 16, 9, 16, 16, 16, 16, None, None) == -3
    assert L.dllm_evict_by_confidence(1, 1 << 18, 16, 16, None, 0, 16, 16, 16, 16, None, None) == -5
    assert L.dllm_evict_by_confidence(1, 8, None, 16, None, 8, 16, 16, 16, 16, None, None) == -1
    # self-verification: window, threshold, shapes and limits before any launch
    sv = lambda B, Ln, n, W, tau, dp=16: L.dllm_self_verify(B, Ln, dp, n, 16, 16, W, tau, 16, 16, None, None,
                                                            16, 16, None, None, None)
    assert sv(1, 8, 2, 1, 0.5) == -1 and sv(1, 8, 2, 9, 0.5) == -1 and sv(1, 8, 2, 3, -0.5) == -1
    assert sv(1, 8, 2, 3, float("nan")) == -1 and sv(1, 8, 9, 3, 0.5) == -3 and sv(0, 8, 2, 3, 0.5) == -3
    assert sv(1, 1 << 18, 2, 3, 0.5) == -5 and sv(1, 8, 2, 3, 0.5, dp=None) == -1
    assert L.dllm_sink_rolling_map(1, 10, 4, 8, 16, 16, 11, None) == -3                     # n_keys < S+R
    assert L.dllm_facache_maps(1, 8, 8, 16, 16, 16, None) == -3                             # block = L
    assert L.dllm_facache_maps(1, 8, 2, None, 16, 16, None) == -1
    desc = dl._KVCache(B=1, L=64, n_kv_heads=2, d_head=64, dtype=1, k=16, v=16)
    # no memo, bad head ratio, bad dtypes, misaligned memo: rejected on the host
    assert L.dllm_facache_merge(ctypes.byref(desc), 16, 1, 4, 8, None, 0, 0.0, None, 16, 16, 1,
                                None, None, 0, None) == -1
    assert L.dllm_facache_merge(ctypes.byref(desc), 16, 1, 3, 8, None, 0, 0.0, 16, 16, 16, 1,
                                None, None, 0, None) == -3
    assert L.dllm_facache_merge(ctypes.byref(desc), 16, 2, 4, 8, None, 0, 0.0, 16, 16, 16, 1,
                                None, None, 0, None) == -2
    assert L.dllm_facache_merge(ctypes.byref(desc), 16, 1, 4, 8, None, 0, 0.0, 20, 16, 16, 1,
                                None, None, 0, None) == -4
    assert L.dllm_facache_merge(ctypes.byref(desc), 16, 1, 4, 8, None, 0, -1.0, 16, 16, 16, 1,
                                None, None, 0, None) == -1


def test_workspace_sizes(dl):
    L = dl.lib()
    assert L.dllm_vocab_stats_workspace(32768, 126464) == 0          # one workgroup per row
    assert L.dllm_vocab_stats_workspace(512, 126464) == 0            # one (wider) workgroup per row
    assert L.dllm_vocab_stats_workspace(64, 126464) > 0              # rows split across workgroups
    # 8 sequences x 12 KV heads, one 32-row group each: 8-wave workgroups, no key split
    desc = dl._KVCache(B=8, L=1024, n_kv_heads=12, d_head=64, dtype=1, k=16, v=16)
    assert L.dllm_block_attention_workspace(ctypes.byref(desc), 1, 12, 32, 1024) == 0
    # 4 sequences x 8 KV heads x 256 grouped rows: one workgroup per KV head
    # shares each tile, and the keys split over 8 workgroups
    desc = dl._KVCache(B=4, L=32768, n_kv_heads=8, d_head=128, dtype=2, k=16, v=16, k_scale=16,
                       v_scale=16)
    assert L.dllm_block_attention_workspace(ctypes.byref(desc), 1, 32, 64, 8192) == 8 * 4 * 32 * 64 * 130 * 4
    # FACache merge at a LLaDA-shaped step: 16 x 32 heads x 2016 queries
    # outside the block over the 32 block keys, one tile per workgroup
    desc = dl._KVCache(B=16, L=2048, n_kv_heads=32, d_head=128, dtype=1, k=16, v=16)
    assert L.dllm_facache_merge_workspace(ctypes.byref(desc), 1, 32, 2016, 32) == 0


def test_host_policies_match_the_oracle(dl, orc):
    """refresh interval and quotas are host arithmetic: equal to the oracle's"""
    import numpy as np
    for T in list(range(0, 130)) + [400, 4096]:
        assert dl.dllm_refresh_interval(T) == orc.refresh_interval(T), T
    for w0, w1, T in [(16, 2, 64), (8, 4, 10), (4, 4, 3), (16, 2, 1)]:
        for step in range(T + 3):
            assert dl.dllm_parallel_width(w0, w1, T, step) == orc.parallel_width(w0, w1, T, step)
    rng = np.random.default_rng(3)
    for trial in range(200):
        lens = rng.integers(0, 300, size=int(rng.integers(1, 9)))
        frac = float(rng.choice([0.0, 0.2, 0.5, 1.0]))
        need = int(np.minimum(np.ceil(frac * lens), lens).sum())
        budget = int(rng.integers(max(0, need - 20), lens.sum() + 50))
        try:
            ref = orc.cache_quotas(lens, budget, min_frac=frac)
        except ValueError:
            with pytest.raises(dl.DllmError):
                dl.dllm_cache_quotas(lens, budget, frac)
            continue
        assert np.array_equal(dl.dllm_cache_quotas(lens, budget, frac), ref), trial


def test_confidence_decay_table(dl, orc):
    """the host table is exp(-lambda k) from the C library, the same function
    the oracle's confidence calls: equal bit for bit to Python's math.exp of
    the same float64 product, with bad arguments rejected"""
    import math

    import numpy as np
    for lam in (3.0 / 16, 3.0 / 64, 0.25, 0.0, 1e-3, 7.5):
        t = dl.dllm_confidence_decay(lam, 300).numpy()
        ref = np.array([math.exp(-lam * float(k)) for k in range(300)])
        assert np.array_equal(t.view(np.uint64), ref.view(np.uint64)), lam
        assert t[0] == 1.0 and (np.diff(t) <= 0).all()
    L = dl.lib()
    buf = (ctypes.c_double * 4)()
    assert L.dllm_confidence_decay(0.1, 0, buf) == -1
    assert L.dllm_confidence_decay(-0.1, 4, buf) == -1
    assert L.dllm_confidence_decay(float("nan"), 4, buf) == -1
    assert L.dllm_confidence_decay(float("inf"), 4, buf) == -1
    assert L.dllm_confidence_decay(0.1, 4, None) == -1


def test_noalloc_scratch_limit(dl):
    """the allocation-free call rejects, on the host, a call whose key-split
    partials exceed the library's per-GPU scratch"""
    L = dl.lib()
    desc = dl._KVCache(B=1, L=200000, n_kv_heads=8, d_head=128, dtype=2, k=16, v=16, k_scale=16, v_scale=16)
    need = L.dllm_block_attention_workspace(ctypes.byref(desc), 1, 32, 64, 131072)
    assert need > dl.NOALLOC_SCRATCH_BYTES
    assert L.dllm_scatter_attention_noalloc(ctypes.byref(desc), 16, 16, 1, 16, 64, None, 16, 1, 32, 64, 16,
                                            131072, 0.0, 16, 1, None, None) == -5
    # argument errors are those of dllm_scatter_attention
    assert L.dllm_scatter_attention_noalloc(ctypes.byref(desc), 16, 16, 7, 16, 64, None, 16, 1, 32, 64, 16,
                                            131072, 0.0, 16, 1, None, None) == -2
    assert L.dllm_scatter_attention_noalloc(ctypes.byref(desc), 16, 16, 1, 16, 64, None, None, 1, 32, 64, 16,
                                            131072, 0.0, 16, 1, None, None) == -1


def test_workspace_size_dispatches_to_each_query(dl):
    L = dl.lib()
    gqa = dl._KVCache(B=4, L=32768, n_kv_heads=8, d_head=128, dtype=2, k=16, v=16, k_scale=16,
                      v_scale=16)
    mha = dl._KVCache(B=16, L=2048, n_kv_heads=32, d_head=128, dtype=1, k=16, v=16)
    ref = dl.Cache(gqa, None, None, None, None)
    for desc, Hq, n_q, n_keys in [(gqa, 32, 64, 8192), (gqa, 32, 7, 100), (mha, 32, 32, 2048),
                                  (mha, 32, 2016, 32), (mha, 30, 32, 2048), (mha, 32, 0, 2048)]:
        c = dl.Cache(desc, None, None, None, None)
        want = L.dllm_block_attention_workspace(ctypes.byref(desc), 1, Hq, n_q, n_keys)
        assert dl.dllm_workspace_size(dl.WS_BLOCK_ATTENTION, c, dl.BF16, Hq, n_q, n_keys) == want
        want = L.dllm_facache_merge_workspace(ctypes.byref(desc), 1, Hq, n_q, n_keys)
        assert dl.dllm_workspace_size(dl.WS_FACACHE_MERGE, c, dl.BF16, Hq, n_q, n_keys) == want
    assert dl.dllm_workspace_size(dl.WS_BLOCK_ATTENTION, ref, dl.BF16, 32, 64, 8192) > 0
    for N, V in [(64, 126464), (512, 126464), (8192, 50257), (0, 7), (3, 0)]:
        assert dl.dllm_workspace_size(dl.WS_VOCAB_STATS, N=N, V=V) == L.dllm_vocab_stats_workspace(N, V)
    assert dl.dllm_workspace_size(dl.WS_VOCAB_STATS, N=64, V=126464) > 0
    # an unknown kind, a missing cache and a NULL argument block answer 0
    assert dl.dllm_workspace_size(3, ref, dl.BF16, 32, 64, 8192) == 0
    assert dl.dllm_workspace_size(dl.WS_BLOCK_ATTENTION, None, dl.BF16, 32, 64, 8192) == 0
    assert L.dllm_workspace_size(dl.WS_VOCAB_STATS, None) == 0
