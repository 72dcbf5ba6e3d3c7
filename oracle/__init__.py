"""Plain fp64 CPU oracle for one step of cached masked-diffusion decoding.

TEST INFRASTRUCTURE ONLY.  The tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` are the only callers.  The product path
(``cached_denoising_amd``) never imports this package, and this package never
imports the product; the two meet only at the seeded input generators in
``workloads``.

The arithmetic lives in ``oracle.c`` (C11, IEEE binary64, no FMA contraction,
no fast-math).  This module only marshals numpy arrays into it.  Storage
formats: float32 arrays as ``np.float32``, bfloat16 as raw ``np.uint16`` bits,
OCP e4m3fn codes as ``np.uint8`` with float32 per-128-group scales.

Citations name the page and its section:
  [SWD]     Stable Window Decoding blog page (wmrh.cn/news/51151)
  [LaCache] "LaCache: Exact Caching and Precision-Adaptive Inference for
            Diffusion Large Language Models" (gist.science explainer)
  [Sinks]   attention-sinks / rolling K/V cache blog page (wmrh.cn/news/159578)
  [Flash]   Flash-dLLM page: I/O-aware KV cache and self-verifying parallel
            decoding (bjdmk.com.cn/news/5926815)
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

F32, BF16, E4M3 = 0, 1, 2
F64 = 9                      # oracle-only: rows of float64 values (fp8_quant_rows)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SOURCES = [os.path.join(_HERE, "oracle.c")]
GCC_FLAGS = ["-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
             "-fno-unsafe-math-optimizations", "-shared", "-fPIC", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    """Compile ``liboracle.so`` with gcc (always recompiles)."""
    cmd = ["gcc", *GCC_FLAGS, "-o", LIB_PATH + ".tmp", *SOURCES, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    global _lib
    _lib = None
    return LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        i32, i64, dbl = ctypes.c_int, ctypes.c_int64, ctypes.c_double
        L.oracle_set_threads.argtypes = [i32]
        L.oracle_set_threads.restype = i32
        L.oracle_get_threads.restype = i32
        L.oracle_bf16_value.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_value.restype = dbl
        L.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_value.restype = dbl
        L.oracle_e4m3_encode.argtypes = [ctypes.c_float]
        L.oracle_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_e4m3_quantize_group.argtypes = [P, i32, P, P]
        L.oracle_scatter_kv.argtypes = [i32, i32, i32, i32, i32, P, P, P, P, i32, P, P, P, i32]
        L.oracle_scatter_kv.restype = i32
        L.oracle_check_positions.argtypes = [i32, i32, P, i32, P, P]
        L.oracle_check_positions.restype = i32
        L.oracle_sink_rolling_keys.argtypes = [i32, i32, i32, P]
        L.oracle_sink_rolling_keys.restype = i32
        L.oracle_block_attention.argtypes = [i32, i32, i32, i32, i32, P, P, P, P, i32, P, i32, i32,
                                             P, i32, dbl, P, P, P, i32]
        L.oracle_block_attention.restype = i32
        L.oracle_facache_merge.argtypes = [i32, i32, i32, i32, i32, P, P, P, P, i32, P, i32, i32,
                                           P, P, P, i32, dbl, P, P, P, i32]
        L.oracle_facache_merge.restype = i32
        L.oracle_e8m0_exponent.argtypes = [dbl]
        L.oracle_e8m0_exponent.restype = i32
        L.oracle_e8m0_value.argtypes = [ctypes.c_uint8]
        L.oracle_e8m0_value.restype = dbl
        L.oracle_fp8_quantize_pow2.argtypes = [P, i32, P, P]
        L.oracle_fp8_quant_rows.argtypes = [i32, P, i64, i32, i64, P, P]
        L.oracle_fp8_quant_rows.restype = i32
        L.oracle_fp8_quant_weight.argtypes = [i32, P, i32, i32, P, P]
        L.oracle_fp8_quant_weight.restype = i32
        L.oracle_fp8_gemm.argtypes = [P, P, P, P, i64, i32, i32, P, i64, P]
        L.oracle_fp8_gemm.restype = i32
        L.oracle_addnorm.argtypes = [i32, P, P, P, dbl, i64, i32, P, P]
        L.oracle_addnorm.restype = i32
        L.oracle_silu.argtypes = [dbl]
        L.oracle_silu.restype = dbl
        L.oracle_swiglu.argtypes = [P, P, i64, P]
        L.oracle_vocab_stats.argtypes = [i32, P, i64, i64, i64, P, P, P, P, i64]
        L.oracle_vocab_stats.restype = i32
        L.oracle_stability_step.argtypes = [i32, i32, i32, P, i32, P, P, P, P, P, P, P, P, P,
                                            i32, dbl, i32, i32, dbl, dbl, dbl, i32, dbl, i64,
                                            i32, i32, i32, P, P, P, P, P]
        L.oracle_dynamic_radius.argtypes = [i32, i32, i32, i32]
        L.oracle_dynamic_radius.restype = i32
        L.oracle_is_refresh_step.argtypes = [i32, i32]
        L.oracle_is_refresh_step.restype = i32
        L.oracle_refresh_interval.argtypes = [i32]
        L.oracle_refresh_interval.restype = i32
        L.oracle_cache_quotas.argtypes = [i32, P, i64, dbl, P]
        L.oracle_cache_quotas.restype = i32
        L.oracle_evict_by_confidence.argtypes = [i32, i32, P, P, P, i32, P, P, P, P, P]
        L.oracle_evict_by_confidence.restype = i32
        L.oracle_stability_step.restype = i32
        L.oracle_parallel_width.argtypes = [i32, i32, i32, i32]
        L.oracle_parallel_width.restype = i32
        L.oracle_self_verify.argtypes = [i32, i32, P, i32, P, P, i32, dbl, P, P, P, P, P, P, P, P]
        L.oracle_self_verify.restype = i32
        _lib = L
    return _lib


def _ptr(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what}: bad argument (rc={rc})")


def set_threads(n: int) -> int:
    return lib().oracle_set_threads(int(n))


def get_threads() -> int:
    return lib().oracle_get_threads()


# ---- number formats ---------------------------------------------------------

def bf16_value(bits: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return np.array([lib().oracle_bf16_value(int(b)) for b in bits.ravel()]).reshape(bits.shape)


def e4m3_value(codes) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    return np.array([lib().oracle_e4m3_value(int(c)) for c in codes.ravel()]).reshape(codes.shape)


def e4m3_encode(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    f = lib().oracle_e4m3_encode
    return np.array([f(float(v)) for v in x.ravel()], dtype=np.uint8).reshape(x.shape)


def e4m3_quantize_group(x):
    x = np.ascontiguousarray(x, dtype=np.float32)
    codes = np.zeros(x.shape, dtype=np.uint8)
    scale = np.zeros(1, dtype=np.float32)
    lib().oracle_e4m3_quantize_group(_ptr(x), x.size, _ptr(codes), _ptr(scale))
    return codes, float(scale[0])


# ---- A1 ---------------------------------------------------------------------

def scatter_kv(cache_k, cache_v, k_scale, v_scale, cache_dtype, k_new, v_new, src_dtype, pos):
    """In-place: cache[b, h, pos[b, j], :] = new[b, j, h, :] (quantized for e4m3)."""
    B, Hkv, L, d = cache_k.shape
    n = pos.shape[1]
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    rc = lib().oracle_scatter_kv(cache_dtype, B, L, Hkv, d, _ptr(cache_k), _ptr(cache_v),
                                 _ptr(k_scale), _ptr(v_scale), src_dtype,
                                 _ptr(np.ascontiguousarray(k_new)), _ptr(np.ascontiguousarray(v_new)),
                                 _ptr(pos), n)
    _check(rc, "scatter_kv")


# ---- A2 ---------------------------------------------------------------------

def check_positions(L: int, pos):
    """(bad, dup) per sequence of pos [B, n] int32: entries outside [0, L)
    other than -1, and entries repeating an earlier entry."""
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    B, n = pos.shape
    bad = np.zeros(B, np.int32)
    dup = np.zeros(B, np.int32)
    _check(lib().oracle_check_positions(B, int(L), _ptr(pos), n, _ptr(bad), _ptr(dup)), "check_positions")
    return bad, dup


def sink_rolling_keys(S: int, R: int, end: int) -> np.ndarray:
    out = np.zeros(S + R, dtype=np.int32)
    k = lib().oracle_sink_rolling_keys(S, R, end, _ptr(out))
    if k < 0:
        raise ValueError("oracle sink_rolling_keys: bad argument")
    return out[:k].copy()


# ---- A3 ---------------------------------------------------------------------

def block_attention(cache_k, cache_v, k_scale, v_scale, cache_dtype, q, q_dtype,
                    key_idx=None, scale=0.0, heads=None):
    """softmax(q K^T * scale) V over the selected keys, fp64.

    Returns (out [B, Hq, b, d], lse [B, Hq, b]) or, with ``heads`` (an
    [n, 2] array of (batch, query-head) pairs), ([n, b, d], [n, b]).
    """
    B, Hkv, L, d = cache_k.shape
    _, Hq, b, _ = q.shape
    q = np.ascontiguousarray(q)
    if key_idx is not None:
        key_idx = np.ascontiguousarray(key_idx, dtype=np.int32)
        n_keys = key_idx.shape[1]
    else:
        n_keys = L
    if heads is not None:
        heads = np.ascontiguousarray(heads, dtype=np.int32).reshape(-1, 2)
        out = np.zeros((heads.shape[0], b, d))
        lse = np.zeros((heads.shape[0], b))
        nh = heads.shape[0]
    else:
        out = np.zeros((B, Hq, b, d))
        lse = np.zeros((B, Hq, b))
        nh = 0
    rc = lib().oracle_block_attention(cache_dtype, B, L, Hkv, d, _ptr(cache_k), _ptr(cache_v),
                                      _ptr(k_scale), _ptr(v_scale), q_dtype, _ptr(q), Hq, b,
                                      _ptr(key_idx), n_keys, float(scale), _ptr(out), _ptr(lse),
                                      _ptr(heads), nh)
    _check(rc, "block_attention")
    return out, lse


# ---- N1 ---------------------------------------------------------------------

def facache_key_maps(L: int, b: int, start) -> tuple[np.ndarray, np.ndarray]:
    """Unchanged and changed key positions of a SAR step, per sequence.

    [LaCache, problem statement and Methodology 1]: within one block's
    denoising steps the prompt and the masked suffix keep their token ids,
    only the active block [start, start + b) changes.  Returns
    (unchanged [B, L - b], block [B, b]), both ascending int32.
    """
    start = np.asarray(start, dtype=np.int64).reshape(-1)
    B = start.size
    un = np.zeros((B, L - b), dtype=np.int32)
    blk = np.zeros((B, b), dtype=np.int32)
    for i, o in enumerate(start):
        if not 0 <= o <= L - b:
            raise ValueError("oracle facache_key_maps: block outside the sequence")
        allpos = np.arange(L)
        inside = (allpos >= o) & (allpos < o + b)
        un[i] = allpos[~inside]
        blk[i] = allpos[inside]
    return un, blk


def facache_merge(cache_k, cache_v, k_scale, v_scale, cache_dtype, q, q_dtype, memo_o, memo_lse,
                  key_idx=None, scale=0.0, heads=None):
    """Memoized state (memo_o = O~/l, memo_lse = m + ln l) continued over the
    listed keys, then normalised, fp64.  Shapes and ``heads`` as in
    ``block_attention`` with b = n_q; memo_o [B, Hq, n_q, d] and memo_lse
    [B, Hq, n_q] are float32.
    """
    B, Hkv, L, d = cache_k.shape
    _, Hq, n_q, _ = q.shape
    q = np.ascontiguousarray(q)
    memo_o = np.ascontiguousarray(memo_o, dtype=np.float32)
    memo_lse = np.ascontiguousarray(memo_lse, dtype=np.float32)
    assert memo_o.shape == (B, Hq, n_q, d) and memo_lse.shape == (B, Hq, n_q)
    if key_idx is not None:
        key_idx = np.ascontiguousarray(key_idx, dtype=np.int32)
        n_keys = key_idx.shape[1]
    else:
        n_keys = L
    if heads is not None:
        heads = np.ascontiguousarray(heads, dtype=np.int32).reshape(-1, 2)
        nh = heads.shape[0]
        out = np.zeros((nh, n_q, d))
        lse = np.zeros((nh, n_q))
    else:
        nh = 0
        out = np.zeros((B, Hq, n_q, d))
        lse = np.zeros((B, Hq, n_q))
    rc = lib().oracle_facache_merge(cache_dtype, B, L, Hkv, d, _ptr(cache_k), _ptr(cache_v),
                                    _ptr(k_scale), _ptr(v_scale), q_dtype, _ptr(q), Hq, n_q,
                                    _ptr(memo_o), _ptr(memo_lse), _ptr(key_idx), n_keys,
                                    float(scale), _ptr(out), _ptr(lse), _ptr(heads), nh)
    _check(rc, "facache_merge")
    return out, lse


# ---- N2 ---------------------------------------------------------------------

def e8m0_exponent(amax: float) -> int:
    """smallest e >= -127 with amax <= 448 * 2^e [LaCache, Methodology 2;
    power-of-two group scales are a reading]"""
    return lib().oracle_e8m0_exponent(float(amax))


def e8m0_value(code: int) -> float:
    return lib().oracle_e8m0_value(int(code))


def fp8_quantize_pow2(x):
    """one group: (codes uint8, e8m0 code)"""
    x = np.ascontiguousarray(x, dtype=np.float64)
    codes = np.zeros(x.size, dtype=np.uint8)
    sc = np.zeros(1, dtype=np.uint8)
    lib().oracle_fp8_quantize_pow2(_ptr(x), x.size, _ptr(codes), _ptr(sc))
    return codes, int(sc[0])


def fp8_quant_rows(x, dtype):
    """x: [M, K] float32, bfloat16 bits (uint16) or float64 (dtype F64);
    returns (codes [M, K] uint8, scales [K/128, M] uint8 E8M0)."""
    x = np.ascontiguousarray(x)
    M, K = x.shape
    codes = np.zeros((M, K), dtype=np.uint8)
    scales = np.zeros((K // 128, M), dtype=np.uint8)
    _check(lib().oracle_fp8_quant_rows(dtype, _ptr(x), M, K, K, _ptr(codes), _ptr(scales)), "fp8_quant_rows")
    return codes, scales


def fp8_quant_weight(w, dtype):
    """w: [N, K]; returns (codes [N, K], scales [N/128, K/128] E8M0)."""
    w = np.ascontiguousarray(w)
    N, K = w.shape
    codes = np.zeros((N, K), dtype=np.uint8)
    scales = np.zeros((N // 128, K // 128), dtype=np.uint8)
    _check(lib().oracle_fp8_quant_weight(dtype, _ptr(w), N, K, _ptr(codes), _ptr(scales)), "fp8_quant_weight")
    return codes, scales


def fp8_gemm(a, sa, b, sb, rows=None):
    """dequant(A) dequant(B)^T in fp64; rows selects output rows of A."""
    a, sa, b, sb = (np.ascontiguousarray(t, dtype=np.uint8) for t in (a, sa, b, sb))
    M, K = a.shape
    N = b.shape[0]
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        c = np.zeros((rows.size, N))
        n_rows = rows.size
    else:
        c = np.zeros((M, N))
        n_rows = 0
    _check(lib().oracle_fp8_gemm(_ptr(a), _ptr(sa), _ptr(b), _ptr(sb), M, N, K, _ptr(rows), n_rows, _ptr(c)),
           "fp8_gemm")
    return c


def addnorm(x, res, gamma, eps, dtype):
    """(res_out in dtype storage, y fp64 [M, K])"""
    x = np.ascontiguousarray(x)
    M, K = x.shape
    res = np.ascontiguousarray(res) if res is not None else None
    gamma = np.ascontiguousarray(gamma)
    res_out = np.zeros_like(x)
    y = np.zeros((M, K))
    _check(lib().oracle_addnorm(dtype, _ptr(x), _ptr(res), _ptr(gamma), float(eps), M, K, _ptr(res_out), _ptr(y)),
           "addnorm")
    return res_out, y


def silu(g: float) -> float:
    return lib().oracle_silu(float(g))


def swiglu(g, u):
    g = np.ascontiguousarray(g, dtype=np.float64)
    u = np.ascontiguousarray(u, dtype=np.float64)
    y = np.zeros_like(g)
    lib().oracle_swiglu(_ptr(g), _ptr(u), g.size, _ptr(y))
    return y


# ---- A4 ---------------------------------------------------------------------

def vocab_stats(logits, dtype, V=None, rows=None):
    """argmax (lowest index of the max), maxprob, entropy per row, fp64.

    ``logits`` is [N, stride] (f32, or uint16 bf16 bits); V <= stride is the
    vocabulary size (default: the full row).
    """
    logits = np.ascontiguousarray(logits)
    N, stride = logits.shape
    V = stride if V is None else V
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        n_out = rows.shape[0]
    else:
        n_out = N
    am = np.zeros(n_out, dtype=np.int32)
    mp = np.zeros(n_out)
    en = np.zeros(n_out)
    rc = lib().oracle_vocab_stats(dtype, _ptr(logits), N, V, stride, _ptr(am), _ptr(mp), _ptr(en),
                                  _ptr(rows), 0 if rows is None else n_out)
    _check(rc, "vocab_stats")
    return am, mp, en


# ---- A5-A7 ------------------------------------------------------------------

class StabilityState:
    """Per-sequence decode state: step-history ring plus sticky stable flags."""

    def __init__(self, B: int, L: int, D: int):
        self.B, self.L, self.D = B, L, D
        self.ring_argmax = np.zeros((D, B, L), dtype=np.int32)
        self.ring_maxprob = np.zeros((D, B, L), dtype=np.float32)
        self.ring_step = np.full((D, B, L), -1, dtype=np.int32)
        self.entropy_latest = np.zeros((B, L), dtype=np.float32)
        self.t_write = np.zeros((B, L), dtype=np.int32)
        self.stable = np.zeros((B, L), dtype=np.uint8)
        self.cached = np.zeros((B, L), dtype=np.uint8)      # positions holding K/V (N3 budget)

    def copy(self):
        c = StabilityState.__new__(StabilityState)
        c.B, c.L, c.D = self.B, self.L, self.D
        for k in ("ring_argmax", "ring_maxprob", "ring_step", "entropy_latest", "t_write", "stable",
                  "cached"):
            setattr(c, k, getattr(self, k).copy())
        return c


def stability_step(state: StabilityState, step, pos, argmax, maxprob, entropy, *, K, tau, R,
                   alpha=0.0, beta=0.0, lam=0.0, conf_thresh=0.0, V=2, R_early=0, T_steps=0,
                   refresh_every=0, n_decay=4096):
    """One step of history update, stability test, confidence and window mask.

    pos: [B, n] recomputed positions or None (all L).  argmax/maxprob/entropy
    are [B, n] (float32 maxprob/entropy).  The confidence's age s - t_write is
    clamped to [0, n_decay - 1].  Returns dict with mask, conf (float64),
    next_pos, count, all_stable.  ``state`` is updated in place.
    """
    B, L, D = state.B, state.L, state.D
    if pos is not None:
        pos = np.ascontiguousarray(pos, dtype=np.int32)
        n = pos.shape[1]
    else:
        n = L
    argmax = np.ascontiguousarray(argmax, dtype=np.int32).reshape(B, n)
    maxprob = np.ascontiguousarray(maxprob, dtype=np.float32).reshape(B, n)
    entropy = np.ascontiguousarray(entropy, dtype=np.float32).reshape(B, n)
    mask = np.zeros((B, L), dtype=np.uint8)
    conf = np.zeros((B, L))
    next_pos = np.zeros((B, L), dtype=np.int32)
    count = np.zeros(B, dtype=np.int32)
    all_stable = np.zeros(B, dtype=np.uint8)
    rc = lib().oracle_stability_step(B, L, int(step), _ptr(pos), n, _ptr(argmax), _ptr(maxprob),
                                     _ptr(entropy), _ptr(state.ring_argmax), _ptr(state.ring_maxprob),
                                     _ptr(state.ring_step), _ptr(state.entropy_latest),
                                     _ptr(state.t_write), _ptr(state.stable), int(K), float(tau), D,
                                     int(R), float(alpha), float(beta), float(lam), int(n_decay),
                                     float(conf_thresh), int(V), int(R_early), int(T_steps),
                                     int(refresh_every), _ptr(mask), _ptr(conf),
                                     _ptr(next_pos), _ptr(count), _ptr(all_stable))
    _check(rc, "stability_step")
    return dict(mask=mask, conf=conf, next_pos=next_pos, count=count, all_stable=all_stable)


# ---- N3 ---------------------------------------------------------------------

def dynamic_radius(R_early: int, R: int, T: int, step: int) -> int:
    return lib().oracle_dynamic_radius(int(R_early), int(R), int(T), int(step))


def is_refresh_step(F: int, step: int) -> bool:
    return bool(lib().oracle_is_refresh_step(int(F), int(step)))


def refresh_interval(T: int) -> int:
    return lib().oracle_refresh_interval(int(T))


def cache_quotas(lens, budget: int, min_frac: float = 0.2):
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    q = np.zeros(lens.size, dtype=np.int32)
    _check(lib().oracle_cache_quotas(lens.size, _ptr(lens), int(budget), float(min_frac), _ptr(q)),
           "cache_quotas")
    return q


def evict_by_confidence(state: StabilityState, conf, quota, pos, mask):
    """In place on state.cached and mask (uint8 [B, L]); conf float32
    [B, L]; quota int32 [B].  Returns dict(next_pos, count, evicted)."""
    B, L = state.B, state.L
    conf = np.ascontiguousarray(conf, dtype=np.float32)
    quota = np.ascontiguousarray(quota, dtype=np.int32)
    if pos is not None:
        pos = np.ascontiguousarray(pos, dtype=np.int32)
        n = pos.shape[1]
    else:
        n = L
    assert mask.dtype == np.uint8 and mask.flags["C_CONTIGUOUS"]
    next_pos = np.zeros((B, L), dtype=np.int32)
    count = np.zeros(B, dtype=np.int32)
    evicted = np.zeros(B, dtype=np.int32)
    _check(lib().oracle_evict_by_confidence(B, L, _ptr(conf), _ptr(quota), _ptr(pos), n, _ptr(state.cached),
                                            _ptr(mask), _ptr(next_pos), _ptr(count), _ptr(evicted)),
           "evict_by_confidence")
    return dict(next_pos=next_pos, count=count, evicted=evicted)


def parallel_width(w_early: int, w_late: int, T: int, step: int) -> int:
    return lib().oracle_parallel_width(int(w_early), int(w_late), int(T), int(step))


def self_verify(L: int, dec_pos, p_marg, p_joint, W: int, tau: float, mask, stable=None, cached=None):
    """Self-verification of one step's parallel decodes.  dec_pos int32 [B, n]
    (-1 padding), p_marg float32 [B, n], p_joint float32 [B, n, W-1]; mask,
    stable, cached uint8 [B, L] are updated in place.  Returns dict(rollback,
    next_pos, count, n_rollback, rb_pos)."""
    dec_pos = np.ascontiguousarray(dec_pos, dtype=np.int32)
    B, n = dec_pos.shape
    p_marg = np.ascontiguousarray(p_marg, dtype=np.float32).reshape(B, n)
    p_joint = np.ascontiguousarray(p_joint, dtype=np.float32).reshape(B, n, W - 1)
    for a in (mask, stable, cached):
        assert a is None or (a.dtype == np.uint8 and a.flags["C_CONTIGUOUS"] and a.shape == (B, L))
    rollback = np.zeros((B, L), dtype=np.uint8)
    next_pos = np.zeros((B, L), dtype=np.int32)
    count = np.zeros(B, dtype=np.int32)
    n_rb = np.zeros(B, dtype=np.int32)
    rb_pos = np.zeros((B, n), dtype=np.int32)
    _check(lib().oracle_self_verify(B, L, _ptr(dec_pos), n, _ptr(p_marg), _ptr(p_joint), int(W), float(tau),
                                    _ptr(rollback), _ptr(mask), _ptr(stable), _ptr(cached), _ptr(next_pos),
                                    _ptr(count), _ptr(n_rb), _ptr(rb_pos)), "self_verify")
    return dict(rollback=rollback, next_pos=next_pos, count=count, n_rollback=n_rb, rb_pos=rb_pos)
