"""Python binding of libdllm, the MI355X (gfx950) hot path of cached
masked-diffusion decoding.

Argument marshalling only: every step runs in the HIP kernels behind the C
ABI declared in ``include/dllm.h``.  PyTorch supplies device memory and the
current stream.  The functions keep the C names.  There is no fallback: if
``libdllm.so`` is missing or a tensor is not on a GPU, a call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "F32", "BF16", "E4M3", "DllmError", "lib", "Cache", "StabilityState", "dllm_status_str",
    "dllm_version", "dllm_cache_init", "dllm_scatter_kv", "dllm_sink_rolling_map",
    "dllm_block_attention", "dllm_block_attention_workspace", "dllm_scatter_attention",
    "dllm_facache_maps",
    "dllm_facache_merge", "dllm_facache_merge_workspace", "dllm_fp8_quant_rows",
    "dllm_fp8_addnorm_quant", "dllm_fp8_quant_weight", "dllm_fp8_gemm", "dllm_fp8_gemm_swiglu",
    "dllm_vocab_stats",
    "dllm_vocab_stats_workspace", "dllm_stability_reset", "dllm_stability_mask",
    "dllm_refresh_interval", "dllm_cache_quotas", "dllm_evict_by_confidence",
    "dllm_parallel_width", "dllm_self_verify", "dllm_confidence_decay", "dllm_check_positions",
    "dllm_scatter_attention_noalloc", "NOALLOC_SCRATCH_BYTES", "dllm_workspace_size",
    "WS_BLOCK_ATTENTION", "WS_FACACHE_MERGE", "WS_VOCAB_STATS",
]

F32, BF16, E4M3 = 0, 1, 2
WS_BLOCK_ATTENTION, WS_FACACHE_MERGE, WS_VOCAB_STATS = 0, 1, 2   # dllm_workspace_kind
NOALLOC_SCRATCH_BYTES = 64 << 20      # DLLM_NOALLOC_SCRATCH_BYTES of include/dllm.h
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdllm.so")


class DllmError(RuntimeError):
    pass


class _KVCache(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("L", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("d_head", ctypes.c_int32), ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("k_scale", ctypes.c_void_p),
                ("v_scale", ctypes.c_void_p)]


class _StabParams(ctypes.Structure):
    _fields_ = [("K", ctypes.c_int32), ("D", ctypes.c_int32), ("R", ctypes.c_int32),
                ("advance_step", ctypes.c_int32), ("tau", ctypes.c_double), ("alpha", ctypes.c_double),
                ("beta", ctypes.c_double), ("conf_thresh", ctypes.c_double),
                ("decay", ctypes.c_void_p), ("vocab", ctypes.c_int64),
                ("R_early", ctypes.c_int32), ("T_steps", ctypes.c_int32),
                ("refresh_every", ctypes.c_int32), ("n_decay", ctypes.c_int32)]


class _WsArgs(ctypes.Structure):
    _fields_ = [("cache", ctypes.POINTER(_KVCache)), ("q_dtype", ctypes.c_int32),
                ("Hq", ctypes.c_int32), ("n_q", ctypes.c_int32), ("n_keys", ctypes.c_int32),
                ("N", ctypes.c_int64), ("V", ctypes.c_int64)]


EXPORTS = {
    # name: (restype, argtypes)
    "dllm_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "dllm_version": (ctypes.c_int, []),
    "dllm_cache_init": (ctypes.c_int, [ctypes.POINTER(_KVCache), ctypes.c_int, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p]),
    "dllm_scatter_kv": (ctypes.c_int, [ctypes.POINTER(_KVCache), ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                       ctypes.c_void_p]),
    "dllm_sink_rolling_map": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                             ctypes.c_void_p]),
    "dllm_block_attention": (ctypes.c_int, [ctypes.POINTER(_KVCache), ctypes.c_void_p, ctypes.c_int,
                                            ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                            ctypes.c_int, ctypes.c_float, ctypes.c_void_p,
                                            ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_size_t, ctypes.c_void_p]),
    "dllm_scatter_attention": (ctypes.c_int, [ctypes.POINTER(_KVCache), ctypes.c_void_p,
                                              ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                              ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                              ctypes.c_void_p, ctypes.c_int, ctypes.c_float,
                                              ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                              ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "dllm_scatter_attention_noalloc": (ctypes.c_int, [ctypes.POINTER(_KVCache), ctypes.c_void_p,
                                                      ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                                      ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                                      ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                      ctypes.c_void_p, ctypes.c_int, ctypes.c_float,
                                                      ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                                      ctypes.c_void_p]),
    "dllm_block_attention_workspace": (ctypes.c_size_t, [ctypes.POINTER(_KVCache), ctypes.c_int,
                                                         ctypes.c_int, ctypes.c_int, ctypes.c_int]),
    "dllm_facache_maps": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "dllm_facache_merge": (ctypes.c_int, [ctypes.POINTER(_KVCache), ctypes.c_void_p, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
                                          ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "dllm_facache_merge_workspace": (ctypes.c_size_t, [ctypes.POINTER(_KVCache), ctypes.c_int,
                                                       ctypes.c_int, ctypes.c_int, ctypes.c_int]),
    "dllm_fp8_quant_rows": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                           ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_void_p]),
    "dllm_fp8_addnorm_quant": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.c_int, ctypes.c_float, ctypes.c_int64, ctypes.c_int,
                                              ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.c_void_p]),
    "dllm_fp8_quant_weight": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "dllm_fp8_gemm": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                     ctypes.c_void_p]),
    "dllm_fp8_gemm_swiglu": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "dllm_vocab_stats": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                        ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_size_t, ctypes.c_void_p]),
    "dllm_vocab_stats_workspace": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int64]),
    "dllm_workspace_size": (ctypes.c_size_t, [ctypes.c_int, ctypes.POINTER(_WsArgs)]),
    "dllm_stability_reset": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_void_p]),
    "dllm_stability_mask": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.POINTER(_StabParams), ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_void_p]),
    "dllm_refresh_interval": (ctypes.c_int, [ctypes.c_int]),
    "dllm_confidence_decay": (ctypes.c_int, [ctypes.c_double, ctypes.c_int, ctypes.c_void_p]),
    "dllm_check_positions": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
                                            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "dllm_cache_quotas": (ctypes.c_int, [ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_double,
                                         ctypes.c_void_p]),
    "dllm_evict_by_confidence": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "dllm_parallel_width": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int]),
    "dllm_self_verify": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_double,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
}

_lib = None


def lib():
    """Load libdllm.so (built in-tree by ``build()``); raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise DllmError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def dllm_status_str(status: int) -> str:
    return lib().dllm_status_str(status).decode()


def dllm_version() -> int:
    return lib().dllm_version()


def _check(rc: int, fn: str):
    if rc != 0:
        raise DllmError(f"{fn}: {dllm_status_str(rc)} ({rc})")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return E4M3
    raise DllmError(f"unsupported tensor dtype {t.dtype}")


def _dev(t: Optional[torch.Tensor], name: str, contiguous: bool = True):
    if t is None:
        return None
    if not t.is_cuda:
        raise DllmError(f"{name} must be a GPU tensor")
    if contiguous and not t.is_contiguous():
        raise DllmError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


_I32 = (torch.int32,)
_FLOAT = (torch.float32, torch.bfloat16)
_CODES = (torch.uint8, torch.float8_e4m3fn)


def _want(t: Optional[torch.Tensor], name: str, shape=None, dtypes=None, numel=None,
          required: bool = True):
    """Shape and dtype checks of a tensor argument, before any pointer
    reaches the library: a mismatch raises instead of letting a kernel read
    or write past a buffer."""
    if t is None:
        if required:
            raise DllmError(f"{name} is required")
        return
    if not isinstance(t, torch.Tensor):
        raise DllmError(f"{name} must be a torch.Tensor")
    if dtypes is not None and t.dtype not in dtypes:
        raise DllmError(f"{name}: dtype {t.dtype}, expected one of {[str(d) for d in dtypes]}")
    if shape is not None and tuple(t.shape) != tuple(int(x) for x in shape):
        raise DllmError(f"{name}: shape {tuple(t.shape)}, expected {tuple(int(x) for x in shape)}")
    if numel is not None and t.numel() != int(numel):
        raise DllmError(f"{name}: {t.numel()} elements, expected {int(numel)}")


_CACHE_TORCH = {F32: (torch.float32,), BF16: (torch.bfloat16,), E4M3: _FLOAT}


def _want_rows(cache, k_new, v_new, pos):
    """fresh rows [B, n, Hkv, d] in the cache's source dtype, positions [B, n] int32"""
    B, Hkv, d = cache.desc.B, cache.desc.n_kv_heads, cache.desc.d_head
    _want(pos, "pos", dtypes=_I32)
    if pos.dim() != 2 or pos.shape[0] != B:
        raise DllmError(f"pos: shape {tuple(pos.shape)}, expected [{B}, n]")
    n = pos.shape[1]
    _want(k_new, "k_new", (B, n, Hkv, d), _CACHE_TORCH[cache.desc.dtype])
    _want(v_new, "v_new", (B, n, Hkv, d), (k_new.dtype,))
    return n


def _want_queries(cache, q):
    _want(q, "q", dtypes=_FLOAT)
    if q.dim() != 4 or q.shape[0] != cache.desc.B or q.shape[3] != cache.desc.d_head:
        raise DllmError(f"q: shape {tuple(q.shape)}, expected [{cache.desc.B}, Hq, b, {cache.desc.d_head}]")
    if q.shape[1] % cache.desc.n_kv_heads != 0:
        raise DllmError(f"q: {q.shape[1]} query heads, not a multiple of {cache.desc.n_kv_heads} KV heads")
    return q.shape


def _want_key_map(cache, key_idx):
    if key_idx is None:
        return cache.desc.L
    _want(key_idx, "key_idx", dtypes=_I32)
    if key_idx.dim() != 2 or key_idx.shape[0] != cache.desc.B:
        raise DllmError(f"key_idx: shape {tuple(key_idx.shape)}, expected [{cache.desc.B}, n_keys]")
    return key_idx.shape[1]


def _want_out(out, lse, B, Hq, b, d):
    _want(out, "out", (B, Hq, b, d), _FLOAT)
    _want(lse, "lse", (B, Hq, b), (torch.float32,), required=False)


def _want_counter(t, name):
    _want(t, name, dtypes=_I32, required=False)
    if t is not None and t.numel() < 1:
        raise DllmError(f"{name} must hold at least one int32")


class Cache:
    """One layer's persistent K/V cache: the C descriptor plus the tensors it
    points to (kept alive here)."""

    def __init__(self, desc: _KVCache, k, v, k_scale, v_scale):
        self.desc, self.k, self.v, self.k_scale, self.v_scale = desc, k, v, k_scale, v_scale

    @property
    def dtype(self) -> int:
        return self.desc.dtype


def dllm_cache_init(k: torch.Tensor, v: torch.Tensor, dtype: Optional[int] = None,
                    k_scale: Optional[torch.Tensor] = None,
                    v_scale: Optional[torch.Tensor] = None) -> Cache:
    """k, v: [B, Hkv, L, d] GPU tensors (float32, bfloat16, or uint8 e4m3 codes
    with float32 scales [B, Hkv, L, d/128]).  Zero-fills them."""
    dtype = _dtype_code(k) if dtype is None else dtype
    B, H, L, d = k.shape
    desc = _KVCache()
    rc = lib().dllm_cache_init(ctypes.byref(desc), B, L, H, d, dtype, _dev(k, "k"), _dev(v, "v"),
                               _dev(k_scale, "k_scale"), _dev(v_scale, "v_scale"), _stream())
    _check(rc, "dllm_cache_init")
    return Cache(desc, k, v, k_scale, v_scale)


def dllm_scatter_kv(cache: Cache, k_new: torch.Tensor, v_new: torch.Tensor, pos: torch.Tensor,
                    bad_count: Optional[torch.Tensor] = None):
    """k_new, v_new: [B, n, Hkv, d]; pos: [B, n] int32 (-1 = padding)."""
    n = _want_rows(cache, k_new, v_new, pos)
    _want_counter(bad_count, "bad_count")
    rc = lib().dllm_scatter_kv(ctypes.byref(cache.desc), _dev(k_new, "k_new"), _dev(v_new, "v_new"),
                               _dtype_code(k_new), _dev(pos, "pos"), n, _dev(bad_count, "bad_count"),
                               _stream())
    _check(rc, "dllm_scatter_kv")


def dllm_sink_rolling_map(L: int, S: int, R: int, end: torch.Tensor, key_idx: torch.Tensor):
    """key_idx[b] = sinks [0, min(S, e)) then [max(S, e-R), e), -1 padded."""
    _want(key_idx, "key_idx", dtypes=_I32)
    if key_idx.dim() != 2:
        raise DllmError("key_idx must be [B, n_keys]")
    B, n_keys = key_idx.shape
    _want(end, "end", (B,), _I32)
    rc = lib().dllm_sink_rolling_map(B, L, S, R, _dev(end, "end"), _dev(key_idx, "key_idx"), n_keys,
                                     _stream())
    _check(rc, "dllm_sink_rolling_map")
    return key_idx


def dllm_block_attention_workspace(cache: Cache, q_dtype: int, Hq: int, b: int, n_keys: int) -> int:
    return lib().dllm_block_attention_workspace(ctypes.byref(cache.desc), q_dtype, Hq, b, n_keys)


def dllm_block_attention(cache: Cache, q: torch.Tensor, key_idx: Optional[torch.Tensor] = None,
                         scale: float = 0.0, out: Optional[torch.Tensor] = None,
                         out_dtype: Optional[torch.dtype] = None, lse: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None):
    """q: [B, Hq, b, d]; returns out [B, Hq, b, d] (and fills lse if given)."""
    B, Hq, b, d = _want_queries(cache, q)
    n_keys = _want_key_map(cache, key_idx)
    if out is None:
        out = torch.empty((B, Hq, b, d), dtype=out_dtype or q.dtype, device=q.device)
    _want_out(out, lse, B, Hq, b, d)
    ws_need = dllm_block_attention_workspace(cache, _dtype_code(q), Hq, b, n_keys)
    if workspace is None and ws_need:
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = lib().dllm_block_attention(ctypes.byref(cache.desc), _dev(q, "q"), _dtype_code(q), Hq, b,
                                    _dev(key_idx, "key_idx"), n_keys, float(scale), _dev(out, "out"),
                                    _dtype_code(out), _dev(lse, "lse"), _dev(workspace, "workspace"),
                                    ws_bytes, _stream())
    _check(rc, "dllm_block_attention")
    return out


def dllm_scatter_attention(cache: Cache, k_new: torch.Tensor, v_new: torch.Tensor, pos: torch.Tensor,
                           q: torch.Tensor, key_idx: Optional[torch.Tensor] = None, scale: float = 0.0,
                           out: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
                           lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                           bad_count: Optional[torch.Tensor] = None):
    """dllm_scatter_kv(cache, k_new, v_new, pos) then dllm_block_attention(cache,
    q, ...) in one call; returns out [B, Hq, b, d]."""
    B, Hq, b, d = _want_queries(cache, q)
    n = _want_rows(cache, k_new, v_new, pos)
    _want_counter(bad_count, "bad_count")
    n_keys = _want_key_map(cache, key_idx)
    if out is None:
        out = torch.empty((B, Hq, b, d), dtype=out_dtype or q.dtype, device=q.device)
    _want_out(out, lse, B, Hq, b, d)
    ws_need = dllm_block_attention_workspace(cache, _dtype_code(q), Hq, b, n_keys)
    if workspace is None and ws_need:
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = lib().dllm_scatter_attention(ctypes.byref(cache.desc), _dev(k_new, "k_new"), _dev(v_new, "v_new"),
                                      _dtype_code(k_new), _dev(pos, "pos"), n, _dev(bad_count, "bad_count"),
                                      _dev(q, "q"), _dtype_code(q), Hq, b, _dev(key_idx, "key_idx"), n_keys,
                                      float(scale), _dev(out, "out"), _dtype_code(out), _dev(lse, "lse"),
                                      _dev(workspace, "workspace"), ws_bytes, _stream())
    _check(rc, "dllm_scatter_attention")
    return out


def dllm_scatter_attention_noalloc(cache: Cache, k_new: torch.Tensor, v_new: torch.Tensor, pos: torch.Tensor,
                                   q: torch.Tensor, out: torch.Tensor, key_idx: Optional[torch.Tensor] = None,
                                   scale: float = 0.0, lse: Optional[torch.Tensor] = None,
                                   bad_count: Optional[torch.Tensor] = None):
    """dllm_scatter_attention without a workspace: the library's own per-GPU
    scratch holds the key-split partials, and nothing is allocated (the caller
    passes ``out``).  Calls that overlap on one GPU race on that scratch."""
    B, Hq, b, d = _want_queries(cache, q)
    n = _want_rows(cache, k_new, v_new, pos)
    _want_counter(bad_count, "bad_count")
    n_keys = _want_key_map(cache, key_idx)
    _want_out(out, lse, B, Hq, b, d)
    rc = lib().dllm_scatter_attention_noalloc(ctypes.byref(cache.desc), _dev(k_new, "k_new"), _dev(v_new, "v_new"),
                                              _dtype_code(k_new), _dev(pos, "pos"), n,
                                              _dev(bad_count, "bad_count"), _dev(q, "q"), _dtype_code(q), Hq, b,
                                              _dev(key_idx, "key_idx"), n_keys, float(scale), _dev(out, "out"),
                                              _dtype_code(out), _dev(lse, "lse"), _stream())
    _check(rc, "dllm_scatter_attention_noalloc")
    return out


def dllm_facache_maps(L: int, blk: int, start: torch.Tensor,
                      unchanged_idx: Optional[torch.Tensor] = None,
                      block_idx: Optional[torch.Tensor] = None):
    """start: [B] int32 block offsets; returns (unchanged_idx [B, L - blk],
    block_idx [B, blk]) int32."""
    _want(start, "start", dtypes=_I32)
    if start.dim() != 1:
        raise DllmError("start must be [B]")
    B = start.shape[0]
    if not 1 <= blk < L:
        raise DllmError(f"block length {blk} must be in [1, L) with L = {L}")
    if unchanged_idx is None:
        unchanged_idx = torch.empty((B, L - blk), dtype=torch.int32, device=start.device)
    if block_idx is None:
        block_idx = torch.empty((B, blk), dtype=torch.int32, device=start.device)
    _want(unchanged_idx, "unchanged_idx", (B, L - blk), _I32)
    _want(block_idx, "block_idx", (B, blk), _I32)
    rc = lib().dllm_facache_maps(B, L, blk, _dev(start, "start"), _dev(unchanged_idx, "unchanged_idx"),
                                 _dev(block_idx, "block_idx"), _stream())
    _check(rc, "dllm_facache_maps")
    return unchanged_idx, block_idx


def dllm_facache_merge_workspace(cache: Cache, q_dtype: int, Hq: int, n_q: int, n_keys: int) -> int:
    return lib().dllm_facache_merge_workspace(ctypes.byref(cache.desc), q_dtype, Hq, n_q, n_keys)


def dllm_facache_merge(cache: Cache, q: torch.Tensor, memo_o: torch.Tensor, memo_lse: torch.Tensor,
                       key_idx: Optional[torch.Tensor] = None, scale: float = 0.0,
                       out: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
                       lse: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None):
    """q: [B, Hq, n_q, d] queries outside the block; memo_o [B, Hq, n_q, d]
    and memo_lse [B, Hq, n_q] float32 (a dllm_block_attention output over the
    unchanged keys); key_idx: [B, n_keys] changed keys.  Returns out."""
    B, Hq, n_q, d = _want_queries(cache, q)
    if memo_o.dtype != torch.float32 or memo_lse.dtype != torch.float32:
        raise DllmError("memo_o and memo_lse must be float32")
    if tuple(memo_o.shape) != (B, Hq, n_q, d) or tuple(memo_lse.shape) != (B, Hq, n_q):
        raise DllmError("memo shapes must be [B, Hq, n_q, d] and [B, Hq, n_q]")
    n_keys = _want_key_map(cache, key_idx)
    if out is None:
        out = torch.empty((B, Hq, n_q, d), dtype=out_dtype or q.dtype, device=q.device)
    _want_out(out, lse, B, Hq, n_q, d)
    ws_need = dllm_facache_merge_workspace(cache, _dtype_code(q), Hq, n_q, n_keys)
    if workspace is None and ws_need:
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = lib().dllm_facache_merge(ctypes.byref(cache.desc), _dev(q, "q"), _dtype_code(q), Hq, n_q,
                                  _dev(key_idx, "key_idx"), n_keys, float(scale),
                                  _dev(memo_o, "memo_o"), _dev(memo_lse, "memo_lse"), _dev(out, "out"),
                                  _dtype_code(out), _dev(lse, "lse"), _dev(workspace, "workspace"),
                                  ws_bytes, _stream())
    _check(rc, "dllm_facache_merge")
    return out


def _u8(t: torch.Tensor, name: str):
    if t.dtype not in (torch.uint8, torch.float8_e4m3fn):
        raise DllmError(f"{name} must be uint8 codes")
    return _dev(t, name)


def dllm_fp8_quant_rows(x: torch.Tensor, codes: Optional[torch.Tensor] = None,
                        scales: Optional[torch.Tensor] = None):
    """x: [M, K] float32/bfloat16 (rows may be strided); returns (codes
    [M, K] uint8, scales [K/128, M] uint8 E8M0)."""
    _want(x, "x", dtypes=_FLOAT)
    if x.dim() != 2:
        raise DllmError("x must be [M, K]")
    M, K = x.shape
    if x.stride(1) != 1:
        raise DllmError("x rows must be contiguous")
    codes = torch.empty((M, K), dtype=torch.uint8, device=x.device) if codes is None else codes
    scales = torch.empty((K // 128, M), dtype=torch.uint8, device=x.device) if scales is None else scales
    _want(codes, "codes", (M, K), _CODES)
    _want(scales, "scales", (K // 128, M), _CODES)
    rc = lib().dllm_fp8_quant_rows(_dev(x, "x", contiguous=False), _dtype_code(x), M, K, x.stride(0),
                                   _u8(codes, "codes"), _u8(scales, "scales"), _stream())
    _check(rc, "dllm_fp8_quant_rows")
    return codes, scales


def dllm_fp8_addnorm_quant(x: torch.Tensor, residual: Optional[torch.Tensor], gamma: torch.Tensor,
                           eps: float = 1e-6, residual_out: Optional[torch.Tensor] = None,
                           codes: Optional[torch.Tensor] = None, scales: Optional[torch.Tensor] = None,
                           write_residual: bool = True):
    """r = x + residual (stored in residual_out), y = RMSNorm(r) * gamma,
    quantised per 1 x 128 group; returns (residual_out, codes, scales)."""
    _want(x, "x", dtypes=_FLOAT)
    if x.dim() != 2:
        raise DllmError("x must be [M, K]")
    M, K = x.shape
    dev = x.device
    _want(residual, "residual", (M, K), (x.dtype,), required=False)
    _want(gamma, "gamma", (K,), (x.dtype,))
    if write_residual and residual_out is None:
        residual_out = torch.empty_like(x)
    if write_residual:
        _want(residual_out, "residual_out", (M, K), (x.dtype,))
    codes = torch.empty((M, K), dtype=torch.uint8, device=dev) if codes is None else codes
    scales = torch.empty((K // 128, M), dtype=torch.uint8, device=dev) if scales is None else scales
    _want(codes, "codes", (M, K), _CODES)
    _want(scales, "scales", (K // 128, M), _CODES)
    rc = lib().dllm_fp8_addnorm_quant(_dev(x, "x"), _dev(residual, "residual"), _dev(gamma, "gamma"),
                                      _dtype_code(x), float(eps), M, K,
                                      _dev(residual_out, "residual_out") if write_residual else None,
                                      _u8(codes, "codes"), _u8(scales, "scales"), _stream())
    _check(rc, "dllm_fp8_addnorm_quant")
    return residual_out, codes, scales


def dllm_fp8_quant_weight(w: torch.Tensor, codes: Optional[torch.Tensor] = None,
                          scales: Optional[torch.Tensor] = None):
    """w: [N, K]; returns (codes [N, K], scales [N/128, K/128])."""
    _want(w, "w", dtypes=_FLOAT)
    if w.dim() != 2:
        raise DllmError("w must be [N, K]")
    N, K = w.shape
    codes = torch.empty((N, K), dtype=torch.uint8, device=w.device) if codes is None else codes
    scales = torch.empty((N // 128, K // 128), dtype=torch.uint8, device=w.device) if scales is None else scales
    _want(codes, "codes", (N, K), _CODES)
    _want(scales, "scales", (N // 128, K // 128), _CODES)
    rc = lib().dllm_fp8_quant_weight(_dev(w, "w"), _dtype_code(w), N, K, _u8(codes, "codes"),
                                     _u8(scales, "scales"), _stream())
    _check(rc, "dllm_fp8_quant_weight")
    return codes, scales


def _want_gemm(a, a_scale, w, w_scale):
    _want(a, "a", dtypes=_CODES)
    _want(w, "w", dtypes=_CODES)
    if a.dim() != 2 or w.dim() != 2 or a.shape[1] != w.shape[1]:
        raise DllmError(f"a [M, K] and w [N, K] disagree: {tuple(a.shape)}, {tuple(w.shape)}")
    M, K = a.shape
    N = w.shape[0]
    _want(a_scale, "a_scale", (K // 128, M), _CODES)
    _want(w_scale, "w_scale", (N // 128, K // 128), _CODES)
    return M, K, N


def dllm_fp8_gemm(a: torch.Tensor, a_scale: torch.Tensor, w: torch.Tensor, w_scale: torch.Tensor,
                  out: Optional[torch.Tensor] = None):
    """C = dequant(A) dequant(W)^T, bf16 [M, N]."""
    M, K, N = _want_gemm(a, a_scale, w, w_scale)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=a.device) if out is None else out
    _want(out, "out", (M, N), (torch.bfloat16,))
    rc = lib().dllm_fp8_gemm(_u8(a, "a"), _u8(a_scale, "a_scale"), _u8(w, "w"), _u8(w_scale, "w_scale"),
                             M, N, K, _dev(out, "out"), _stream())
    _check(rc, "dllm_fp8_gemm")
    return out


def dllm_fp8_gemm_swiglu(a: torch.Tensor, a_scale: torch.Tensor, w: torch.Tensor, w_scale: torch.Tensor,
                         out_codes: Optional[torch.Tensor] = None,
                         out_scales: Optional[torch.Tensor] = None):
    """h = silu(gate) * up from the interleaved Gate-Up weight, quantised:
    returns (codes [M, N/2], scales [N/256, M])."""
    M, K, N = _want_gemm(a, a_scale, w, w_scale)
    dev = a.device
    out_codes = torch.empty((M, N // 2), dtype=torch.uint8, device=dev) if out_codes is None else out_codes
    out_scales = torch.empty((N // 256, M), dtype=torch.uint8, device=dev) if out_scales is None else out_scales
    _want(out_codes, "out_codes", (M, N // 2), _CODES)
    _want(out_scales, "out_scales", (N // 256, M), _CODES)
    rc = lib().dllm_fp8_gemm_swiglu(_u8(a, "a"), _u8(a_scale, "a_scale"), _u8(w, "w"),
                                    _u8(w_scale, "w_scale"), M, N, K, _u8(out_codes, "out_codes"),
                                    _u8(out_scales, "out_scales"), _stream())
    _check(rc, "dllm_fp8_gemm_swiglu")
    return out_codes, out_scales


def dllm_vocab_stats_workspace(N: int, V: int) -> int:
    return lib().dllm_vocab_stats_workspace(N, V)


def dllm_workspace_size(which: int, cache: Optional[Cache] = None, q_dtype: int = BF16, Hq: int = 0,
                        n_q: int = 0, n_keys: int = 0, N: int = 0, V: int = 0) -> int:
    """Workspace bytes of the call `which` names (WS_*), from the shape fields
    that kind reads; 0 for an unknown kind or rejected shapes."""
    args = _WsArgs(cache=ctypes.pointer(cache.desc) if cache is not None else None,
                   q_dtype=q_dtype, Hq=Hq, n_q=n_q, n_keys=n_keys, N=N, V=V)
    return lib().dllm_workspace_size(which, ctypes.byref(args))


def dllm_vocab_stats(logits: torch.Tensor, V: Optional[int] = None,
                     argmax: Optional[torch.Tensor] = None, maxprob: Optional[torch.Tensor] = None,
                     entropy: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None):
    """logits: [N, >= V] (rows may be a strided view); returns (argmax, maxprob, entropy)."""
    _want(logits, "logits", dtypes=_FLOAT)
    if logits.dim() != 2:
        raise DllmError("logits must be [N, >= V]")
    N = logits.shape[0]
    V = logits.shape[1] if V is None else V
    if not 1 <= V <= logits.shape[1]:
        raise DllmError(f"V = {V} must be in [1, {logits.shape[1]}]")
    if logits.stride(1) != 1:
        raise DllmError("logits rows must be contiguous")
    dev = logits.device
    argmax = torch.empty(N, dtype=torch.int32, device=dev) if argmax is None else argmax
    maxprob = torch.empty(N, dtype=torch.float32, device=dev) if maxprob is None else maxprob
    entropy = torch.empty(N, dtype=torch.float32, device=dev) if entropy is None else entropy
    _want(argmax, "argmax", (N,), _I32)
    _want(maxprob, "maxprob", (N,), (torch.float32,))
    _want(entropy, "entropy", (N,), (torch.float32,))
    ws_need = dllm_vocab_stats_workspace(N, V)
    if workspace is None and ws_need:
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = lib().dllm_vocab_stats(_dev(logits, "logits", contiguous=False), _dtype_code(logits), N, V,
                                logits.stride(0), _dev(argmax, "argmax"), _dev(maxprob, "maxprob"),
                                _dev(entropy, "entropy"), _dev(workspace, "workspace"), ws_bytes,
                                _stream())
    _check(rc, "dllm_vocab_stats")
    return argmax, maxprob, entropy


class StabilityState:
    """Device decode state of B sequences of length L with ring depth D."""

    def __init__(self, B: int, L: int, D: int, device="cuda"):
        self.B, self.L, self.D = B, L, D
        self.ring_argmax = torch.empty((D, B, L), dtype=torch.int32, device=device)
        self.ring_maxprob = torch.empty((D, B, L), dtype=torch.float32, device=device)
        self.ring_step = torch.empty((D, B, L), dtype=torch.int32, device=device)
        self.entropy_latest = torch.empty((B, L), dtype=torch.float32, device=device)
        self.t_write = torch.empty((B, L), dtype=torch.int32, device=device)
        self.stable = torch.empty((B, L), dtype=torch.uint8, device=device)
        self.mask = torch.empty((B, L), dtype=torch.uint8, device=device)
        self.conf = torch.empty((B, L), dtype=torch.float32, device=device)
        self.next_pos = torch.empty((B, L), dtype=torch.int32, device=device)
        self.count = torch.empty((B,), dtype=torch.int32, device=device)
        self.all_stable = torch.empty((B,), dtype=torch.uint8, device=device)
        self.cached = torch.zeros((B, L), dtype=torch.uint8, device=device)   # K/V held per position
        self._decay = {}                      # (lambda, n) -> device table of exp(-lambda k)
        dllm_stability_reset(self)

    def decay_table(self, lam: float, n: int = 4096) -> torch.Tensor:
        """The device copy of dllm_confidence_decay(lam, n), made once per
        (lam, n) and kept with the state (call it before capturing a graph)."""
        key = (float(lam), int(n))
        t = self._decay.get(key)
        if t is None:
            if torch.cuda.is_current_stream_capturing():
                raise DllmError("the decay table must be made before graph capture: call decay_table() first")
            t = dllm_confidence_decay(lam, n).to(self.mask.device)
            self._decay[key] = t
        return t


def dllm_confidence_decay(lam: float, n: int = 4096) -> torch.Tensor:
    """Host table exp(-lam * k), k = 0 .. n-1, float64 (CPU tensor)."""
    t = torch.empty(int(n), dtype=torch.float64)
    rc = lib().dllm_confidence_decay(float(lam), int(n), t.data_ptr())
    _check(rc, "dllm_confidence_decay")
    return t


def dllm_check_positions(L: int, pos: torch.Tensor, bad: Optional[torch.Tensor] = None,
                         dup: Optional[torch.Tensor] = None):
    """Per sequence: entries of pos [B, n] outside [0, L) (other than -1),
    and entries repeating an earlier position.  Returns (bad, dup) [B] int32."""
    _want(pos, "pos", dtypes=_I32)
    if pos.dim() != 2:
        raise DllmError("pos must be [B, n]")
    B, n = pos.shape
    bad = torch.empty(B, dtype=torch.int32, device=pos.device) if bad is None else bad
    dup = torch.empty(B, dtype=torch.int32, device=pos.device) if dup is None else dup
    _want(bad, "bad", (B,), _I32)
    _want(dup, "dup", (B,), _I32)
    rc = lib().dllm_check_positions(B, int(L), _dev(pos, "pos"), n, _dev(bad, "bad"), _dev(dup, "dup"),
                                    _stream())
    _check(rc, "dllm_check_positions")
    return bad, dup


def dllm_stability_reset(st: StabilityState):
    rc = lib().dllm_stability_reset(st.B, st.L, st.D, _dev(st.ring_argmax, "ring_argmax"),
                                    _dev(st.ring_maxprob, "ring_maxprob"), _dev(st.ring_step, "ring_step"),
                                    _dev(st.entropy_latest, "entropy_latest"), _dev(st.t_write, "t_write"),
                                    _dev(st.stable, "stable"), _stream())
    _check(rc, "dllm_stability_reset")


def dllm_stability_mask(st: StabilityState, step, pos: Optional[torch.Tensor],
                        argmax: torch.Tensor, maxprob: torch.Tensor, entropy: torch.Tensor, *,
                        K: int, tau: float, R: int, alpha: float = 0.0, beta: float = 0.0,
                        lam: float = 0.0, conf_thresh: float = 0.0, V: int = 2,
                        with_conf: bool = True, advance_step: bool = False, R_early: int = 0,
                        T_steps: int = 0, refresh_every: int = 0, n_decay: int = 4096):
    """One step of history, stability, confidence and window mask; outputs
    land in st.mask, st.conf, st.next_pos, st.count, st.all_stable.  ``step``
    is an int, or a [B] int32 GPU tensor of per-sequence step numbers read
    when the kernel runs (for captured graphs); with ``advance_step`` the
    kernel increments that tensor once it has used it.  ``R_early`` and
    ``T_steps`` widen the window radius from R_early to R over T_steps steps;
    ``refresh_every`` > 0 makes every such step (after step 0) a full refresh.
    The confidence's age factor exp(-lam * dt) is read from the state's
    n_decay-entry table (ages past the end read its last entry)."""
    if pos is not None:
        _want(pos, "pos", dtypes=_I32)
        if pos.dim() != 2 or pos.shape[0] != st.B:
            raise DllmError(f"pos: shape {tuple(pos.shape)}, expected [{st.B}, n]")
    n = pos.shape[1] if pos is not None else st.L
    _want(argmax, "argmax", dtypes=_I32, numel=st.B * n)
    _want(maxprob, "maxprob", dtypes=(torch.float32,), numel=st.B * n)
    _want(entropy, "entropy", dtypes=(torch.float32,), numel=st.B * n)
    decay = st.decay_table(lam, n_decay) if beta != 0.0 else None
    prm = _StabParams(K=K, D=st.D, R=R, advance_step=int(advance_step), tau=tau, alpha=alpha, beta=beta,
                      conf_thresh=conf_thresh, decay=decay.data_ptr() if decay is not None else None,
                      vocab=V, R_early=R_early, T_steps=T_steps, refresh_every=refresh_every,
                      n_decay=int(n_decay) if decay is not None else 0)
    if isinstance(step, torch.Tensor):
        if step.dtype != torch.int32 or step.numel() != st.B:
            raise ValueError("step tensor: [B] int32 per-sequence step numbers")
        step_host, step_dev = 0, _dev(step, "step")
    else:
        step_host, step_dev = int(step), None
    rc = lib().dllm_stability_mask(st.B, st.L, step_host, step_dev, _dev(pos, "pos"), n, _dev(argmax, "argmax"),
                                   _dev(maxprob, "maxprob"), _dev(entropy, "entropy"),
                                   _dev(st.ring_argmax, "ring_argmax"), _dev(st.ring_maxprob, "ring_maxprob"),
                                   _dev(st.ring_step, "ring_step"), _dev(st.entropy_latest, "entropy_latest"),
                                   _dev(st.t_write, "t_write"), _dev(st.stable, "stable"),
                                   ctypes.byref(prm), _dev(st.mask, "mask"),
                                   _dev(st.conf, "conf") if with_conf else None,
                                   _dev(st.next_pos, "next_pos"), _dev(st.count, "count"),
                                   _dev(st.all_stable, "all_stable"), _stream())
    _check(rc, "dllm_stability_mask")
    return st


def dllm_refresh_interval(T: int) -> int:
    """Full-refresh interval for a trajectory of T steps."""
    return lib().dllm_refresh_interval(int(T))


def dllm_cache_quotas(lens, budget: int, min_frac: float = 0.2):
    """Per-request cache quotas (host): guaranteed ceil(min_frac * len), the
    rest of the budget in arrival order.  Returns an int32 numpy array."""
    import numpy as np
    ln = np.ascontiguousarray(np.asarray(lens, dtype=np.int32))
    q = np.zeros_like(ln)
    rc = lib().dllm_cache_quotas(int(ln.size), ln.ctypes.data, int(budget), float(min_frac), q.ctypes.data)
    _check(rc, "dllm_cache_quotas")
    return q


def dllm_evict_by_confidence(st: StabilityState, quota: torch.Tensor, pos: Optional[torch.Tensor],
                             evicted: Optional[torch.Tensor] = None):
    """Mark the recomputed positions cached, evict the lowest-confidence ones
    beyond each sequence's quota, and add every uncached position to the next
    step's mask (st.cached, st.mask, st.next_pos, st.count updated; st.conf is
    the confidence the preceding stability step wrote)."""
    if quota.dtype != torch.int32 or quota.numel() != st.B:
        raise ValueError("quota: [B] int32")
    if pos is not None:
        _want(pos, "pos", dtypes=_I32)
        if pos.dim() != 2 or pos.shape[0] != st.B:
            raise DllmError(f"pos: shape {tuple(pos.shape)}, expected [{st.B}, n]")
    _want(evicted, "evicted", (st.B,), _I32, required=False)
    n = pos.shape[1] if pos is not None else st.L
    rc = lib().dllm_evict_by_confidence(st.B, st.L, _dev(st.conf, "conf"), _dev(quota, "quota"),
                                        _dev(pos, "pos"), n, _dev(st.cached, "cached"), _dev(st.mask, "mask"),
                                        _dev(st.next_pos, "next_pos"), _dev(st.count, "count"),
                                        _dev(evicted, "evicted") if evicted is not None else None, _stream())
    _check(rc, "dllm_evict_by_confidence")
    return st


def dllm_parallel_width(w_early: int, w_late: int, T: int, step: int) -> int:
    """Positions decoded in parallel at a step: w_early falling to w_late."""
    return lib().dllm_parallel_width(int(w_early), int(w_late), int(T), int(step))


def dllm_self_verify(st: StabilityState, dec_pos: torch.Tensor, p_marg: torch.Tensor,
                     p_joint: torch.Tensor, W: int, tau: float = 0.5, rollback: Optional[torch.Tensor] = None,
                     n_rollback: Optional[torch.Tensor] = None, rb_pos: Optional[torch.Tensor] = None,
                     update_stable: bool = True, update_cached: bool = True):
    """Conflict check of the step's parallel decodes (dec_pos [B, n] int32,
    ascending then -1; p_marg [B, n] and p_joint [B, n, W-1] float32).
    Withdrawn positions go into st.mask (and out of st.stable / st.cached);
    st.next_pos / st.count are compacted again.  Returns the [B, L] u8
    withdrawal flags."""
    B, n = dec_pos.shape
    if dec_pos.dtype != torch.int32 or B != st.B:
        raise ValueError("dec_pos: [B, n] int32")
    if p_marg.dtype != torch.float32 or p_marg.numel() != B * n:
        raise ValueError("p_marg: [B, n] float32")
    if p_joint.dtype != torch.float32 or p_joint.numel() != B * n * (W - 1):
        raise ValueError("p_joint: [B, n, W-1] float32")
    if rollback is None:
        rollback = torch.empty((st.B, st.L), dtype=torch.uint8, device=st.mask.device)
    rc = lib().dllm_self_verify(st.B, st.L, _dev(dec_pos, "dec_pos"), n, _dev(p_marg, "p_marg"),
                                _dev(p_joint, "p_joint"), int(W), float(tau), _dev(rollback, "rollback"),
                                _dev(st.mask, "mask"), _dev(st.stable, "stable") if update_stable else None,
                                _dev(st.cached, "cached") if update_cached else None,
                                _dev(st.next_pos, "next_pos"), _dev(st.count, "count"),
                                _dev(n_rollback, "n_rollback") if n_rollback is not None else None,
                                _dev(rb_pos, "rb_pos") if rb_pos is not None else None, _stream())
    _check(rc, "dllm_self_verify")
    return rollback
