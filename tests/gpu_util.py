"""Shared helpers of the GPU parity tests (host-side only)."""
import sys

import numpy as np
import torch

import workloads as W


def need_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need an MI355X; run them with -m gpu on a GPU host")
    import cached_denoising_amd as D
    D.lib()
    return D


def say(*a):
    """name the case before each GPU step, flushed, so a failing run names it"""
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def bits(t):
    return W.as_numpy_bits(t)


def cache_np(cache):
    """oracle-side copies of a device cache (storage bytes)"""
    ck, cv = bits(cache.k), bits(cache.v)
    ks = cache.k_scale.cpu().numpy() if cache.k_scale is not None else None
    vs = cache.v_scale.cpu().numpy() if cache.v_scale is not None else None
    return ck, cv, ks, vs


def attn_errors(out, ref):
    """max-abs error and max-abs error normalised by max |ref|"""
    o = out.float().cpu().numpy().astype(np.float64)
    e = np.abs(o - ref).max()
    return e, e / max(np.abs(ref).max(), 1e-30)


def new_cache(D, B, Hkv, L, d, dtype, device="cuda"):
    tdt = {W.F32: torch.float32, W.BF16: torch.bfloat16, W.E4M3: torch.uint8}[dtype]
    k = torch.empty((B, Hkv, L, d), dtype=tdt, device=device)
    v = torch.empty_like(k)
    ks = vs = None
    if dtype == W.E4M3:
        ks = torch.empty((B, Hkv, L, d // 128), dtype=torch.float32, device=device)
        vs = torch.empty_like(ks)
    return D.dllm_cache_init(k, v, dtype, ks, vs)
