"""Seeded synthetic inputs for one step of cached masked-diffusion decoding.

This module is shared by the oracle side and the HIP side of every test and
of the benchmark.  It holds no arithmetic of the method: it only draws
random numbers, rounds them to the storage format (round-to-nearest-even,
as torch's dtype conversion does) and plants the structure the workloads
call for (peaked tokens, exact ties, block positions).  Everything is
reproducible from the seeds below.

Shapes follow the models the pages use: GPT-2 small (12 heads x 64, vocab
50257) from the attention-sinks page's config listing, and LLaDA-8B (32 heads
x 128, vocab 126464, prompt + masked suffix SAR blocks) from the LaCache
explainer's experiments section.  No dataset item is used; these tensors
stand in for the benchmark suites the pages evaluate on.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

F32, BF16, E4M3 = 0, 1, 2
TORCH_DTYPE = {F32: torch.float32, BF16: torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    seed: int
    B: int = 1
    L: int = 64
    Hq: int = 4
    Hkv: int = 4
    d: int = 16
    kv_dtype: int = F32          # cache storage
    q_dtype: int = F32           # query / fresh-row storage
    b: int = 8                   # active block length
    V: int = 0                   # vocabulary (0: no vocab pass)
    V_stride: int = 0            # row stride of logits (>= V)
    logit_rows: str = "all"      # "all" positions or "block" rows
    logit_sigma: float = 1.0
    peak_frac: float = 0.0
    peak_lo: float = 0.0
    peak_hi: float = 0.0
    tie_frac: float = 0.0
    T: int = 0                   # steps of a trajectory (0: single step)
    K: int = 3
    tau: float = 0.95
    R: int = 2
    D: int = 3                   # history ring depth
    alpha: float = 0.0
    beta: float = 0.0
    lam: float = 0.0
    conf_thresh: float = 0.0
    sinks: int = 0               # >0: sink + rolling key map
    rolling: int = 0
    block_mode: str = "fixed"    # "fixed" start, "random" offset, "sar", "end"
    block_start: int = 0
    qkv_std: float = 0.25

    @property
    def n_logit_rows(self) -> int:
        return self.B * (self.L if self.logit_rows == "all" else self.b)


CONFIGS = {
    # tiny parity case: everything small enough for the oracle in milliseconds
    "tiny": Config(name="tiny", seed=1001, B=1, L=64, Hq=4, Hkv=4, d=16, kv_dtype=F32, q_dtype=F32,
                   b=8, block_mode="fixed", block_start=32, V=512, V_stride=512,
                   logit_sigma=1.0, peak_frac=0.4, peak_lo=8.0, peak_hi=8.0, T=16, K=3, tau=0.95,
                   R=2, D=16, alpha=0.7, beta=0.3, lam=3.0 / 16, conf_thresh=0.8,
                   qkv_std=1.0 / math.sqrt(16)),
    # GPT-2-small-shaped step (12 heads x 64, vocab 50257, rows unaligned)
    "gpt2": Config(name="gpt2", seed=1002, B=8, L=1024, Hq=12, Hkv=12, d=64, kv_dtype=BF16,
                   q_dtype=BF16, b=32, block_mode="random", V=50257, V_stride=50257,
                   logit_sigma=math.sqrt(2.0), peak_frac=0.6, peak_lo=6.0, peak_hi=6.0, K=3,
                   tau=0.95, R=2, D=3, qkv_std=1.0 / 8),
    # LLaDA-8B-shaped SAR step: 1536 prompt + 512 masked suffix, block of 32
    "llada": Config(name="llada", seed=1003, B=16, L=2048, Hq=32, Hkv=32, d=128, kv_dtype=BF16,
                    q_dtype=BF16, b=32, block_mode="sar", block_start=1536, V=126464,
                    V_stride=126464, logit_rows="block", logit_sigma=math.sqrt(1.5),
                    peak_frac=1.0, peak_lo=0.0, peak_hi=10.0, qkv_std=1.0 / math.sqrt(128)),
    # vocab-stats-heavy sweep with exact ties and a 64-step history ring
    "vocab": Config(name="vocab", seed=1004, B=64, L=512, V=126464, V_stride=126464,
                    logit_sigma=1.0, peak_frac=0.7, peak_lo=4.0, peak_hi=12.0, tie_frac=0.01,
                    T=64, K=3, tau=0.9, R=3, D=64, alpha=0.7, beta=0.3, lam=3.0 / 64,
                    conf_thresh=0.8, b=0),
    # long context, e4m3 cache with per-128 scales, GQA 32/8, sink + rolling map
    "longctx": Config(name="longctx", seed=1005, B=4, L=32768, Hq=32, Hkv=8, d=128,
                      kv_dtype=E4M3, q_dtype=BF16, b=64, block_mode="end", sinks=4,
                      rolling=8188, qkv_std=1.0 / math.sqrt(128)),
}

# the order the five workloads are listed in
ORDER = ["tiny", "gpt2", "llada", "vocab", "longctx"]


def generator(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _randn(shape, std, g, device, dtype=torch.float32):
    return (torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std).to(dtype)


def src_dtype(cfg: Config) -> int:
    """storage format of fresh K/V rows and queries (e4m3 caches take bf16)"""
    return cfg.q_dtype


def block_positions(cfg: Config, device="cpu") -> torch.Tensor:
    """[B, b] int32 positions of the active block of each sequence."""
    g = generator(cfg.seed * 7 + 1, "cpu")
    B, L, b = cfg.B, cfg.L, cfg.b
    if cfg.block_mode == "fixed":
        starts = torch.full((B,), cfg.block_start, dtype=torch.int64)
    elif cfg.block_mode == "random":
        starts = torch.randint(0, L - b + 1, (B,), generator=g)
    elif cfg.block_mode == "sar":
        starts = cfg.block_start + b * torch.randint(0, (L - cfg.block_start) // b, (B,), generator=g)
    elif cfg.block_mode == "end":
        starts = torch.full((B,), L - b, dtype=torch.int64)
    else:
        raise ValueError(cfg.block_mode)
    pos = starts[:, None] + torch.arange(b)[None, :]
    return pos.to(torch.int32).to(device)


def kv_rows(cfg: Config, device="cpu", which: str = "cache", step: int = 0, B: Optional[int] = None,
            n: Optional[int] = None):
    """Rows in the layout fresh K/V arrive in: [B, n, Hkv, d] for K and V.

    which="cache": the n = L rows a full forward would write (fills the cache);
    which="fresh": the b recomputed block rows of `step`.
    """
    B = cfg.B if B is None else B
    if which == "cache":
        n = cfg.L if n is None else n
        seed = cfg.seed * 7 + 2
    else:
        n = cfg.b if n is None else n
        seed = cfg.seed * 7 + 3 + 1000 * step
    g = generator(seed, device)
    dt = TORCH_DTYPE[src_dtype(cfg)]
    k = _randn((B, n, cfg.Hkv, cfg.d), cfg.qkv_std, g, device, dt)
    v = _randn((B, n, cfg.Hkv, cfg.d), cfg.qkv_std, g, device, dt)
    return k, v


def queries(cfg: Config, device="cpu", step: int = 0, scale_std: float = 1.0, B=None, b=None):
    """[B, Hq, b, d] queries of the active block; scale_std > 1 sharpens."""
    B = cfg.B if B is None else B
    b = cfg.b if b is None else b
    g = generator(cfg.seed * 7 + 4 + 1000 * step, device)
    return _randn((B, cfg.Hq, b, cfg.d), cfg.qkv_std * scale_std, g, device,
                  TORCH_DTYPE[cfg.q_dtype])


def outside_queries(cfg: Config, device="cpu", B=None, n: Optional[int] = None):
    """[B, Hq, n, d] queries of the positions outside the active block
    (n = L - b), unchanged over a block's steps."""
    B = cfg.B if B is None else B
    n = cfg.L - cfg.b if n is None else n
    g = generator(cfg.seed * 7 + 7, device)
    return _randn((B, cfg.Hq, n, cfg.d), cfg.qkv_std, g, device, TORCH_DTYPE[cfg.q_dtype])


def memo_state(B: int, Hq: int, n: int, d: int, seed: int, o_std: float, lse_mean: float,
               lse_std: float = 1.0, empty_frac: float = 0.0, device="cpu"):
    """A random memoized softmax state in its stored form: o [B, Hq, n, d]
    ~ N(0, o_std), lse [B, Hq, n] ~ N(lse_mean, lse_std) float32, with a
    fraction of rows marked empty (lse = -inf)."""
    g = generator(seed, "cpu")
    o = torch.randn((B, Hq, n, d), generator=g) * o_std
    lse = torch.randn((B, Hq, n), generator=g) * lse_std + lse_mean
    if empty_frac > 0:
        lse[torch.rand((B, Hq, n), generator=g) < empty_frac] = float("-inf")
    return o.to(device), lse.to(device)


def fp8_codes(shape, seed: int, device="cpu", exp_lo: int = 0, exp_hi: int = 15) -> torch.Tensor:
    """OCP e4m3fn codes with a uniform sign and mantissa and an exponent field
    uniform in [exp_lo, exp_hi] (field 0: subnormals; the NaN code of field
    15 is replaced by the largest finite code), uint8"""
    g = generator(seed, "cpu")
    sign = torch.randint(0, 2, shape, generator=g, dtype=torch.int32)
    e = torch.randint(exp_lo, exp_hi + 1, shape, generator=g, dtype=torch.int32)
    m = torch.randint(0, 8, shape, generator=g, dtype=torch.int32)
    c = (sign << 7) | (e << 3) | m
    c = torch.where((c & 0x7F) == 0x7F, c - 1, c)
    return c.to(torch.uint8).to(device)


def e8m0_codes(shape, seed: int, lo: int, hi: int, device="cpu") -> torch.Tensor:
    """E8M0 scale codes drawn uniformly from [lo, hi], uint8"""
    g = generator(seed, "cpu")
    return torch.randint(lo, hi + 1, shape, generator=g, dtype=torch.int32).to(torch.uint8).to(device)


# the FFN of a LLaDA-8B-shaped layer: hidden 4096 (32 heads x 128), SwiGLU
# width 12288 (the pages give no FFN width; 3x the hidden width is taken)
FFN_HIDDEN, FFN_INTER = 4096, 12288


def ffn_inputs(M: int, seed: int, device="cpu", K: int = FFN_HIDDEN, I: int = FFN_INTER):
    """hidden states x and residual [M, K] ~ N(0, 1), RMS-norm weight
    gamma ~ 1 + N(0, 0.1^2) [K], Gate-Up weight [2I, K] with gate and up
    128-row blocks interleaved ~ N(0, 1/K), FF-Out weight [K, I] ~ N(0, 1/I),
    all bf16"""
    g = generator(seed, device)
    x = _randn((M, K), 1.0, g, device, torch.bfloat16)
    res = _randn((M, K), 1.0, g, device, torch.bfloat16)
    gamma = (1.0 + torch.randn((K,), generator=g, device=device) * 0.1).to(torch.bfloat16)
    w_gu = _randn((2 * I, K), 1.0 / math.sqrt(K), g, device, torch.bfloat16)
    w_out = _randn((K, I), 1.0 / math.sqrt(I), g, device, torch.bfloat16)
    return x, res, gamma, w_gu, w_out


def logits(cfg: Config, device="cpu", step: int = 0, rows: Optional[int] = None,
           stride: Optional[int] = None, dtype: Optional[int] = None):
    """[rows, stride] logits (only the first V columns are used).

    Peaked rows get +U(peak_lo, peak_hi) on one token that is fixed per row
    across steps (drawn from the config seed); the noise is redrawn per step.
    Tie rows get two distinct tokens set to the same large value (exact tie
    of the row maximum).
    """
    N = cfg.n_logit_rows if rows is None else rows
    V = cfg.V
    stride = cfg.V_stride if stride is None else stride
    dtype = (F32 if cfg.name == "tiny" else BF16) if dtype is None else dtype
    g = generator(cfg.seed * 7 + 5 + 1000 * step, device)
    x = torch.randn((N, stride), generator=g, device=device, dtype=torch.float32)
    x.mul_(cfg.logit_sigma)
    gs = generator(cfg.seed * 7 + 6, "cpu")            # per-row structure, fixed across steps
    n_peak = int(round(cfg.peak_frac * N))
    if n_peak:
        prow = torch.randperm(N, generator=gs)[:n_peak]
        ptok = torch.randint(0, V, (n_peak,), generator=gs)
        if cfg.peak_hi > cfg.peak_lo:
            amp = cfg.peak_lo + (cfg.peak_hi - cfg.peak_lo) * torch.rand(n_peak, generator=gs)
        else:
            amp = torch.full((n_peak,), cfg.peak_lo)
        x[prow.to(device), ptok.to(device)] += amp.to(device)
    n_tie = int(round(cfg.tie_frac * N))
    if n_tie:
        trow = torch.randperm(N, generator=gs)[:n_tie]
        t1 = torch.randint(0, V, (n_tie,), generator=gs)
        t2 = (t1 + 1 + torch.randint(0, V - 1, (n_tie,), generator=gs)) % V
        x[trow.to(device), t1.to(device)] = 16.0
        x[trow.to(device), t2.to(device)] = 16.0
    if stride > V:
        x[:, V:] = 0.0
    return x.to(TORCH_DTYPE[dtype])


def sharp_query_scale(cfg: Config) -> float:
    """factor on the query std that makes the score std about 3 (a peaked
    softmax), instead of the near-uniform softmax of the stated inputs"""
    # score std = std_q * std_k * sqrt(d) * (1/sqrt(d)) = std_q * std_k
    return 3.0 / (cfg.qkv_std * cfg.qkv_std)


def as_numpy_bits(t: torch.Tensor):
    """CPU numpy view of a tensor in the oracle's storage: bf16 as uint16 bits."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    return t.numpy()
