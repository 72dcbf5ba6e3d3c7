"""Benchmark of one decode step of the cached masked-diffusion hot path.

A step is one pass over the calls of the GPT-2-small-shaped workload
(B=8 sequences of L=1024, 12 heads x 64, bf16 K/V cache, active block of 32
at a per-sequence offset, vocab 50257 bf16 logits for every position):
    dllm_scatter_attention (the scatter of the block's K/V rows, then the
    block attention) -> dllm_vocab_stats -> dllm_stability_mask
all on one stream with inputs resident in HBM.  Prints one JSON line.

With --config facache a step is the first-layer attention of a later
denoising step of a LLaDA-shaped block with FACache (B=16, L=2048, 32 heads
x 128, block 32): scatter the block's K/V, the block's queries over all L
keys, and the 2016 queries outside the block continued from their memoized
state over the 32 block keys.  The memo is filled once, before the timed
steps (the block's first step); a full recompute of all 2048 queries over
all 2048 keys is timed beside it.

With --config ffn a step is the FFN of one LLaDA-shaped layer in per-group
FP8 on the same 16 x 2048 step (32768 tokens, hidden 4096, SwiGLU width
12288): add & norm fused with the 1 x 128 quantisation, the Gate-Up product
fused with SwiGLU and the quantisation of its output, the FF-Out product in
bf16.  The weights are quantised once, before the timed steps.

With --config policies a step is the decode policies on the vocab sweep's
64 x 512 positions: the stability mask with the window radius ramped from
0 to 3 over the 64-step trajectory and a full refresh at the interval for
that length, then the eviction of the lowest-confidence cached positions
beyond each sequence's quota (half the positions shared out with a 20%
guarantee per request).  The step statistics are computed once, before the
timed steps.  The eviction alone is also timed at the long-context shape
(4 x 32768, quota 8192).

With --config verify a step is the self-verification of one step's
parallel decodes on the vocab sweep's 64 x 512 positions: 16 positions
decoded per sequence (the early parallel width), a window of 4 positions,
tau 0.5, seeded marginals and pair joints with planted conflicts.  The same
kernel is also timed at the long-context shape (4 x 32768, its 64-position
block decoded at once).

Timing.  The K timed steps are one captured HIP graph, replayed behind
untimed replays so that the host's launch of the graph (reported apart) is
not inside the event pair.  Per call, HIP events on the launch stream give
three figures: hot (an event pair around each call of 100 eager steps), cold
(the same after a 1 GiB device read that evicts the caches) and b2b (back-to-
back launches of the call alone from a graph, one event pair around them).
The events are created without the system-scope fence a default event
performs at record.  The roofline takes the cold figure for a call whose
bytes fit the 256 MB last-level cache and the hot figure otherwise.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config gpt2]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "denoise steps/sec (block attn + vocab stats); achieved HBM GB/s vs peak"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0      # dense bf16 matrix peak of MI355X
MFMA_FP8_PEAK_TFLOPS = 5000.0       # dense fp8 matrix peak of MI355X
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "cached_denoising_amd", "csrc")
# the source files of each call whose counters a profile summary records
KERNEL_SRC = {"vocab_stats": ["vocab_stats.hip"],
              "facache_merge": ["attention.hip", "attention_shared.hip", "attn_common.hpp"],
              "scatter_attention": ["attention.hip", "attention_shared.hip", "attn_common.hpp", "scatter.hip"],
              "scatter": ["scatter.hip"], "stability": ["stability.hip"],
              "fp8_addnorm": ["fp8_ffn.hip", "common.hpp", "attn_common.hpp"],
              "fp8_gateup": ["fp8_ffn.hip", "common.hpp", "attn_common.hpp"],
              "fp8_ffout": ["fp8_ffn.hip", "common.hpp", "attn_common.hpp"], "evict": ["stability.hip"],
              "verify": ["verify.hip"]}


class Event:
    """A HIP timing event created without the system-scope fence that a
    default event performs when it is recorded (a write-back and invalidate
    of the caches, which adds microseconds to every timed call and slows the
    work after it).  It comes from the HIP runtime torch has loaded, so it
    records on torch's streams."""
    _hip = None

    @classmethod
    def hip(cls):
        if cls._hip is None:
            import torch
            path = os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so")
            L = ctypes.CDLL(path if os.path.exists(path) else "libamdhip64.so.7")
            L.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            L.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            L.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._hip = L
        return cls._hip

    def __init__(self):
        self.ev = ctypes.c_void_p()
        if self.hip().hipEventCreateWithFlags(ctypes.byref(self.ev), 0x20000000) != 0:   # hipEventDisableSystemFence
            raise RuntimeError("hipEventCreateWithFlags failed")

    def record(self):
        import torch
        if self.hip().hipEventRecord(self.ev, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_time(self, end) -> float:
        """milliseconds from this event to `end` (both complete)"""
        ms = ctypes.c_float()
        if self.hip().hipEventElapsedTime(ctypes.byref(ms), self.ev, end.ev) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def __del__(self):
        if self.ev and self._hip is not None:
            self._hip.hipEventDestroy(self.ev)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="gpt2",
                    choices=["gpt2", "llada", "vocab", "longctx", "facache", "ffn", "policies", "verify"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true",
                    help="launch every kernel from Python instead of replaying a captured graph")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy 5 times (HBM counter calibration)")
    return ap.parse_args()


def copy_calibration():
    """A plain copy of known size: its FETCH_SIZE / WRITE_SIZE counters give
    the factor from counter units to bytes for the kernels measured alike."""
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "bytes_written": n, "launches": 5}), flush=True)


def kernel_sha(paths):
    h = hashlib.sha256()
    for path in paths:
        h.update(open(path, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, config):
    """HBM bytes per launch of a kernel from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source"""
    path = os.path.join(PROFILES, f"{kernel}_{config}_pmc.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_sha = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    m_tb = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_sha or not m_tb or m_sha.group(1) != kernel_sha([os.path.join(CSRC, f) for f in KERNEL_SRC[kernel]]):
        return None
    return float(m_tb.group(1))


class Step:
    """All device buffers of one workload and the kernels of one step."""

    def __init__(self, D, W, cfg, dev, facache=False):
        import torch
        self.D, self.W, self.cfg, self.dev = D, W, cfg, dev
        B, L, H, d = cfg.B, cfg.L, cfg.Hkv, cfg.d
        kvt = {W.BF16: torch.bfloat16, W.E4M3: torch.uint8, W.F32: torch.float32}[cfg.kv_dtype]
        self.has_attn = cfg.b > 0 and d > 0 and cfg.name != "vocab"
        self.has_vocab = cfg.V > 0 and not facache
        self.has_stab = cfg.name in ("gpt2", "vocab", "tiny") and not facache
        self.facache = facache
        self.attn_split = False
        if self.has_attn:
            k = torch.empty((B, H, L, d), dtype=kvt, device=dev)
            v = torch.empty_like(k)
            ks = vs = None
            if cfg.kv_dtype == W.E4M3:
                ks = torch.empty((B, H, L, d // 128), dtype=torch.float32, device=dev)
                vs = torch.empty_like(ks)
            self.cache = D.dllm_cache_init(k, v, cfg.kv_dtype, ks, vs)
            kc, vc = W.kv_rows(cfg, device=dev)
            D.dllm_scatter_kv(self.cache, kc, vc, torch.arange(L, dtype=torch.int32, device=dev).repeat(B, 1))
            del kc, vc
            self.kn, self.vn = W.kv_rows(cfg, device=dev, which="fresh")
            self.pos = W.block_positions(cfg, dev)
            self.q = W.queries(cfg, device=dev)
            self.key_idx = None
            if cfg.sinks:
                end = (self.pos[:, -1] + 1).contiguous()
                self.key_idx = torch.empty((B, cfg.sinks + cfg.rolling), dtype=torch.int32, device=dev)
                D.dllm_sink_rolling_map(L, cfg.sinks, cfg.rolling, end, self.key_idx)
            n_keys = L if self.key_idx is None else self.key_idx.shape[1]
            self.n_keys = n_keys
            self.out = torch.empty((B, cfg.Hq, cfg.b, d), dtype=torch.bfloat16, device=dev)
            wsb = D.dllm_block_attention_workspace(self.cache, W.BF16, cfg.Hq, cfg.b, n_keys)
            self.attn_ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
            # a workspace is needed only when the keys are split over workgroups
            self.attn_split = wsb > 0
        if facache:
            # the memo of the queries outside the block over the unchanged keys,
            # filled once (the block's first step)
            self.n_q = L - cfg.b
            self.un, self.blk = D.dllm_facache_maps(L, cfg.b, self.pos[:, 0].contiguous())
            self.qu = W.outside_queries(cfg, device=dev)
            self.memo_lse = torch.empty((B, cfg.Hq, self.n_q), dtype=torch.float32, device=dev)
            self.memo_o = D.dllm_block_attention(self.cache, self.qu, key_idx=self.un,
                                                 out_dtype=torch.float32, lse=self.memo_lse)
            self.out_u = torch.empty((B, cfg.Hq, self.n_q, d), dtype=torch.bfloat16, device=dev)
            wsb = D.dllm_facache_merge_workspace(self.cache, W.BF16, cfg.Hq, self.n_q, cfg.b)
            self.fa_ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
        if self.has_vocab:
            self.logits = W.logits(cfg, device=dev)
            N = self.logits.shape[0]
            self.N = N
            self.am = torch.empty(N, dtype=torch.int32, device=dev)
            self.mp = torch.empty(N, dtype=torch.float32, device=dev)
            self.en = torch.empty(N, dtype=torch.float32, device=dev)
            wsb = D.dllm_vocab_stats_workspace(N, cfg.V)
            self.vocab_ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
        if self.has_stab:
            self.st = D.StabilityState(B, L, cfg.D, device=dev)
            self.kw = dict(K=cfg.K, tau=cfg.tau, R=cfg.R, alpha=cfg.alpha, beta=cfg.beta,
                           lam=cfg.lam, conf_thresh=cfg.conf_thresh, V=cfg.V)
            if cfg.beta != 0.0:
                self.st.decay_table(cfg.lam)      # the age-factor table, made before any capture
        # per-sequence decode step numbers live on the device and the
        # stability kernel advances them, so a captured graph of several steps
        # replays successive steps
        self.step_t = torch.zeros(B, dtype=torch.int32, device=dev)
    def calls(self):
        """the step's calls in order, as (name, function) pairs"""
        D, cfg = self.D, self.cfg
        out = []
        if self.has_attn:
            # the block's fresh K/V rows into the cache, then its queries over
            # the keys, in one call
            out.append(("scatter_attention", lambda: D.dllm_scatter_attention(
                self.cache, self.kn, self.vn, self.pos, self.q, key_idx=self.key_idx, out=self.out,
                workspace=self.attn_ws)))
        if self.facache:
            out.append(("facache_merge", lambda: D.dllm_facache_merge(
                self.cache, self.qu, self.memo_o, self.memo_lse, key_idx=self.blk, out=self.out_u,
                workspace=self.fa_ws)))
        if self.has_vocab:
            out.append(("vocab_stats", lambda: D.dllm_vocab_stats(
                self.logits, V=cfg.V, argmax=self.am, maxprob=self.mp, entropy=self.en, workspace=self.vocab_ws)))
        if self.has_stab:
            B, L = cfg.B, cfg.L
            out.append(("stability", lambda: D.dllm_stability_mask(
                self.st, self.step_t, None, self.am.view(B, L), self.mp.view(B, L), self.en.view(B, L),
                advance_step=True, **self.kw)))
        return out

    def algorithmic_bytes(self):
        """bytes each kernel must move (reads + writes), per launch"""
        cfg = self.cfg
        out = {}
        if self.has_attn:
            esz = 1 if cfg.kv_dtype == self.W.E4M3 else 2
            rows = cfg.B * cfg.b * cfg.Hkv
            scale_b = 4 * 2 if cfg.kv_dtype == self.W.E4M3 else 0
            # the scatter: fresh bf16 rows in, cache rows (and scales) out,
            # positions; the attention: the selected keys' K and V rows (and
            # scales), queries in and output out, all bf16
            scatter = rows * cfg.d * (2 * 2 + 2 * esz) + rows * scale_b + cfg.B * cfg.b * 4
            kv = cfg.B * cfg.Hkv * self.n_keys * (cfg.d * esz * 2 + scale_b)
            qo = cfg.B * cfg.Hq * cfg.b * cfg.d * 2 * 2
            out["scatter_attention"] = scatter + kv + qo
        if self.facache:
            rows = cfg.B * cfg.Hq * self.n_q
            # queries and output in bf16, the memo (O and lse) in fp32, the
            # block's K/V rows and its key list
            out["facache_merge"] = (rows * (cfg.d * 2 * 2 + (cfg.d + 1) * 4)
                                    + cfg.B * cfg.Hkv * cfg.b * cfg.d * 2 * 2 + cfg.B * cfg.b * 4)
        if self.has_vocab:
            out["vocab_stats"] = self.N * cfg.V * 2 + self.N * 12
        if self.has_stab:
            BL = cfg.B * cfg.L
            # stats in (12) + ring slot write (12) + K-1 ring reads (12 each) +
            # state read/write (entropy 4, t_write 4, stable 1: twice) + outputs
            # (mask 1, conf 4, next_pos 4)
            out["stability"] = BL * (12 + 12 + 12 * (cfg.K - 1) + 2 * 9 + 9)
        return out

    def algorithmic_flops(self):
        """matrix flops of the attention call: QK^T and PV, 2 flops per
        multiply-add, for every (query head, query, key, dim)"""
        cfg = self.cfg
        if not self.has_attn:
            return {}
        out = {"scatter_attention": 4 * cfg.B * cfg.Hq * cfg.b * self.n_keys * cfg.d}
        if self.facache:
            out["facache_merge"] = 4 * cfg.B * cfg.Hq * self.n_q * cfg.b * cfg.d
        return out

    def full_recompute_us(self, reps=3):
        """the first-layer attention without FACache: all L queries over all
        L keys, timed alone (a full forward's attention)"""
        import torch
        cfg = self.cfg
        qall = self.W.queries(cfg, device=self.dev, b=cfg.L)
        out = torch.empty((cfg.B, cfg.Hq, cfg.L, cfg.d), dtype=torch.bfloat16, device=self.dev)
        run = lambda: self.D.dllm_block_attention(self.cache, qall, out=out)
        run()
        torch.cuda.synchronize()
        e0, e1 = Event(), Event()
        e0.record()
        for _ in range(reps):
            run()
        e1.record()
        torch.cuda.synchronize()
        return 1000.0 * e0.elapsed_time(e1) / reps


class FfnStep:
    """One FFN of a LLaDA-shaped layer in per-group FP8 on M tokens."""

    def __init__(self, D, W, dev, M=16 * 2048):
        import torch
        self.D, self.W, self.M = D, W, M
        self.K, self.I = W.FFN_HIDDEN, W.FFN_INTER
        self.x, self.res, self.gamma, w_gu, w_out = W.ffn_inputs(M, seed=21, device=dev)
        self.w_gu_bf16, self.w_out_bf16 = w_gu, w_out
        self.cgu, self.sgu = D.dllm_fp8_quant_weight(w_gu)
        self.cout, self.sout = D.dllm_fp8_quant_weight(w_out)
        self.r_out = torch.empty_like(self.x)
        self.ca = torch.empty((M, self.K), dtype=torch.uint8, device=dev)
        self.sa = torch.empty((self.K // 128, M), dtype=torch.uint8, device=dev)
        self.ch = torch.empty((M, self.I), dtype=torch.uint8, device=dev)
        self.sh = torch.empty((self.I // 128, M), dtype=torch.uint8, device=dev)
        self.out = torch.empty((M, self.K), dtype=torch.bfloat16, device=dev)
        self.facache = False

    def calls(self):
        D = self.D
        return [
            ("fp8_addnorm", lambda: D.dllm_fp8_addnorm_quant(self.x, self.res, self.gamma, eps=1e-6,
                                                             residual_out=self.r_out, codes=self.ca, scales=self.sa)),
            ("fp8_gateup", lambda: D.dllm_fp8_gemm_swiglu(self.ca, self.sa, self.cgu, self.sgu, out_codes=self.ch,
                                                          out_scales=self.sh)),
            ("fp8_ffout", lambda: D.dllm_fp8_gemm(self.ch, self.sh, self.cout, self.sout, out=self.out)),
        ]

    def algorithmic_bytes(self):
        M, K, I = self.M, self.K, self.I
        return {
            # x, residual in, residual out (bf16), gamma, codes and scales out
            "fp8_addnorm": M * K * 2 * 3 + K * 2 + M * K + M * K // 128,
            # activation codes and scales, weight codes and scales, SwiGLU codes and scales out
            "fp8_gateup": M * K + M * K // 128 + 2 * I * K + 2 * I * K // 16384 + M * I + M * I // 128,
            "fp8_ffout": M * I + M * I // 128 + K * I + K * I // 16384 + M * K * 2,
        }

    def algorithmic_flops(self):
        M, K, I = self.M, self.K, self.I
        return {"fp8_gateup": 2 * M * 2 * I * K, "fp8_ffout": 2 * M * K * I}


class PolicyStep:
    """Stability mask with the ramped radius and refresh schedule, then the
    quota eviction, on B x L positions with fixed step statistics."""

    def __init__(self, D, W, cfg, dev):
        import torch
        self.D, self.W, self.cfg = D, W, cfg
        B, L = cfg.B, cfg.L
        self.B, self.L = B, L
        logits = W.logits(cfg, device=dev)
        am, mp, en = D.dllm_vocab_stats(logits, V=cfg.V)
        del logits
        self.am, self.mp, self.en = am.view(B, L), mp.view(B, L), en.view(B, L)
        self.st = D.StabilityState(B, L, cfg.D, device=dev)
        self.refresh = D.dllm_refresh_interval(cfg.T)
        self.kw = dict(K=cfg.K, tau=cfg.tau, R=cfg.R, alpha=cfg.alpha, beta=cfg.beta, lam=cfg.lam,
                       conf_thresh=cfg.conf_thresh, V=cfg.V, R_early=0, T_steps=cfg.T,
                       refresh_every=self.refresh)
        self.st.decay_table(cfg.lam)
        self.quota_host = D.dllm_cache_quotas([L] * B, B * L // 2, 0.2)
        self.quota = torch.from_numpy(self.quota_host).to(dev)
        self.evicted = torch.zeros(B, dtype=torch.int32, device=dev)
        self.step_t = torch.zeros(B, dtype=torch.int32, device=dev)
        self.facache = False
        self.attn_split = False

    def calls(self):
        D = self.D
        return [
            ("stability", lambda: D.dllm_stability_mask(self.st, self.step_t, None, self.am, self.mp, self.en,
                                                        advance_step=True, **self.kw)),
            ("evict", lambda: D.dllm_evict_by_confidence(self.st, self.quota, None, self.evicted)),
        ]

    def algorithmic_bytes(self):
        BL, K = self.B * self.L, self.cfg.K
        return {
            # as the decode step's stability kernel
            "stability": BL * (12 + 12 + 12 * (K - 1) + 2 * 9 + 9),
            # conf (4), cached read and write (2), mask read and write (2),
            # next positions (4), quota and counts
            "evict": BL * 12 + self.B * 12,
        }

    def algorithmic_flops(self):
        return {}

    def evict_longctx_us(self, W, dev, reps=20):
        """the eviction alone on 4 x 32768 positions with a quota of 8192
        (the sink + rolling budget of the long-context workload), every
        position recomputed: the selection runs on each call"""
        import numpy as np
        import torch
        c = W.CONFIGS["longctx"]
        st = self.D.StabilityState(c.B, c.L, 2, device=dev)
        g = torch.Generator(device="cpu").manual_seed(c.seed)
        st.conf.copy_(torch.floor(torch.rand((c.B, c.L), generator=g) * 4096) / 4096)
        st.mask.zero_()
        quota = torch.full((c.B,), c.sinks + c.rolling, dtype=torch.int32, device=dev)
        run = lambda: self.D.dllm_evict_by_confidence(st, quota, None)
        run()
        torch.cuda.synchronize()
        e0, e1 = Event(), Event()
        e0.record()
        for _ in range(reps):
            run()
        e1.record()
        torch.cuda.synchronize()
        return 1000.0 * e0.elapsed_time(e1) / reps


def run_step(step, events=None, flush=None):
    """one step: every call in order on the current stream; with events, an
    event pair around each call (after `flush`, when given)"""
    for name, fn in step.calls():
        if events is not None:
            if flush is not None:
                flush()
            events[name][0].record()
        fn()
        if events is not None:
            events[name][1].record()


def verify_inputs(B, L, n, Wn, seed, dev, block_at_end=False):
    """seeded decodes: n ascending positions per sequence in a cluster,
    marginals U(0.3, 1), pair joints = marginal^2 x a log-normal factor, a
    tenth of them scaled below the conflict threshold"""
    import torch
    g = torch.Generator(device="cpu").manual_seed(seed)
    if block_at_end:
        dec = torch.arange(L - n, L, dtype=torch.int32).repeat(B, 1)
    else:
        starts = torch.randint(0, L - 2 * n + 1, (B, 1), generator=g)
        picks = torch.rand((B, 2 * n), generator=g).argsort(dim=1)[:, :n].sort(dim=1).values
        dec = (starts + picks).to(torch.int32)
    pm = 0.3 + 0.7 * torch.rand((B, n), generator=g)
    fac = torch.exp(0.4 * torch.randn((B, n, Wn - 1), generator=g))
    fac = torch.where(torch.rand((B, n, Wn - 1), generator=g) < 0.1, fac * 0.3, fac)
    pj = pm[:, :, None] * pm[:, :, None] * fac
    return dec.to(dev), pm.float().to(dev), pj.float().to(dev)


class VerifyStep:
    """Self-verification of one step's parallel decodes."""

    def __init__(self, D, W, cfg, dev):
        import torch
        self.D, self.W, self.cfg = D, W, cfg
        self.B, self.L, self.n, self.Wn, self.tau = cfg.B, cfg.L, 16, 4, 0.5
        self.dec, self.pm, self.pj = verify_inputs(self.B, self.L, self.n, self.Wn, 4242, dev)
        self.st = D.StabilityState(self.B, self.L, 2, device=dev)
        self.st.mask.zero_()
        self.st.stable.fill_(1)
        self.st.cached.fill_(1)
        self.rollback = torch.empty((self.B, self.L), dtype=torch.uint8, device=dev)
        self.nrb = torch.zeros(self.B, dtype=torch.int32, device=dev)
        self.rbp = torch.empty((self.B, self.n), dtype=torch.int32, device=dev)
        self.facache = False
        self.attn_split = False

    def calls(self):
        return [("verify", lambda: self.D.dllm_self_verify(self.st, self.dec, self.pm, self.pj, self.Wn, self.tau,
                                                           rollback=self.rollback, n_rollback=self.nrb,
                                                           rb_pos=self.rbp))]

    def algorithmic_bytes(self):
        B, L, n, Wn = self.B, self.L, self.n, self.Wn
        # decodes in (positions, marginals, joints); withdrawal flags out, the
        # mask read, next positions out; counts
        return {"verify": B * (n * (8 + 4 * (Wn - 1)) + L * (1 + 1 + 4) + 12)}

    def algorithmic_flops(self):
        return {}

    def longctx_us(self, dev, reps=20):
        """the same call at the long-context shape: 4 x 32768, the 64-position
        block at the end decoded at once"""
        import torch
        c = self.W.CONFIGS["longctx"]
        dec, pm, pj = verify_inputs(c.B, c.L, c.b, self.Wn, 4243, dev, block_at_end=True)
        st = self.D.StabilityState(c.B, c.L, 2, device=dev)
        st.mask.zero_()
        rb = torch.empty((c.B, c.L), dtype=torch.uint8, device=dev)
        run = lambda: self.D.dllm_self_verify(st, dec, pm, pj, self.Wn, self.tau, rollback=rb)
        run()
        torch.cuda.synchronize()
        e0, e1 = Event(), Event()
        e0.record()
        for _ in range(reps):
            run()
        e1.record()
        torch.cuda.synchronize()
        return 1000.0 * e0.elapsed_time(e1) / reps


def cpu_info():
    """the host CPU's model name and the cores this process may run on"""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        nproc = len(os.sched_getaffinity(0))
    except AttributeError:
        nproc = os.cpu_count() or 1
    return model, nproc


def host_threads():
    """OpenMP threads for the oracle: every core this process may use, or the
    host's share for this GPU where OMP_NUM_THREADS sets one"""
    _, nproc = cpu_info()
    env = os.environ.get("OMP_NUM_THREADS")
    return max(1, min(nproc, int(env))) if env and env.isdigit() else nproc


def cpu_baseline_verify(step, W, frac=1.0):
    """The oracle's self-verification on the whole step."""
    import numpy as np

    import oracle
    dec, pm, pj = (t.cpu().numpy() for t in (step.dec, step.pm, step.pj))
    reps = max(2, int(20 * frac))
    t0 = time.perf_counter()
    for _ in range(reps):
        mask = np.zeros((step.B, step.L), np.uint8)
        oracle.self_verify(step.L, dec, pm, pj, step.Wn, step.tau, mask)
    dt = (time.perf_counter() - t0) / reps
    return dt, f"{reps} whole steps ({step.B} x {step.L} positions, {step.n} decoded each)"


def cpu_baseline_policies(step, W, frac=1.0):
    """The oracle's stability step and eviction on the whole step (the
    bench's shape is small enough)."""
    import numpy as np

    import oracle
    B, L, cfg = step.B, step.L, step.cfg
    ost = oracle.StabilityState(B, L, cfg.D)
    am, mp, en = (t.cpu().numpy() for t in (step.am, step.mp, step.en))
    reps = max(2, int(6 * frac))
    t0 = time.perf_counter()
    for s in range(reps):
        r = oracle.stability_step(ost, s, None, am, mp, en, **step.kw)
        oracle.evict_by_confidence(ost, r["conf"].astype(np.float32), step.quota_host, None, r["mask"])
    dt = (time.perf_counter() - t0) / reps
    return dt, f"{reps} whole steps (stability step + eviction, {B} x {L} positions)"


def cpu_baseline_ffn(step, W, frac=1.0):
    """The oracle's chain on a bounded sample of token rows: add & norm +
    quantisation, Gate-Up + SwiGLU + quantisation, FF-Out; scaled to
    steps/s.  The weight quantisation (once per model) is not timed."""
    import numpy as np

    import oracle
    n = 4 if frac >= 1.0 else 1
    rows = slice(0, n)
    cgu, sgu = oracle.fp8_quant_weight(W.as_numpy_bits(step.w_gu_bf16), oracle.BF16)
    cout, sout = oracle.fp8_quant_weight(W.as_numpy_bits(step.w_out_bf16), oracle.BF16)
    x, r, g = (W.as_numpy_bits(t) for t in (step.x[rows], step.res[rows], step.gamma))
    t0 = time.perf_counter()
    _, y = oracle.addnorm(x, r, g, 1e-6, oracle.BF16)
    ca, sa = oracle.fp8_quant_rows(y, oracle.F64)
    c = oracle.fp8_gemm(ca, sa, cgu, sgu)
    blk = c.reshape(n, c.shape[1] // 256, 2, 128)
    h = oracle.swiglu(blk[:, :, 0, :].reshape(n, -1), blk[:, :, 1, :].reshape(n, -1))
    ch, sh = oracle.fp8_quant_rows(h, oracle.F64)
    oracle.fp8_gemm(ch, sh, cout, sout)
    dt = (time.perf_counter() - t0) * step.M / n
    return dt, f"the FFN chain on {n} of {step.M} token rows, scaled linearly to the step"


def cpu_baseline(step, D, W, cfg, frac=1.0):
    """The oracle as it stands, on a bounded sample of the same step, on the
    host's cores; scaled to seconds per step."""
    import numpy as np
    import torch

    import oracle
    t_total = 0.0
    parts = []
    if step.has_vocab:
        n = max(16, min(step.N, int(1024 * frac)))
        host = W.as_numpy_bits(step.logits[:n])
        t0 = time.perf_counter()
        oracle.vocab_stats(host, W.BF16 if step.logits.dtype == torch.bfloat16 else W.F32, V=cfg.V)
        dt = (time.perf_counter() - t0) * step.N / n
        t_total += dt
        parts.append(f"vocab stats on {n} of {step.N} rows")
    if step.has_attn:
        ck, cv = W.as_numpy_bits(step.cache.k), W.as_numpy_bits(step.cache.v)
        ks = step.cache.k_scale.cpu().numpy() if step.cache.k_scale is not None else None
        vs = step.cache.v_scale.cpu().numpy() if step.cache.v_scale is not None else None
        n_heads = cfg.B * cfg.Hq
        ns = max(1, min(n_heads, int(24 * frac)))
        heads = np.stack([np.arange(ns) % cfg.B, np.arange(ns) % cfg.Hq], 1).astype(np.int32)
        kid = step.key_idx.cpu().numpy() if step.key_idx is not None else None
        t0 = time.perf_counter()
        oracle.block_attention(ck, cv, ks, vs, cfg.kv_dtype, W.as_numpy_bits(step.q), W.BF16,
                               key_idx=kid, heads=heads)
        t_total += (time.perf_counter() - t0) * n_heads / ns
        t0 = time.perf_counter()
        oracle.scatter_kv(ck, cv, ks, vs, cfg.kv_dtype, W.as_numpy_bits(step.kn), W.as_numpy_bits(step.vn),
                          W.BF16, step.pos.cpu().numpy())
        t_total += time.perf_counter() - t0
        parts.append(f"attention on {ns} of {n_heads} (sequence, head) pairs; full scatter")
    if step.facache:
        ck, cv = W.as_numpy_bits(step.cache.k), W.as_numpy_bits(step.cache.v)
        n_heads = cfg.B * cfg.Hq
        ns = max(1, min(n_heads, int(8 * frac)))
        heads = np.stack([np.arange(ns) % cfg.B, np.arange(ns) % cfg.Hq], 1).astype(np.int32)
        mo, ml = step.memo_o.cpu().numpy(), step.memo_lse.cpu().numpy()
        qu = W.as_numpy_bits(step.qu)
        t0 = time.perf_counter()
        oracle.facache_merge(ck, cv, None, None, cfg.kv_dtype, qu, W.BF16, mo, ml,
                             key_idx=step.blk.cpu().numpy(), heads=heads)
        t_total += (time.perf_counter() - t0) * n_heads / ns
        parts.append(f"FACache merge on {ns} of {n_heads} (sequence, head) pairs")
    if step.has_stab:
        ost = oracle.StabilityState(cfg.B, cfg.L, cfg.D)
        am = step.am.cpu().numpy().reshape(cfg.B, cfg.L)
        mp = step.mp.cpu().numpy().reshape(cfg.B, cfg.L)
        en = step.en.cpu().numpy().reshape(cfg.B, cfg.L)
        t0 = time.perf_counter()
        for s in range(3):
            oracle.stability_step(ost, s, None, am, mp, en, **step.kw)
        t_total += (time.perf_counter() - t0) / 3
        parts.append("full stability step")
    return t_total, "; ".join(parts) + "; times scaled linearly to the whole step"


# the seeded inputs of each workload's step, by attribute name (the cache as
# the timed steps leave it: every step writes the same fresh rows)
INPUT_NAMES = ("logits", "q", "kn", "vn", "pos", "key_idx", "qu", "memo_o", "memo_lse",
               "x", "res", "gamma", "w_gu_bf16", "w_out_bf16", "am", "mp", "en", "dec", "pm", "pj")


def inputs_sha256(step):
    """SHA-256 of the bytes of every input of the step (and of the cache)"""
    import torch
    names = [n for n in INPUT_NAMES
             if not (n in ("am", "mp", "en") and getattr(step, "has_vocab", False))]   # outputs there
    tensors = {n: getattr(step, n) for n in names if isinstance(getattr(step, n, None), torch.Tensor)}
    cache = getattr(step, "cache", None)
    if cache is not None:
        for n in ("k", "v", "k_scale", "v_scale"):
            if getattr(cache, n, None) is not None:
                tensors["cache." + n] = getattr(cache, n)
    out = {}
    for n, t in tensors.items():
        h = hashlib.sha256()
        flat = t.contiguous().view(-1).view(torch.uint8)
        for i in range(0, flat.numel(), 1 << 28):             # 256 MiB at a time through host memory
            h.update(flat[i:i + (1 << 28)].cpu().numpy().tobytes())
        out[n] = h.hexdigest()
    return out


def padded_stride_vocab_us(step, W, reps=50):
    """vocab_stats on the same logits in rows padded to a 16-byte multiple
    (the other stride the GPT-2-shaped rows are tested at), back to back"""
    import torch
    N, V = step.logits.shape
    stride = (V + 7) // 8 * 8
    padded = torch.zeros((N, stride), dtype=step.logits.dtype, device=step.logits.device)
    padded[:, :V] = step.logits
    run = lambda: step.D.dllm_vocab_stats(padded[:, :V], V=V, argmax=step.am, maxprob=step.mp,
                                          entropy=step.en, workspace=step.vocab_ws)
    run()
    torch.cuda.synchronize()
    e0, e1 = Event(), Event()
    e0.record()
    for _ in range(reps):
        run()
    e1.record()
    torch.cuda.synchronize()
    us = 1000.0 * e0.elapsed_time(e1) / reps
    del padded
    return stride, us


CPU_BUDGET_S = 12.0     # seconds of oracle runs on every core; half that on one thread


def repeat_timed(call, budget):
    """call() -> (seconds per step, sample), repeated until `budget` seconds
    have passed (at least once): the median, the sample, the repeats and the
    seconds spent"""
    t0 = time.perf_counter()
    dts, sample = [], ""
    while True:
        dt, sample = call()
        dts.append(dt)
        if time.perf_counter() - t0 >= budget:
            break
    return statistics.median(dts), sample, len(dts), time.perf_counter() - t0


def cpu_baseline_line(fn):
    """fn(frac) -> (seconds per step, sample): the oracle on every host core
    this process may use, then on one thread on a quarter of the sample, each
    repeated for a bounded time (median of the repeats)"""
    import oracle
    model, nproc = cpu_info()
    threads = oracle.set_threads(host_threads())
    dt, sample, reps, spent = repeat_timed(lambda: fn(1.0), CPU_BUDGET_S)
    oracle.set_threads(1)
    dt1, sample1, reps1, spent1 = repeat_timed(lambda: fn(0.25), CPU_BUDGET_S / 2)
    oracle.set_threads(threads)
    sig = lambda x: float(f"{x:.4g}")                     # four significant figures
    return {"value": sig(1.0 / dt), "unit": "steps/s", "cores": threads, "kind": "oracle",
            "sample": sample, "repeats": reps, "seconds": round(spent, 1), "cpu_model": model,
            "nproc": nproc, "value_1thread": sig(1.0 / dt1), "sample_1thread": sample1,
            "repeats_1thread": reps1, "seconds_1thread": round(spent1, 1)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); there is no "
              f"multi-GPU path", file=sys.stderr)
        sys.exit(2)
    import torch

    import cached_denoising_amd as D
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration()
        return
    cfg = W.CONFIGS[{"facache": "llada", "ffn": "llada", "policies": "vocab", "verify": "vocab"}.get(
        args.config, args.config)]
    if args.config == "ffn":
        step = FfnStep(D, W, dev)
    elif args.config == "policies":
        step = PolicyStep(D, W, cfg, dev)
    elif args.config == "verify":
        step = VerifyStep(D, W, cfg, dev)
    else:
        step = Step(D, W, cfg, dev, facache=args.config == "facache")
    for _ in range(args.warmup):
        run_step(step)
    torch.cuda.synchronize()

    names = [n for n, _ in step.calls()]
    start = Event()
    end = Event()
    graph = None
    launch = {}
    if not args.eager:
        # the K timed steps as one HIP graph: no launch gaps between the
        # kernels of a step or between steps
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(args.steps):
                run_step(step)
        torch.cuda.synchronize()
        graph.replay()                      # one untimed replay
        torch.cuda.synchronize()
        # one replay launched onto an idle GPU: its events also hold the
        # host's launch of the graph
        start.record()
        graph.replay()
        end.record()
        torch.cuda.synchronize()
        idle_ms = start.elapsed_time(end)
        # the timed replay is queued behind untimed ones (at least 3 ms of
        # GPU work), so the GPU is busy when the host launches it and its
        # events hold only the GPU's time for the K steps
        n_pre = max(1, int(3.0 / max(idle_ms, 1e-3)) + 1)
        torch.cuda.synchronize()
        t_wall = time.perf_counter()
        for _ in range(n_pre):
            graph.replay()
        start.record()
        graph.replay()
        end.record()
        torch.cuda.synchronize()
        t_wall = time.perf_counter() - t_wall
        ms = start.elapsed_time(end) / args.steps
        launch = {"graph_replay_from_idle_ms": round(idle_ms, 4),
                  "graph_launch_overhead_ms": round(idle_ms - ms * args.steps, 4),
                  "untimed_replays_queued_ahead": n_pre}
    else:
        torch.cuda.synchronize()
        t_wall = time.perf_counter()
        start.record()
        for i in range(args.steps):
            run_step(step)
        end.record()
        torch.cuda.synchronize()
        t_wall = time.perf_counter() - t_wall
        ms = start.elapsed_time(end) / args.steps

    # Per-call times, HIP event pairs on the launch stream:
    #   hot   an event pair around each call of 100 eager steps, queued behind
    #         GPU work so that no host launch gap falls inside a pair;
    #   cold  the same with a 1 GiB device read before every call, which
    #         leaves the 256 MB last-level cache and the L2s holding other,
    #         clean data (a write would leave them dirty, and the call would
    #         pay the write-back of someone else's data);
    #   b2b   one event pair around R back-to-back launches of the call alone,
    #         replayed from a captured graph behind 5 ms of queued GPU work:
    #         the kernel's own duration, free of the few microseconds an event
    #         pair adds to every call.
    iters = max(100, args.steps)
    flush_buf = torch.ones(1 << 28, dtype=torch.int32, device=dev)      # 1 GiB
    flush = lambda: flush_buf.amax()                                     # a read of every byte

    def busy(ms_target):
        # queued GPU work while the host enqueues a pass: replays of the
        # timed graph (which keep the clocks where the timed region had
        # them), else reads of the flush buffer
        if graph is not None:
            for _ in range(min(200, max(1, int(ms_target / max(ms * args.steps, 1e-3)) + 1))):
                graph.replay()
        else:
            for _ in range(max(1, int(ms_target / 0.25))):
                flush()

    def pct_stats(t):
        t = sorted(t)
        pct = lambda q: t[min(len(t) - 1, int(round(q * (len(t) - 1))))]
        lo, hi = pct(0.1), pct(0.9)
        mid = [x for x in t if lo <= x <= hi]             # a host hiccup in one call does not move it
        return {"mean": sum(t) / len(t), "tmean": sum(mid) / len(mid), "p10": lo, "p50": pct(0.5), "p90": hi}

    def kernel_pass(cold):
        ev = {n: [[Event() for _ in range(2)] for _ in range(iters)]
              for n in names}
        busy(max(20.0, 0.15 * iters * len(names)))       # about 150 us of host time per call
        for i in range(iters):
            run_step(step, {n: ev[n][i] for n in names}, flush=flush if cold else None)
        torch.cuda.synchronize()
        return {n: pct_stats([1000.0 * e[0].elapsed_time(e[1]) for e in ev[n]]) for n in names}

    hot = kernel_pass(False)
    cold = kernel_pass(True)

    def b2b_pass(rounds=5):
        out = {}
        for n, fn in step.calls():
            reps = int(min(400, max(20, 1000.0 / max(hot[n]["mean"], 1e-3))))   # about 1 ms per replay
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for _ in range(reps):
                    fn()
            g.replay()
            torch.cuda.synchronize()
            for _ in range(20):
                flush()                                  # about 5 ms of queued GPU work
            e0, e1 = Event(), Event()
            e0.record()
            for _ in range(rounds):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            out[n] = {"mean": 1000.0 * e0.elapsed_time(e1) / (reps * rounds), "launches": reps * rounds,
                      "reps": reps}
            del g
        return out

    b2b = b2b_pass()
    del flush_buf
    kernel_timing = ("HIP events without the system-scope fence, on the launch stream: hot/cold = an event pair "
                     "around each call of %d eager steps (cold: after a 1 GiB device read), b2b = one event pair "
                     "around back-to-back launches of the call alone from a captured graph; a cold roofline figure "
                     "is the mean of the cold launches between their 10th and 90th percentiles" % iters)
    per_kernel_us = {n: hot[n]["tmean"] for n in names}
    alg = step.algorithmic_bytes()
    flops = step.algorithmic_flops()
    # the dominant kernel is the one the step spends the most time in; it is
    # bound by the matrix cores when its flops per byte exceed the ridge
    dom = max(per_kernel_us, key=per_kernel_us.get)
    # a working set that fits the 256 MB last-level cache is timed cold for
    # the roofline: the hot figure would be a cache rate, not an HBM one.  A
    # larger one never stays in that cache, and takes the back-to-back figure:
    # in the timed graph the calls run back to back, and a memory-bound call
    # runs slower so than between the eager pass's event pairs (its duration in
    # the graph replays of the kernel trace matches the back-to-back one)
    mall_resident = alg[dom] < 256 * 2 ** 20
    dom_us = cold[dom]["tmean"] if mall_resident else b2b[dom]["mean"]
    traffic = measured_traffic(dom, args.config)
    fp8 = dom.startswith("fp8_")
    peak_mfma = MFMA_FP8_PEAK_TFLOPS if fp8 else MFMA_BF16_PEAK_TFLOPS
    ridge = peak_mfma * 1e12 / (HBM_PEAK_GBS * 1e9)
    if dom in flops and flops[dom] / alg[dom] > ridge:
        achieved = flops[dom] / (dom_us * 1e-6) / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak_mfma,
                    "unit": "TFLOP/s", "frac": round(achieved / peak_mfma, 4),
                    "traffic": traffic, "algorithmic_flops_per_launch": flops[dom]}
    else:
        achieved = alg[dom] / (dom_us * 1e-6) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic}
    roofline.update({"kernel": dom, "algorithmic_bytes_per_launch": alg[dom],
                     "avg_launch_us": round(dom_us, 2), "timing": "cold" if mall_resident else "b2b",
                     "kernel_timing": kernel_timing})
    if dom == "scatter_attention":
        fused = step.cfg.kv_dtype == W.BF16 and step.key_idx is None
        roofline["kernel_note"] = (
            "dllm_scatter_attention call = " +
            ("attn_mfma_kernel writing the block's rows itself" if fused else
             "scatter kernel, then the attention kernel") +
            (" + attn_merge_kernel of the key splits" if step.attn_split else ""))
    if dom == "facache_merge":
        roofline["kernel_note"] = "facache_merge call = attn_shared_kernel started from the memo, one key tile"
    extra = {}
    if step.facache:
        full = step.full_recompute_us()
        # the block's scatter is inside the first call: the FACache side
        # carries it and the full recompute does not
        fa = per_kernel_us["scatter_attention"] + per_kernel_us["facache_merge"]
        extra = {"full_recompute_attention_us": round(full, 1),
                 "facache_attention_us": round(fa, 1),
                 "facache_speedup_vs_full": round(full / fa, 2)}
    if args.config == "policies":
        extra = {"evict_longctx_us": round(step.evict_longctx_us(W, dev), 2),
                 "refresh_every": step.refresh}
    if args.config == "verify":
        extra = {"verify_longctx_us": round(step.longctx_us(dev), 2),
                 "withdrawn_per_step": int(step.nrb.sum().item())}
    if args.config == "gpt2":
        stride, us = padded_stride_vocab_us(step, W)
        extra = {"vocab_stats_padded_stride": stride, "vocab_stats_padded_stride_b2b_us": round(us, 2)}
    if args.no_cpu_baseline:
        cpu = None
    elif args.config == "ffn":
        cpu = cpu_baseline_line(lambda f: cpu_baseline_ffn(step, W, f))
    elif args.config == "policies":
        cpu = cpu_baseline_line(lambda f: cpu_baseline_policies(step, W, f))
    elif args.config == "verify":
        cpu = cpu_baseline_line(lambda f: cpu_baseline_verify(step, W, f))
    else:
        cpu = cpu_baseline_line(lambda f: cpu_baseline(step, D, W, cfg, f))
    desc = {
        "gpt2": "GPT-2-small-shaped decode step: B=8, L=1024, 12 heads x d64, bf16 K/V cache, "
                "block b=32 at a random offset, vocab 50257 bf16 logits for all 8192 positions, "
                "K=3 tau=0.95 R=2",
        "llada": "LLaDA-8B-shaped SAR step: B=16, L=2048, 32 heads x d128, bf16 K/V, block 32, "
                 "vocab 126464 bf16 logits for the 512 block rows",
        "vocab": "vocab-stats sweep: 32768 rows x 126464 bf16 logits, 64-step ring, K=3 tau=0.9 R=3",
        "longctx": "long-context step: B=4, L=32768, 32/8 GQA heads x d128, e4m3 K/V with "
                   "per-128 scales, block 64, 4 sinks + 8188 rolling keys",
        "ffn": "LLaDA-8B-shaped FFN of one layer in per-group FP8 on a 16 x 2048 step: 32768 tokens, "
               "hidden 4096, SwiGLU width 12288, e4m3 codes with E8M0 scales per 1x128 activation "
               "group and 128x128 weight block (add & norm + quant, Gate-Up + SwiGLU + quant, "
               "FF-Out to bf16)",
        "policies": "decode policies on the vocab sweep's 64 x 512 positions: stability mask with the "
                    "window radius ramped 0 -> 3 over 64 steps and a full refresh every 6 steps, then "
                    "confidence-ordered eviction to per-request quotas (half the positions, 20% "
                    "guaranteed each)",
        "verify": "self-verification of one step's parallel decodes on the vocab sweep's 64 x 512 "
                  "positions: 16 decoded per sequence, window 4, tau 0.5, conflicts planted in a tenth "
                  "of the pair joints",
        "facache": "LLaDA-8B-shaped first-layer attention of a later step of a block, with FACache: "
                   "B=16, L=2048, 32 heads x d128, bf16 K/V, block 32 (scatter, block queries over "
                   "all keys, 2016 outside queries from their memo over the block keys)",
    }[args.config]
    metric = {"facache": "first-layer attention steps/sec with FACache (scatter + block attention + memo merge)",
              "ffn": "FP8 FFN steps/sec (add & norm + quant, Gate-Up + SwiGLU + quant, FF-Out)",
              "policies": "decode-policy steps/sec (stability mask with ramp + refresh, quota eviction)",
              "verify": "self-verification steps/sec (conflict scores, withdrawal, mask recompaction)"}.get(
        args.config, METRIC)
    dtype = {"ffn": "e4m3 x e4m3 -> f32 (E8M0 group scales)", "policies": "f64 decisions, f32 keys",
             "verify": "f64 scores"}.get(
        args.config, "bf16")
    line = {
        "metric": metric, "value": round(1000.0 / ms, 2), "unit": "steps/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
        "data": "synthetic",
        "config": ({"workload": desc, "tokens": step.M, "hidden": step.K, "ffn_width": step.I}
                   if args.config == "ffn" else
                   {"workload": desc, "name": cfg.name, "B": cfg.B, "L": cfg.L, "heads": cfg.Hq,
                    "kv_heads": cfg.Hkv, "d_head": cfg.d, "block": cfg.b, "vocab": cfg.V})
                  | {"launch": "eager" if graph is None else "hip graph of the timed steps"},
        "kernels_us": {n: round(v, 2) for n, v in per_kernel_us.items()},
        "kernels_us_pct": {n: {"hot": {k: round(v, 2) for k, v in hot[n].items()},
                               "cold": {k: round(v, 2) for k, v in cold[n].items()},
                               "b2b": {k: round(v, 2) for k, v in b2b[n].items()}} for n in names},
        **launch,
        "roofline": roofline,
        **extra,
        "cpu_baseline": cpu,
        "inputs_sha256": inputs_sha256(step),
        "wall_s": round(t_wall, 3),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
