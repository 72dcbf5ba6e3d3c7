"""A decode step captured in a HIP graph replays to the same results as the
same step launched eagerly: every replay is checked bit for bit, with the
program's own eager work and synchronisations between replays.  The
per-sequence step numbers live in device memory and the stability kernel
advances them, so successive replays are successive steps."""
import dataclasses

import pytest
import torch

import workloads as W
from gpu_util import need_gpu, new_cache, say

pytestmark = pytest.mark.gpu


class Step:
    def __init__(self, D, cfg):
        self.D, self.cfg = D, cfg
        self.cache = new_cache(D, cfg.B, cfg.Hkv, cfg.L, cfg.d, cfg.kv_dtype)
        k, v = W.kv_rows(cfg, device="cuda")
        D.dllm_scatter_kv(self.cache, k, v,
                          torch.arange(cfg.L, dtype=torch.int32, device="cuda").repeat(cfg.B, 1))
        self.kn, self.vn = W.kv_rows(cfg, device="cuda", which="fresh")
        self.pos = W.block_positions(cfg, "cuda")
        self.q = W.queries(cfg, device="cuda")
        self.out = torch.empty((cfg.B, cfg.Hq, cfg.b, cfg.d), dtype=torch.bfloat16, device="cuda")
        ws = D.dllm_block_attention_workspace(self.cache, W.BF16, cfg.Hq, cfg.b, cfg.L)
        self.ws = torch.empty(max(ws, 16), dtype=torch.uint8, device="cuda")
        self.logits = [W.logits(cfg, device="cuda", step=s) for s in range(2)]
        N = self.logits[0].shape[0]
        self.am = torch.empty(N, dtype=torch.int32, device="cuda")
        self.mp = torch.empty(N, device="cuda")
        self.en = torch.empty(N, device="cuda")
        self.vws = torch.empty(max(D.dllm_vocab_stats_workspace(N, cfg.V), 16), dtype=torch.uint8,
                               device="cuda")
        self.st = D.StabilityState(cfg.B, cfg.L, cfg.D)
        self.step_t = torch.zeros(cfg.B, dtype=torch.int32, device="cuda")
        self.kw = dict(K=cfg.K, tau=cfg.tau, R=cfg.R, V=cfg.V)

    def run(self, which):
        D, cfg = self.D, self.cfg
        D.dllm_scatter_kv(self.cache, self.kn, self.vn, self.pos)
        D.dllm_block_attention(self.cache, self.q, out=self.out, workspace=self.ws)
        D.dllm_vocab_stats(self.logits[which], V=cfg.V, argmax=self.am, maxprob=self.mp,
                           entropy=self.en, workspace=self.vws)
        D.dllm_stability_mask(self.st, self.step_t, None, self.am.view(cfg.B, cfg.L),
                              self.mp.view(cfg.B, cfg.L), self.en.view(cfg.B, cfg.L), advance_step=True,
                              **self.kw)

    def snapshot(self):
        st = self.st
        return [t.clone() for t in (self.out, self.am, self.mp, self.en, st.mask, st.stable, st.ring_step,
                                    st.ring_argmax, st.next_pos, st.count, self.step_t)]


def test_graph_replays_match_eager():
    D = need_gpu()
    # a small GPT-2-shaped step whose positions settle within a few steps
    cfg = dataclasses.replace(W.CONFIGS["gpt2"], B=2, L=256, V=4096, V_stride=4096, peak_lo=14.0,
                              peak_hi=14.0, K=2, tau=0.9)
    say("graph capture: eager reference")
    ref = Step(D, cfg)
    expect = []
    for i in range(4):
        ref.run(i % 2)
        torch.cuda.synchronize()
        expect.append(ref.snapshot())
    say("graph capture: capture and replays")
    g_step = Step(D, cfg)
    torch.cuda.synchronize()
    graphs = []
    for which in range(2):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            g_step.run(which)
        graphs.append(g)
    torch.cuda.synchronize()
    # capturing runs nothing: the state is still the initial one
    assert int(g_step.step_t.abs().sum()) == 0
    for i in range(4):
        graphs[i % 2].replay()
        torch.cuda.synchronize()
        # eager work between replays
        junk = torch.randn(1000, device="cuda").sum()
        torch.cuda.synchronize()
        got = g_step.snapshot()
        for a, b in zip(got, expect[i]):
            assert torch.equal(a, b), f"replay {i}"
        del junk
    assert int(g_step.st.stable.sum()) > 0
