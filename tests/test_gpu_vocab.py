"""GPU parity of dllm_vocab_stats against the oracle.

Bar: argmax bit-exact; maxprob within 1e-3 absolute (stated) and 1e-4
relative (derived: the stated absolute bar is loose where max-probs are
~1e-3); entropy within 1e-3 absolute (stated)."""
import dataclasses

import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import bits, need_gpu, say

pytestmark = pytest.mark.gpu

MP_ABS, MP_REL, H_ABS = 1e-3, 1e-4, 1e-3


def _compare(orc, logits, dtype, V, rows=None, label=""):
    D = need_gpu()
    say("vocab_stats", label, tuple(logits.shape), "V", V)
    am, mp, en = D.dllm_vocab_stats(logits, V=V)
    torch.cuda.synchronize()
    am, mp, en = am.cpu().numpy(), mp.cpu().numpy(), en.cpu().numpy()
    if rows is None:
        host = bits(logits)
        oam, omp, oen = orc.vocab_stats(host, dtype, V=V)
        sel = slice(None)
    else:
        host = bits(logits[torch.as_tensor(rows, device=logits.device)])
        oam, omp, oen = orc.vocab_stats(host, dtype, V=V)
        sel = np.asarray(rows)
    am, mp, en = am[sel], mp[sel], en[sel]
    bad = np.flatnonzero(am != oam)
    assert bad.size == 0, (label, bad[:5], am[bad[:5]], oam[bad[:5]])
    assert np.all(np.abs(mp - omp) <= MP_ABS), label
    assert np.all(np.abs(mp - omp) <= MP_REL * omp + 1e-12), (label, np.max(np.abs(mp - omp) / omp))
    assert np.all(np.abs(en - oen) <= H_ABS), (label, np.max(np.abs(en - oen)))
    return am, mp, en


def test_vocab_tiny(orc):
    cfg = W.CONFIGS["tiny"]
    for step in range(3):
        x = W.logits(cfg, device="cuda", step=step)
        _compare(orc, x, W.F32, cfg.V, label=f"tiny step {step}")


def test_vocab_special_rows(orc):
    V = 5003
    x = torch.randn((12, V)) * 2
    x[0] = 0.25                                           # uniform
    x[1] = -float("inf"); x[1, 4321] = 3.0                # one finite logit
    x[2] = -float("inf"); x[2, [17, 4000]] = -1.5         # two-way tie, rest -inf
    x[3, [5, 9, 4999]] = 40.0                             # three-way tie among finite
    x[4] = -3000.0; x[4, 77] = 0.0                        # gap of 3000
    x[5, :2500] = -float("inf")                           # half masked
    x[6, V - 1] = 50.0                                    # max in the last column
    x[7, 0] = 50.0                                        # max in the first column
    for dt, tdt in ((W.F32, torch.float32), (W.BF16, torch.bfloat16)):
        xd = x.to(tdt).cuda()
        am, mp, en = _compare(orc, xd, dt, V, label=f"special dtype {dt}")
        assert am[0] == 0 and am[1] == 4321 and am[2] == 17 and am[3] == 5 and am[6] == V - 1


@pytest.mark.parametrize("V,stride,N", [(50257, 50257, 40), (50257, 50264, 40), (126464, 126464, 24),
                                        (1000, 1003, 700), (7, 9, 33), (70001, 70001, 3)])
def test_vocab_strides_and_splits(orc, V, stride, N):
    """odd strides (rows not 16-byte aligned), few rows (rows split across
    workgroups and merged), ragged tails"""
    g = torch.Generator().manual_seed(V + stride + N)
    x = torch.randn((N, stride), generator=g) * 1.5
    x[torch.arange(N), torch.randint(0, V, (N,), generator=g)] += 7.0
    x[:, V:] = 1e4                                        # padding must be ignored
    for dt, tdt in ((W.BF16, torch.bfloat16), (W.F32, torch.float32)):
        _compare(orc, x.to(tdt).cuda(), dt, V, label=f"V{V} stride{stride} N{N} dt{dt}")


def test_vocab_edge_sizes(orc):
    """no rows; one logit per row (max-prob exactly 1, entropy exactly 0);
    rows shorter than one 16-byte vector; a view whose rows all start off
    the 16-byte grid (the head and tail of every row peeled)"""
    D = need_gpu()
    for dt, tdt in ((W.F32, torch.float32), (W.BF16, torch.bfloat16)):
        am, mp, en = D.dllm_vocab_stats(torch.zeros((0, 10), dtype=tdt, device="cuda"))
        assert am.numel() == mp.numel() == en.numel() == 0
        x = torch.randn((37, 3), generator=torch.Generator().manual_seed(5)) * 4
        am, mp, en = _compare(orc, x.to(tdt).cuda(), dt, 1, label=f"V1 dt{dt}")
        # the exponent argument is x log2(e) minus the rounded m log2(e), so
        # the one probability is 1 within the rounding of that product
        assert np.all(am == 0)
        assert np.all(np.abs(mp - 1.0) <= 4e-7) and np.all(np.abs(en) <= 1e-6), (mp.min(), mp.max(), en)
        for V in (2, 3, 7, 8, 9):
            _compare(orc, x.repeat(1, 3).to(tdt).cuda(), dt, V, label=f"V{V} dt{dt}")
        big = torch.randn((50, 1100), generator=torch.Generator().manual_seed(6)).to(tdt).cuda()
        view = big[:, 5:5 + 1000]                            # row stride 1100, start off the grid
        _compare(orc, view, dt, 1000, label=f"offset view dt{dt}")


def test_vocab_gpt2_full_sampled(orc):
    cfg = W.CONFIGS["gpt2"]
    x = W.logits(cfg, device="cuda")
    rows = np.random.default_rng(0).choice(x.shape[0], 192, replace=False)
    _compare(orc, x, W.BF16, cfg.V, rows=rows, label="gpt2 8192x50257")
    # padded-stride variant of the same logits
    xp = torch.zeros((x.shape[0], 50264), dtype=x.dtype, device="cuda")
    xp[:, :cfg.V] = x
    _compare(orc, xp, W.BF16, cfg.V, rows=rows, label="gpt2 stride 50264")


def test_vocab_llada_block_rows(orc):
    cfg = W.CONFIGS["llada"]
    x = W.logits(cfg, device="cuda")                        # 512 x 126464: every row
    _compare(orc, x, W.BF16, cfg.V, label="llada 512x126464")


def test_vocab_sweep_full_sampled(orc):
    cfg = W.CONFIGS["vocab"]
    x = W.logits(cfg, device="cuda")                        # 32768 x 126464 bf16, 8.3 GB
    xf = x[:, :].float()
    top2 = torch.topk(xf, 2, dim=1).values
    tie_rows = torch.nonzero(top2[:, 0] == top2[:, 1]).flatten().cpu().numpy()
    del xf, top2
    assert tie_rows.size >= 300                             # ~1% planted exact ties
    rng = np.random.default_rng(1)
    rows = np.unique(np.concatenate([rng.choice(x.shape[0], 128, replace=False), tie_rows[:64],
                                     [0, x.shape[0] - 1]]))
    _compare(orc, x, W.BF16, cfg.V, rows=rows, label="vocab sweep 32768x126464")


def test_vocab_deterministic():
    D = need_gpu()
    cfg = dataclasses.replace(W.CONFIGS["llada"])
    x = W.logits(cfg, device="cuda")
    say("vocab determinism")
    a = [t.clone() for t in D.dllm_vocab_stats(x)]
    b = D.dllm_vocab_stats(x)
    for u, v in zip(a, b):
        assert torch.equal(u, v)
