"""GPU parity of dllm_stability_reset / dllm_stability_mask against the
oracle on shared step statistics: stable flags, masks, next positions,
counts, all-stable flags, the ring state and the float32 confidence, all bit
for bit.  Both sides evaluate the confidence as the same chain of single
float64 operations (no fused multiply-add) on the same age factor (the C
library's exp of the same product), so its value and every decision on it
are equal by construction; a threshold set to a confidence's exact float64
value pins the strict comparison."""
import dataclasses
import json
import os

import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import need_gpu, say

pytestmark = pytest.mark.gpu
GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _state_equal(gst, ost, label):
    for name in ("ring_argmax", "ring_maxprob", "ring_step", "entropy_latest", "t_write", "stable"):
        a = getattr(gst, name).cpu().numpy()
        b = getattr(ost, name)
        assert np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                              b.view(np.uint32) if b.dtype == np.float32 else b), (label, name)


def _step(orc, D, gst, ost, step, pos, am, mp, en, kw, label):
    say("stability", label, "step", step)
    D.dllm_stability_mask(gst, step, None if pos is None else pos.cuda(), am.cuda(), mp.cuda(), en.cuda(), **kw)
    torch.cuda.synchronize()
    r = orc.stability_step(ost, step, None if pos is None else pos.numpy(), am.numpy(), mp.numpy(),
                           en.numpy(), **kw)
    _state_equal(gst, ost, (label, step))
    mask = gst.mask.cpu().numpy()
    if not np.array_equal(mask, r["mask"]):
        conf = r["conf"]
        margin = np.abs(conf - kw.get("conf_thresh", 0.0)).min()
        raise AssertionError(f"{label} step {step}: mask differs; closest confidence margin {margin:.3e}")
    assert np.array_equal(gst.next_pos.cpu().numpy(), r["next_pos"]), (label, step)
    assert np.array_equal(gst.count.cpu().numpy(), r["count"]), (label, step)
    assert np.array_equal(gst.all_stable.cpu().numpy(), r["all_stable"]), (label, step)
    conf32 = r["conf"].astype(np.float32)
    assert np.array_equal(gst.conf.cpu().numpy().view(np.uint32), conf32.view(np.uint32)), (label, step)
    return r


def _kw(cfg):
    return dict(K=cfg.K, tau=cfg.tau, R=cfg.R, alpha=cfg.alpha, beta=cfg.beta, lam=cfg.lam,
                conf_thresh=cfg.conf_thresh, V=max(cfg.V, 2))


def test_swd_page_example_gpu(orc):
    D = need_gpu()
    g = json.load(open(os.path.join(GOLD, "swd_window_example.json")))
    L = g["L"]
    gst = D.StabilityState(1, L, 3)
    st = torch.zeros((1, L), dtype=torch.uint8)
    st[0, torch.tensor(g["stable_1based"]) - 1] = 1
    gst.stable.copy_(st)
    e = torch.zeros((1, 0))
    say("swd example")
    D.dllm_stability_mask(gst, 5, torch.zeros((1, 0), dtype=torch.int32, device="cuda"),
                          e.int().cuda(), e.cuda(), e.cuda(), K=3, tau=0.95, R=g["R"], V=100)
    torch.cuda.synchronize()
    assert (torch.nonzero(gst.mask[0]).flatten().cpu() + 1).tolist() == g["mask_1based"]


@pytest.mark.parametrize("peak", [8.0, 12.0])
def test_tiny_trajectory_shared_stats(orc, peak):
    """16 steps of the tiny workload: GPU vocab stats of each step's logits feed
    both the GPU kernel and the oracle, with the confidence gate on and off.
    With the stated +8 peak over 512 N(0,1) logits the max-prob is about 0.78,
    below tau = 0.95, so nothing settles; +12 gives about 0.995 and the
    planted positions settle after K steps."""
    D = need_gpu()
    cfg = dataclasses.replace(W.CONFIGS["tiny"], peak_lo=peak, peak_hi=peak)
    for thresh in (cfg.conf_thresh, 0.0):
        kw = dict(_kw(cfg), conf_thresh=thresh)
        gst = D.StabilityState(cfg.B, cfg.L, cfg.D)
        ost = orc.StabilityState(cfg.B, cfg.L, cfg.D)
        n_stable = []
        for s in range(cfg.T):
            x = W.logits(cfg, device="cuda", step=s)
            am, mp, en = (t.cpu() for t in D.dllm_vocab_stats(x))
            _step(orc, D, gst, ost, s, None, am.view(1, -1), mp.view(1, -1), en.view(1, -1), kw,
                  f"tiny thresh {thresh}")
            n_stable.append(int(ost.stable.sum()))
        if peak > 10:
            assert n_stable[-1] > 0                   # the planted peaks settle
            assert n_stable[cfg.K - 2] == 0           # not before K steps


def _structured(cfg, B, L, T, seed):
    """per-position settle steps; after settling the argmax is the planted
    token and the max-prob is U(0.85, 1): many means near tau"""
    rng = np.random.default_rng(seed)
    settle = rng.integers(0, T, (B, L))
    tok = rng.integers(0, 50, (B, L))
    ams, mps, ens = [], [], []
    for s in range(T):
        noise_tok = rng.integers(0, 50, (B, L))
        settled = s >= settle
        am = np.where(settled, tok, noise_tok).astype(np.int32)
        mp = np.where(settled, rng.uniform(0.85, 1.0, (B, L)), rng.uniform(0.0, 0.9, (B, L))).astype(np.float32)
        en = np.where(settled, rng.uniform(0, 0.5, (B, L)), rng.uniform(1, 11, (B, L))).astype(np.float32)
        ams.append(am); mps.append(mp); ens.append(en)
    return ams, mps, ens


@pytest.mark.parametrize("thresh", [0.8, 0.0])
def test_sweep_structured_history(orc, thresh):
    D = need_gpu()
    cfg = W.CONFIGS["vocab"]
    B, L, T = cfg.B, cfg.L, 24
    kw = dict(_kw(cfg), conf_thresh=thresh)
    ams, mps, ens = _structured(cfg, B, L, T, seed=7)
    gst = D.StabilityState(B, L, cfg.D)
    ost = orc.StabilityState(B, L, cfg.D)
    total_stable = 0
    for s in range(T):
        r = _step(orc, D, gst, ost, s, None, torch.from_numpy(ams[s]), torch.from_numpy(mps[s]),
                  torch.from_numpy(ens[s]), kw, f"sweep thresh {thresh}")
        total_stable = int(ost.stable.sum())
    assert 0 < total_stable < B * L


def test_masked_positions_and_padding(orc):
    """recompute only the previous mask's positions (next_pos, -1 padded), as
    a decode loop would"""
    D = need_gpu()
    cfg = dataclasses.replace(W.CONFIGS["gpt2"], K=2, tau=0.9, R=2)
    B, L, T = 4, 300, 12
    kw = dict(K=2, tau=0.9, R=2, alpha=0.7, beta=0.3, lam=0.25, conf_thresh=0.5, V=50257)
    ams, mps, ens = _structured(cfg, B, L, T, seed=11)
    gst = D.StabilityState(B, L, 4)
    ost = orc.StabilityState(B, L, 4)
    pos = None
    for s in range(T):
        if pos is None:
            am, mp, en = ams[s], mps[s], ens[s]
        else:
            p = pos.numpy()
            safe = np.where(p < 0, 0, p)
            am = np.take_along_axis(ams[s], safe, 1)
            mp = np.take_along_axis(mps[s], safe, 1)
            en = np.take_along_axis(ens[s], safe, 1)
        r = _step(orc, D, gst, ost, s, pos, torch.from_numpy(np.ascontiguousarray(am)),
                  torch.from_numpy(np.ascontiguousarray(mp)), torch.from_numpy(np.ascontiguousarray(en)),
                  kw, "masked")
        pos = torch.from_numpy(r["next_pos"].copy())
    assert int(ost.stable.sum()) > 0


def test_large_L_and_radius(orc):
    D = need_gpu()
    B, L, T = 2, 40000, 4
    kw = dict(K=1, tau=0.5, R=700, alpha=0.7, beta=0.3, lam=0.1, conf_thresh=0.75, V=1000)
    rng = np.random.default_rng(3)
    gst = D.StabilityState(B, L, 2)
    ost = orc.StabilityState(B, L, 2)
    for s in range(T):
        am = rng.integers(0, 3, (B, L)).astype(np.int32)
        mp = (rng.uniform(0, 1, (B, L)) ** 0.05).astype(np.float32)
        en = rng.uniform(0, 0.3, (B, L)).astype(np.float32)
        _step(orc, D, gst, ost, s, None, torch.from_numpy(am), torch.from_numpy(mp), torch.from_numpy(en),
              kw, "large L")


def test_per_sequence_device_steps(orc):
    """sequences at different decode steps: the [B] device step numbers are
    read per sequence and advanced by the kernel; each sequence matches the
    oracle run on its own with its own step numbers"""
    D = need_gpu()
    cfg = W.CONFIGS["vocab"]
    B, L, T = 3, 257, 10
    start = np.array([0, 5, 11], dtype=np.int32)
    kw = dict(_kw(cfg), conf_thresh=0.8)
    ams, mps, ens = _structured(cfg, B, L, T, seed=13)
    gst = D.StabilityState(B, L, cfg.D)
    osts = [orc.StabilityState(1, L, cfg.D) for _ in range(B)]
    step_t = torch.from_numpy(start.copy()).cuda()
    say("stability per-sequence steps", start.tolist())
    for s in range(T):
        D.dllm_stability_mask(gst, step_t, None, torch.from_numpy(ams[s]).cuda(), torch.from_numpy(mps[s]).cuda(),
                              torch.from_numpy(ens[s]).cuda(), advance_step=True, **kw)
        torch.cuda.synchronize()
        for b in range(B):
            r = orc.stability_step(osts[b], int(start[b]) + s, None, ams[s][b:b + 1], mps[s][b:b + 1],
                                   ens[s][b:b + 1], **kw)
            assert np.array_equal(gst.mask[b].cpu().numpy(), r["mask"][0]), (b, s)
            assert np.array_equal(gst.next_pos[b].cpu().numpy(), r["next_pos"][0]), (b, s)
            assert int(gst.count[b]) == int(r["count"][0]), (b, s)
            assert np.array_equal(gst.stable[b].cpu().numpy(), osts[b].stable[0]), (b, s)
            assert np.array_equal(gst.ring_step[:, b].cpu().numpy(), osts[b].ring_step[:, 0]), (b, s)
    assert step_t.cpu().tolist() == (start + T).tolist()


def test_threshold_equal_to_confidence(orc):
    """conf_thresh set to one position's float64 confidence exactly: that
    position is not low (strict <), while the threshold one float64 step
    higher makes it low.  With R = 0 and every position stable, the mask is
    the set of low positions, so the GPU's float64 value must equal the
    oracle's bit for bit for the masks to agree."""
    D = need_gpu()
    B, L, V = 1, 96, 126464
    rng = np.random.default_rng(31)
    ent = rng.uniform(0, 3, (B, L)).astype(np.float32)
    t_w = rng.integers(0, 20, (B, L)).astype(np.int32)
    kw = dict(K=3, tau=0.9, R=0, alpha=0.7, beta=0.3, lam=3.0 / 64, V=V)
    none = np.zeros((B, 0), np.int32)

    def fresh_states():
        gst = D.StabilityState(B, L, 3)
        ost = orc.StabilityState(B, L, 3)
        gst.stable.fill_(1)
        gst.entropy_latest.copy_(torch.from_numpy(ent))
        gst.t_write.copy_(torch.from_numpy(t_w))
        ost.stable[:] = 1
        ost.entropy_latest[:] = ent
        ost.t_write[:] = t_w
        return gst, ost

    _, probe = fresh_states()
    c64 = orc.stability_step(probe, 20, none, none, none.astype(np.float32), none.astype(np.float32),
                             conf_thresh=0.0, **kw)["conf"]
    e = torch.zeros((B, 0), device="cuda")
    for p in rng.choice(L, 8, replace=False):
        for th in (float(c64[0, p]), float(np.nextafter(c64[0, p], np.inf))):
            gst, ost = fresh_states()
            say("stability exact threshold position", int(p), repr(th))
            D.dllm_stability_mask(gst, 20, torch.zeros((B, 0), dtype=torch.int32, device="cuda"),
                                  e.int(), e, e, conf_thresh=th, **kw)
            torch.cuda.synchronize()
            r = orc.stability_step(ost, 20, none, none, none.astype(np.float32), none.astype(np.float32),
                                   conf_thresh=th, **kw)
            assert r["mask"][0, p] == (0 if th == c64[0, p] else 1)
            assert np.array_equal(gst.mask.cpu().numpy(), r["mask"]), (int(p), th)
            assert np.array_equal(gst.next_pos.cpu().numpy(), r["next_pos"]), (int(p), th)


def test_gpt2_config_stated_parameters(orc):
    """the GPT-2-shaped workload's stability step at its stated parameters
    (8 x 1024 positions, K = 3, tau = 0.95, R = 2, ring depth 3, no
    confidence gate): four steps over every position fed by the GPU vocab
    stats of that step's 8192 x 50257 logits, then twelve steps of the
    structured history recomputing only the previous mask, as a decode loop
    does.  The stated logits peak at a max-prob near 0.18, so nothing
    settles on them; the structured history settles positions near tau."""
    D = need_gpu()
    cfg = W.CONFIGS["gpt2"]
    B, L = cfg.B, cfg.L
    kw = _kw(cfg)
    assert (kw["K"], kw["tau"], kw["R"], cfg.D, kw["alpha"], kw["beta"], kw["conf_thresh"]) == \
        (3, 0.95, 2, 3, 0.0, 0.0, 0.0)
    gst = D.StabilityState(B, L, cfg.D)
    ost = orc.StabilityState(B, L, cfg.D)
    for s in range(4):
        x = W.logits(cfg, device="cuda", step=s)
        am, mp, en = (t.cpu().view(B, L) for t in D.dllm_vocab_stats(x, V=cfg.V))
        del x
        r = _step(orc, D, gst, ost, s, None, am, mp, en, kw, "gpt2 stated logits")
        assert r["all_stable"].sum() == 0 and r["mask"].all()
    ams, mps, ens = _structured(cfg, B, L, 16, seed=41)
    pos = None
    for s in range(4, 16):
        if pos is None:
            am, mp, en = ams[s], mps[s], ens[s]
        else:
            idx = np.where(pos >= 0, pos, 0)
            am, mp, en = (np.ascontiguousarray(np.take_along_axis(x, idx, 1)) for x in (ams[s], mps[s], ens[s]))
        r = _step(orc, D, gst, ost, s, None if pos is None else torch.from_numpy(pos), torch.from_numpy(am),
                  torch.from_numpy(mp), torch.from_numpy(en), kw, "gpt2 structured")
        pos = np.ascontiguousarray(r["next_pos"][:, :max(1, int(r["count"].max()))])
    n_st = int(ost.stable.sum())
    assert 0 < n_st < B * L
