"""GPU parity of the decode policies against the oracle, bit-exact: the
confidence-ordered eviction (cached flags, mask, next positions, counts,
evicted counts) on seeded confidences with exact ties, signed zeros and
infinities, at small ragged lengths and at the long-context and vocab-sweep
shapes; the ramped window radius and the scheduled full refresh inside the
stability step; and a whole trajectory that chains stability step and
eviction under per-request quotas."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import need_gpu, say

pytestmark = pytest.mark.gpu


def _conf(rng, B, L, kind):
    if kind == "ties":
        vals = np.array([0.1, 0.5, 0.5, 0.9, 0.25, 0.0, -0.0], np.float32)
        return rng.choice(vals, size=(B, L))
    if kind == "wide":
        c = rng.standard_normal((B, L)).astype(np.float32)
        c[rng.random((B, L)) < 0.02] = np.inf
        c[rng.random((B, L)) < 0.02] = -np.inf
        c[rng.random((B, L)) < 0.05] = -0.0
        return c
    # quantised to 1/64: many ties among distinct values, as confidences
    # built from a few entropy levels would have
    return (np.floor(rng.random((B, L)) * 64) / 64).astype(np.float32)


def _evict_case(orc, D, B, L, conf, cached, mask, quota, pos, label):
    say("evict", label, "B", B, "L", L)
    gst = D.StabilityState(B, L, 2)
    gst.conf.copy_(torch.from_numpy(conf))
    gst.cached.copy_(torch.from_numpy(cached))
    gst.mask.copy_(torch.from_numpy(mask))
    ev = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    D.dllm_evict_by_confidence(gst, torch.from_numpy(quota).cuda(),
                               None if pos is None else torch.from_numpy(pos).cuda(), ev)
    torch.cuda.synchronize()
    ost = orc.StabilityState(B, L, 2)
    ost.cached[:] = cached
    m = mask.copy()
    r = orc.evict_by_confidence(ost, conf, quota, pos, m)
    assert np.array_equal(gst.cached.cpu().numpy(), ost.cached), label
    assert np.array_equal(gst.mask.cpu().numpy(), m), label
    assert np.array_equal(gst.count.cpu().numpy(), r["count"]), label
    assert np.array_equal(gst.next_pos.cpu().numpy(), r["next_pos"]), label
    assert np.array_equal(ev.cpu().numpy(), r["evicted"]), label
    return r


@pytest.mark.parametrize("kind", ["ties", "wide", "grid"])
def test_evict_small_ragged(orc, kind):
    D = need_gpu()
    rng = np.random.default_rng({"ties": 11, "wide": 12, "grid": 13}[kind])
    for L in (1, 7, 63, 64, 65, 1000, 1024, 1025, 2048, 2049, 3001):
        B = int(rng.integers(1, 5))
        conf = _conf(rng, B, L, kind)
        cached = (rng.random((B, L)) < 0.6).astype(np.uint8)
        mask = (rng.random((B, L)) < 0.2).astype(np.uint8)
        quota = rng.integers(-1, L + 2, size=B).astype(np.int32)
        quota[0] = min(L, max(0, L // 3))
        n = int(rng.integers(0, L + 1))
        pos = None
        if L % 2:
            pos = np.stack([rng.permutation(L)[:n] for _ in range(B)]).astype(np.int32).reshape(B, n)
            if n:
                pos[:, -1] = -1                               # padding
        _evict_case(orc, D, B, L, conf, cached, mask, quota, pos, f"{kind} L={L}")


def test_evict_degenerate(orc):
    D = need_gpu()
    rng = np.random.default_rng(14)
    B, L = 3, 777
    conf = _conf(rng, B, L, "ties")
    # nothing cached and nothing recomputed: every position goes on the mask
    r = _evict_case(orc, D, B, L, conf, np.zeros((B, L), np.uint8), np.zeros((B, L), np.uint8),
                    np.array([5, 0, -1], np.int32), np.full((B, 4), -1, np.int32), "empty")
    assert list(r["count"]) == [L] * B and not r["evicted"].any()
    # every position cached: quota 0 evicts all, quota L and -1 none
    r = _evict_case(orc, D, B, L, conf, np.ones((B, L), np.uint8), np.zeros((B, L), np.uint8),
                    np.array([0, L, -1], np.int32), None, "full")
    assert list(r["evicted"]) == [L, 0, 0]
    # all confidences equal: the lowest positions stay
    eq = np.full((B, L), 0.5, np.float32)
    _evict_case(orc, D, B, L, eq, np.ones((B, L), np.uint8), np.zeros((B, L), np.uint8),
                np.array([1, 100, 776], np.int32), None, "all equal")


def test_evict_keys_beyond_lds(orc):
    """beyond 32768 positions a sequence's keys are read from memory on each
    selection pass: 2 x 70001 (ragged) with quotas of a third and of all but one"""
    D = need_gpu()
    rng = np.random.default_rng(16)
    B, L = 2, 70001
    conf = _conf(rng, B, L, "grid")
    cached = (rng.random((B, L)) < 0.7).astype(np.uint8)
    mask = (rng.random((B, L)) < 0.1).astype(np.uint8)
    pos = np.stack([rng.permutation(L)[:300] for _ in range(B)]).astype(np.int32)
    quota = np.array([L // 3, int(cached[1].sum()) + 290], np.int32)
    r = _evict_case(orc, D, B, L, conf, cached, mask, quota, pos, "beyond lds")
    assert r["evicted"][0] > 0


@pytest.mark.parametrize("shape", ["longctx", "vocab"])
def test_evict_full_size(orc, shape):
    """the long-context shape (4 x 32768) with a cache of 8192 positions per
    sequence -- the sink + rolling budget of that workload -- and the vocab
    sweep's 64 x 512 under quotas shared out of half the positions"""
    D = need_gpu()
    cfg = W.CONFIGS[shape]
    B, L = cfg.B, cfg.L
    rng = np.random.default_rng(15)
    conf = _conf(rng, B, L, "grid")
    cached = (rng.random((B, L)) < 0.5).astype(np.uint8)
    mask = (rng.random((B, L)) < 0.05).astype(np.uint8)
    if shape == "longctx":
        quota = np.full(B, cfg.sinks + cfg.rolling, np.int32)
        pos = np.full((B, 4 * cfg.b), -1, np.int32)
        for b in range(B):
            pos[b, :cfg.b] = np.arange(L - cfg.b, L)           # the block at the end
    else:
        lens = rng.integers(L // 2, L + 1, size=B)
        quota = orc.cache_quotas(lens, B * L // 2)
        pos = None
    r = _evict_case(orc, D, B, L, conf, cached, mask, quota, pos, f"full {shape}")
    assert r["evicted"].sum() > 0


def _stab_kw(cfg):
    return dict(K=cfg.K, tau=cfg.tau, R=cfg.R, alpha=cfg.alpha, beta=cfg.beta, lam=cfg.lam,
                conf_thresh=cfg.conf_thresh, V=max(cfg.V, 2))


def _history(B, L, T, seed):
    rng = np.random.default_rng(seed)
    settle = rng.integers(0, T, (B, L))
    tok = rng.integers(0, 50, (B, L))
    out = []
    for s in range(T):
        settled = s >= settle
        am = np.where(settled, tok, rng.integers(0, 50, (B, L))).astype(np.int32)
        mp = np.where(settled, rng.uniform(0.85, 1.0, (B, L)), rng.uniform(0.0, 0.9, (B, L))).astype(np.float32)
        # a few entropy levels, so that equal confidences occur
        en = np.where(settled, rng.integers(0, 4, (B, L)) * 0.125, rng.integers(8, 80, (B, L)) * 0.125)
        out.append((am, mp, en.astype(np.float32)))
    return out


def _compare_step(gst, ost, r, label):
    for name in ("stable", "t_write", "ring_argmax", "ring_step"):
        assert np.array_equal(getattr(gst, name).cpu().numpy(), getattr(ost, name)), (label, name)
    assert np.array_equal(gst.mask.cpu().numpy(), r["mask"]), label
    assert np.array_equal(gst.next_pos.cpu().numpy(), r["next_pos"]), label
    assert np.array_equal(gst.count.cpu().numpy(), r["count"]), label
    assert np.array_equal(gst.all_stable.cpu().numpy(), r["all_stable"]), label


def test_dynamic_radius_and_refresh(orc):
    """the vocab sweep's shape over 24 steps with the radius ramped from 0 to
    6 and a full refresh at the pages' interval; each step recomputes the
    previous step's mask"""
    D = need_gpu()
    cfg = W.CONFIGS["vocab"]
    B, L, T = cfg.B, cfg.L, 24
    kw = dict(_stab_kw(cfg), R=6, R_early=0, T_steps=T, refresh_every=orc.refresh_interval(T))
    assert D.dllm_refresh_interval(T) == kw["refresh_every"] == 3
    gst, ost = D.StabilityState(B, L, cfg.D), orc.StabilityState(B, L, cfg.D)
    pos = None
    n_refresh = 0
    for s, (am, mp, en) in enumerate(_history(B, L, T, seed=21)):
        say("policies radius/refresh step", s)
        if pos is None:
            a, m, e = am, mp, en
        else:
            idx = np.where(pos >= 0, pos, 0)
            a, m, e = (np.take_along_axis(x, idx, axis=1) for x in (am, mp, en))
        D.dllm_stability_mask(gst, s, None if pos is None else torch.from_numpy(pos).cuda(),
                              torch.from_numpy(a).cuda(), torch.from_numpy(m).cuda(),
                              torch.from_numpy(e).cuda(), **kw)
        torch.cuda.synchronize()
        r = orc.stability_step(ost, s, pos, a, m, e, **kw)
        _compare_step(gst, ost, r, ("radius/refresh", s))
        if orc.is_refresh_step(kw["refresh_every"], s):
            assert r["mask"].all()
            n_refresh += 1
        nxt = r["next_pos"]
        pos = np.ascontiguousarray(nxt[:, :max(1, int(r["count"].max()))])
    assert n_refresh == 7


@pytest.mark.parametrize("gate", ["pages", "entropy only"])
def test_trajectory_with_quotas(orc, gate):
    """stability step, then eviction under per-request quotas, over 20 steps
    of the vocab sweep's shape, with the pages' confidence (alpha 0.7, beta
    0.3, lambda 3/T, threshold 0.8) and with the entropy term alone (alpha 1,
    beta 0).  Both sides compute the same float64 confidence and round it
    once, so they rank and evict on bit-identical float32 values."""
    D = need_gpu()
    cfg = W.CONFIGS["vocab"]
    B, L, T = cfg.B, cfg.L, 20
    if gate == "pages":
        kw = _stab_kw(cfg)
        assert (kw["alpha"], kw["beta"], kw["lam"], kw["conf_thresh"]) == (0.7, 0.3, 3.0 / 64, 0.8)
    else:
        kw = dict(_stab_kw(cfg), alpha=1.0, beta=0.0, lam=0.0, conf_thresh=0.0)
    lens = np.full(B, L)
    quota = orc.cache_quotas(lens, B * L * 3 // 5, min_frac=0.2)
    assert np.array_equal(D.dllm_cache_quotas(lens, B * L * 3 // 5, 0.2), quota)
    q_dev = torch.from_numpy(quota).cuda()
    gst, ost = D.StabilityState(B, L, cfg.D), orc.StabilityState(B, L, cfg.D)
    ev = torch.zeros(B, dtype=torch.int32, device="cuda")
    pos = None
    for s, (am, mp, en) in enumerate(_history(B, L, T, seed=22)):
        say("policies trajectory step", s)
        if pos is None:
            a, m, e = am, mp, en
        else:
            idx = np.where(pos >= 0, pos, 0)
            a, m, e = (np.take_along_axis(x, idx, axis=1) for x in (am, mp, en))
        pd = None if pos is None else torch.from_numpy(pos).cuda()
        D.dllm_stability_mask(gst, s, pd, torch.from_numpy(a).cuda(), torch.from_numpy(m).cuda(),
                              torch.from_numpy(e).cuda(), **kw)
        D.dllm_evict_by_confidence(gst, q_dev, pd, ev)
        torch.cuda.synchronize()
        r = orc.stability_step(ost, s, pos, a, m, e, **kw)
        conf32 = r["conf"].astype(np.float32)
        assert np.array_equal(gst.conf.cpu().numpy().view(np.uint32), conf32.view(np.uint32)), ("conf", s)
        mask = r["mask"].copy()
        re = orc.evict_by_confidence(ost, conf32, quota, pos, mask)
        assert np.array_equal(gst.cached.cpu().numpy(), ost.cached), ("cached", s)
        assert np.array_equal(gst.mask.cpu().numpy(), mask), ("mask", s)
        assert np.array_equal(gst.next_pos.cpu().numpy(), re["next_pos"]), ("next_pos", s)
        assert np.array_equal(gst.count.cpu().numpy(), re["count"]), ("count", s)
        assert np.array_equal(ev.cpu().numpy(), re["evicted"]), ("evicted", s)
        assert (ost.cached.sum(axis=1) <= quota).all()
        pos = np.ascontiguousarray(re["next_pos"][:, :max(1, int(re["count"].max()))])
