"""Pins of the oracle's decode policies (N3): the dynamic radius against its
closed form and applied as the window radius, the refresh schedule against
the page's ranges, the per-request quotas against the page's guarantee and
arrival order, and confidence-ordered eviction against an independent
numpy lexsort on random cases with ties."""
import numpy as np
import pytest


def _state(orc, B, L, D=4):
    return orc.StabilityState(B, L, D)


def test_dynamic_radius_closed_form(orc):
    for R_early, R, T in [(0, 4, 16), (1, 7, 64), (2, 2, 10), (0, 3, 2)]:
        rs = [orc.dynamic_radius(R_early, R, T, s) for s in range(T + 5)]
        assert rs[0] == R_early and rs[T - 1] == R and all(r == R for r in rs[T - 1:])
        assert all(a <= b for a, b in zip(rs, rs[1:]))                   # never narrows
        assert all(r == R_early + (R - R_early) * min(s, T - 1) // (T - 1) for s, r in enumerate(rs))
    assert all(orc.dynamic_radius(0, 5, 1, s) == 5 for s in range(4))       # T <= 1: fixed R
    assert all(orc.dynamic_radius(3, 5, 0, s) == 5 for s in range(4))


def test_dynamic_radius_is_the_window(orc):
    """a step with the ramp gives the mask of a fixed-R step at R_eff"""
    B, L, T = 1, 40, 8
    rng = np.random.default_rng(1)
    for step in (0, 3, 7, 9):
        st1, st2 = _state(orc, B, L), _state(orc, B, L)
        st1.stable[0] = (rng.random(L) < 0.8).astype(np.uint8)
        st2.stable[:] = st1.stable
        am = np.zeros((B, L), np.int32)
        mp = np.full((B, L), 0.5, np.float32)
        en = np.zeros((B, L), np.float32)
        kw = dict(K=3, tau=0.9, alpha=0.0, beta=0.0, lam=0.0, conf_thresh=0.0, V=10)
        pos = np.array([[5]], np.int32)
        a = orc.stability_step(st1, step, pos, am[:, :1], mp[:, :1], en[:, :1], R=6, R_early=1,
                               T_steps=T, **kw)
        r_eff = orc.dynamic_radius(1, 6, T, step)
        b = orc.stability_step(st2, step, pos, am[:, :1], mp[:, :1], en[:, :1], R=r_eff, **kw)
        assert np.array_equal(a["mask"], b["mask"]) and np.array_equal(a["next_pos"], b["next_pos"])


def test_refresh_schedule(orc):
    # the page's ranges: T in 50..100 -> every 5..10 steps, T < 50 -> every 3..5
    for T in range(50, 101):
        assert 5 <= orc.refresh_interval(T) <= 10
    for T in range(1, 50):
        assert 3 <= orc.refresh_interval(T) <= 5
    assert [orc.refresh_interval(T) for T in (16, 30, 50, 64, 100, 400)] == [3, 3, 5, 6, 10, 10]
    assert [s for s in range(13) if orc.is_refresh_step(4, s)] == [4, 8, 12]
    assert not any(orc.is_refresh_step(0, s) for s in range(20))
    # a refresh step computes every position even when only one is unstable
    B, L = 1, 30
    st = _state(orc, B, L)
    st.stable[0] = 1
    st.stable[0, 10] = 0
    kw = dict(K=3, tau=0.9, R=1, V=10)
    one = np.zeros((B, 1), np.int32), np.full((B, 1), 0.5, np.float32), np.zeros((B, 1), np.float32)
    r = orc.stability_step(st.copy(), 8, np.array([[10]], np.int32), *one, refresh_every=4, **kw)
    assert r["mask"].all() and r["count"][0] == L and not r["all_stable"][0]
    r = orc.stability_step(st.copy(), 9, np.array([[10]], np.int32), *one, refresh_every=4, **kw)
    assert list(np.nonzero(r["mask"][0])[0]) == [9, 10, 11]


def test_cache_quotas(orc):
    lens = np.array([100, 7, 40, 55])
    for budget in (41, 60, 120, 202, 1000):
        q = orc.cache_quotas(lens, budget)
        mins = np.ceil(0.2 * lens).astype(int)
        assert np.all(q >= mins) and np.all(q <= lens)
        assert q.sum() == min(budget, lens.sum())
        # arrival order: a later request gets more than its guarantee only
        # when every earlier one is full
        extra = q - mins
        for b in range(len(lens)):
            if extra[b] > 0:
                assert np.all(q[:b] == lens[:b])
    with pytest.raises(ValueError):
        orc.cache_quotas(lens, 40)                       # below the guarantees (20 + 2 + 8 + 11 = 41)
    assert list(orc.cache_quotas([10, 10], 5, min_frac=0.0)) == [5, 0]


def _evict_ref(conf, cached, quota, pos, mask):
    """independent: numpy lexsort by (-conf, position)"""
    B, L = conf.shape
    cached, mask = cached.copy(), mask.copy()
    ev = np.zeros(B, np.int32)
    for b in range(B):
        p = np.arange(L) if pos is None else pos[b]
        p = p[(p >= 0) & (p < L)]
        cached[b, p] = 1
        cand = np.nonzero(cached[b])[0]
        if quota[b] >= 0 and len(cand) > quota[b]:
            order = cand[np.lexsort((cand, -conf[b, cand].astype(np.float64)))]
            drop = order[quota[b]:]
            cached[b, drop] = 0
            ev[b] = len(drop)
        mask[b] |= (cached[b] == 0).astype(np.uint8)
    nxt = np.full((B, L), -1, np.int32)
    cnt = mask.sum(axis=1).astype(np.int32)
    for b in range(B):
        on = np.nonzero(mask[b])[0]
        nxt[b, :len(on)] = on
    return cached, mask, nxt, cnt, ev


def test_evict_matches_lexsort(orc):
    rng = np.random.default_rng(7)
    for trial in range(300):
        B, L = int(rng.integers(1, 4)), int(rng.integers(1, 12))
        conf = rng.choice(np.array([0.1, 0.5, 0.5, 0.9, 0.25], np.float32), size=(B, L))   # ties
        st = _state(orc, B, L)
        st.cached[:] = (rng.random((B, L)) < 0.6).astype(np.uint8)
        mask = (rng.random((B, L)) < 0.3).astype(np.uint8)
        quota = rng.integers(-1, L + 2, size=B).astype(np.int32)
        n = int(rng.integers(0, L + 1))
        pos = None if trial % 5 == 0 else np.stack([rng.permutation(L)[:n] for _ in range(B)]).astype(np.int32)
        if pos is not None and n > 0:
            pos[:, 0] = -1                                # padding
        ref = _evict_ref(conf, st.cached, quota, pos, mask)
        r = orc.evict_by_confidence(st, conf, quota, pos, mask)
        assert np.array_equal(st.cached, ref[0]) and np.array_equal(mask, ref[1]), trial
        assert np.array_equal(r["next_pos"], ref[2]) and np.array_equal(r["count"], ref[3])
        assert np.array_equal(r["evicted"], ref[4])


def test_evict_invariants(orc):
    rng = np.random.default_rng(8)
    B, L = 3, 200
    conf = rng.random((B, L)).astype(np.float32)
    st = _state(orc, B, L)
    quota = np.array([50, 0, -1], np.int32)
    mask = np.zeros((B, L), np.uint8)
    r = orc.evict_by_confidence(st, conf, quota, None, mask)        # every position recomputed
    kept = st.cached.astype(bool)
    assert kept[0].sum() == 50 and kept[1].sum() == 0 and kept[2].all()
    assert conf[0, kept[0]].min() >= conf[0, ~kept[0]].max()          # the most confident stay
    assert list(r["evicted"]) == [150, 200, 0]
    assert np.array_equal(mask.astype(bool), ~kept)                    # the rest is recomputed next step
