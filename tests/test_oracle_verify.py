"""Pins of the oracle's self-verification (N4): the parallel-width ramp
against the page's ranges, the conflict test against closed forms (pairs
of independent tokens, a score exactly at the threshold, the window bound,
zero marginals), the withdrawn span (decoded positions between the pair,
undecoded ones untouched), the state updates, and random cases against an
independent numpy formulation."""
import numpy as np
import pytest


def test_parallel_width_ramp(orc):
    for w0, w1, T in [(16, 2, 64), (8, 4, 10), (12, 3, 2), (16, 2, 100)]:
        ws = [orc.parallel_width(w0, w1, T, s) for s in range(T + 4)]
        assert ws[0] == w0 and ws[T - 1] == w1 and all(w == w1 for w in ws[T - 1:])
        assert all(a >= b for a, b in zip(ws, ws[1:]))                   # never widens
        assert all(w == w0 - (w0 - w1) * min(s, T - 1) // (T - 1) for s, w in enumerate(ws))
    # the page's ranges: 8-16 positions early, 2-4 late
    assert 8 <= orc.parallel_width(16, 2, 64, 0) <= 16 and 2 <= orc.parallel_width(16, 2, 64, 63) <= 4
    assert orc.parallel_width(16, 2, 1, 0) == 2


def _run(orc, L, dec, pm, pj, W, tau=0.5, mask=None, stable=None, cached=None):
    dec = np.asarray(dec, np.int32).reshape(1, -1)
    n = dec.shape[1]
    mask = np.zeros((1, L), np.uint8) if mask is None else mask
    r = orc.self_verify(L, dec, np.asarray(pm, np.float32).reshape(1, n),
                        np.asarray(pj, np.float32).reshape(1, n, W - 1), W, tau, mask, stable, cached)
    return r, mask


def test_independent_pairs_never_conflict(orc):
    L, W = 40, 4
    dec = [3, 4, 5, 7, 8]
    pm = [0.9, 0.5, 0.25, 0.75, 0.6]
    pj = np.zeros((5, W - 1), np.float32)
    pos = {p: i for i, p in enumerate(dec)}
    for j, p in enumerate(dec):
        for d in range(1, W):
            if p + d in pos:
                pj[j, d - 1] = np.float32(pm[j]) * np.float32(pm[pos[p + d]])   # exact here
    r, mask = _run(orc, L, dec, pm, pj, W)
    assert not r["rollback"].any() and not mask.any() and r["count"][0] == 0


def test_threshold_is_strict(orc):
    L, W = 16, 2
    # marginals 0.5 and 0.25: product 0.125, a score of exactly 0.5 at joint 0.0625
    r, _ = _run(orc, L, [6, 7], [0.5, 0.25], [[0.0625], [0.0]], W)
    assert not r["rollback"].any()
    below = np.nextafter(np.float32(0.0625), np.float32(0))
    r, _ = _run(orc, L, [6, 7], [0.5, 0.25], [[below], [0.0]], W)
    assert list(np.nonzero(r["rollback"][0])[0]) == [6, 7]
    # the joint of the pair is read from the earlier position's row only
    r, _ = _run(orc, L, [6, 7], [0.5, 0.25], [[0.0625], [0.0]], W, tau=0.51)
    assert list(np.nonzero(r["rollback"][0])[0]) == [6, 7]


def test_span_window_and_zero_marginal(orc):
    L, W = 32, 4
    dec = [10, 11, 13, 14, 20]
    pm = [0.8] * 5
    ok = 0.64
    pj = np.full((5, W - 1), ok, np.float32)
    pj[0, 2] = 0.1            # (10, 13): distance 3 < W, a conflict
    r, mask = _run(orc, L, dec, pm, pj, W)
    # the decoded positions between the pair go too; 12 was not decoded
    assert list(np.nonzero(r["rollback"][0])[0]) == [10, 11, 13]
    assert list(r["rb_pos"][0][:3]) == [10, 11, 13] and (r["rb_pos"][0][3:] == -1).all()
    assert r["n_rollback"][0] == 3 and list(np.nonzero(mask[0])[0]) == [10, 11, 13]
    # a pair W apart is outside the window: (10, 14) with joint 0 is not checked
    pj = np.full((5, W - 1), ok, np.float32)
    r, _ = _run(orc, L, [10, 14, -1, -1, -1], [0.8, 0.8, 0, 0, 0], np.zeros((5, W - 1)), W)
    assert not r["rollback"].any()
    # a zero marginal makes no conflict, whatever the joint
    r, _ = _run(orc, L, [10, 11], [0.0, 0.9], [[0.0, 0.0, 0.0], [0.0, 0.0, 0.0]], W)
    assert not r["rollback"].any()


def test_state_updates(orc):
    L, W = 24, 3
    rng = np.random.default_rng(3)
    mask = (rng.random((1, L)) < 0.3).astype(np.uint8)
    stable = np.ones((1, L), np.uint8)
    cached = np.ones((1, L), np.uint8)
    m0 = mask.copy()
    dec = [2, 3, 4, 9, 10]
    pj = np.full((5, W - 1), 0.5, np.float32)
    pj[3, 0] = 0.01                                   # (9, 10)
    r, mask = _run(orc, L, dec, [0.7] * 5, pj, W, mask=mask, stable=stable, cached=cached)
    rb = r["rollback"][0].astype(bool)
    assert list(np.nonzero(rb)[0]) == [9, 10]
    assert np.array_equal(mask[0].astype(bool), m0[0].astype(bool) | rb)
    assert np.array_equal(stable[0].astype(bool), ~rb) and np.array_equal(cached[0].astype(bool), ~rb)
    on = np.nonzero(mask[0])[0]
    assert r["count"][0] == len(on) and list(r["next_pos"][0][:len(on)]) == list(on)
    assert (r["next_pos"][0][len(on):] == -1).all()


def _verify_ref(L, dec, pm, pj, W, tau):
    """independent: all (i, j) pairs of decoded positions as a matrix, then
    each decoded position against the union of the conflicting spans"""
    B, n = dec.shape
    rb = np.zeros((B, L), np.uint8)
    for b in range(B):
        v = dec[b] >= 0
        p = dec[b][v].astype(np.int64)
        m = pm[b][v].astype(np.float64)
        jt = pj[b][v].astype(np.float64)
        dist = p[None, :] - p[:, None]                      # [i, j] = p_j - p_i
        inwin = (dist >= 1) & (dist < W)
        prod = m[:, None] * m[None, :]
        joint = np.take_along_axis(jt, np.clip(dist - 1, 0, W - 2), axis=1)
        with np.errstate(divide="ignore", invalid="ignore"):
            conflict = inwin & (prod > 0) & (joint / np.where(prod > 0, prod, 1.0) < tau)
        ii, jj = np.nonzero(conflict)
        for a, c in zip(p[ii], p[jj]):
            rb[b, p[(p >= a) & (p <= c)]] = 1
    return rb


def test_random_against_numpy(orc):
    rng = np.random.default_rng(4)
    for trial in range(200):
        B, L, W = int(rng.integers(1, 4)), int(rng.integers(4, 80)), int(rng.integers(2, 7))
        n = int(rng.integers(0, min(L, 24) + 1))
        dec = np.full((B, n), -1, np.int32)
        for b in range(B):
            k = int(rng.integers(0, n + 1))
            dec[b, :k] = np.sort(rng.choice(L, size=k, replace=False))
        pm = rng.choice(np.array([0.0, 0.3, 0.5, 0.9, 1.0], np.float32), size=(B, n))
        pj = (rng.random((B, n, W - 1)) * 0.9).astype(np.float32)
        tau = float(rng.choice([0.25, 0.5, 0.8]))
        mask = np.zeros((B, L), np.uint8)
        r = orc.self_verify(L, dec, pm, pj, W, tau, mask)
        ref = _verify_ref(L, dec, pm, pj, W, tau)
        assert np.array_equal(r["rollback"], ref), trial
        assert np.array_equal(mask, ref), trial
        assert np.array_equal(r["n_rollback"], ref.sum(axis=1)), trial


def test_bad_arguments(orc):
    with pytest.raises(ValueError):
        orc.self_verify(8, np.array([[9]], np.int32), [[0.5]], np.zeros((1, 1, 2)), 3, 0.5,
                        np.zeros((1, 8), np.uint8))
    with pytest.raises(ValueError):
        orc.self_verify(8, np.array([[1]], np.int32), [[0.5]], np.zeros((1, 1, 0)), 1, 0.5,
                        np.zeros((1, 8), np.uint8))
    # the positions come ascending, padding only after them
    for bad in ([3, 2], [2, 2], [-1, 4], [1, -2]):
        with pytest.raises(ValueError):
            orc.self_verify(8, np.array([bad], np.int32), [[0.5, 0.5]], np.zeros((1, 2, 2)), 3, 0.5,
                            np.zeros((1, 8), np.uint8))
