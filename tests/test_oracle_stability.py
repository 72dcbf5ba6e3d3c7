"""Pins of the oracle's history ring, stability test, confidence score and
window mask (A5-A7): the SWD page's length-20 example, brute force over all
stable patterns against an interval-union formulation, brute force over all
short histories against the page's list-based scheduler formulation, and
closed forms of the confidence score."""
import itertools
import json
import math
import os

import numpy as np
import pytest

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _state(orc, B, L, D):
    return orc.StabilityState(B, L, D)


def _no_update(B):
    return (np.zeros((B, 0), np.int32), np.zeros((B, 0), np.int32), np.zeros((B, 0), np.float32),
            np.zeros((B, 0), np.float32))


def test_swd_page_example(orc):
    g = json.load(open(os.path.join(GOLD, "swd_window_example.json")))
    L, R = g["L"], g["R"]
    st = _state(orc, 1, L, 3)
    st.stable[0, np.array(g["stable_1based"]) - 1] = 1
    pos, am, mp, en = _no_update(1)
    r = orc.stability_step(st, 5, pos, am, mp, en, K=3, tau=0.95, R=R, V=100)
    got = (np.flatnonzero(r["mask"][0]) + 1).tolist()
    assert got == g["mask_1based"]
    assert r["count"][0] == len(got) and r["all_stable"][0] == 0
    assert (r["next_pos"][0, :len(got)] + 1).tolist() == got
    assert np.all(r["next_pos"][0, len(got):] == -1)


def _interval_union(stable, R):
    """the page's get_computation_mask: mark [max(0,u-R), min(L-1,u+R)] for
    every unstable u; all stable -> all ones"""
    L = len(stable)
    if all(stable):
        return [1] * L
    m = [0] * L
    for u in range(L):
        if not stable[u]:
            for j in range(max(0, u - R), min(L - 1, u + R) + 1):
                m[j] = 1
    return m


@pytest.mark.parametrize("L", [1, 2, 5, 11])
def test_window_brute_force(orc, L):
    pats = np.array(list(itertools.product([0, 1], repeat=L)), dtype=np.uint8)
    B = pats.shape[0]
    for R in (0, 1, 2, 3):
        st = _state(orc, B, L, 3)
        st.stable[:] = pats
        pos, am, mp, en = _no_update(B)
        r = orc.stability_step(st, 7, pos, am, mp, en, K=3, tau=0.95, R=R, V=50)
        for i in range(B):
            ref = _interval_union(list(pats[i]), R)
            assert r["mask"][i].tolist() == ref
            assert r["all_stable"][i] == int(all(pats[i]))
            assert r["count"][i] == sum(ref)
            assert r["next_pos"][i, :sum(ref)].tolist() == [j for j in range(L) if ref[j]]
        if R == 0:
            partial = pats.min(1) == 0
            assert np.array_equal(r["mask"][partial], 1 - pats[partial])      # mask = seed


class PageScheduler:
    """the SWD page's scheduler, with its lost operators read as == and >:
    per-position list history trimmed to the last K, stable positions skipped"""

    def __init__(self, L, tau, K):
        self.tau, self.K = tau, K
        self.stable = [False] * L
        self.hist = [([], []) for _ in range(L)]

    def update(self, toks, probs):
        new = list(self.stable)
        for i in range(len(toks)):
            if self.stable[i]:
                continue
            t, p = self.hist[i]
            t.append(int(toks[i]))
            p.append(float(probs[i]))
            if len(t) > self.K:
                del t[:-self.K]
                del p[:-self.K]
            if len(t) == self.K and len(set(t)) == 1 and sum(p) / self.K > self.tau:
                new[i] = True
        self.stable = new


@pytest.mark.parametrize("K", [1, 2, 3])
def test_stability_brute_force_histories(orc, K):
    tau, delta = 0.75, 0.125                     # exactly representable grid
    probs = [tau - delta, tau, tau + delta, 1.0]
    T = 4
    choices = list(itertools.product([0, 1], probs))          # 8 per step
    hists = list(itertools.product(range(8), repeat=T))        # 4096 histories
    L = len(hists)
    tok = np.array([[choices[c][0] for c in h] for h in hists], dtype=np.int32)   # [L, T]
    pr = np.array([[choices[c][1] for c in h] for h in hists], dtype=np.float32)
    st = _state(orc, 1, L, max(K, 3))
    page = PageScheduler(L, tau, K)
    for s in range(T):
        r = orc.stability_step(st, s, None, tok[:, s][None], pr[:, s][None],
                               np.zeros((1, L), np.float32), K=K, tau=tau, R=1, V=10)
        page.update(tok[:, s], pr[:, s])
        assert st.stable[0].tolist() == [int(x) for x in page.stable], s
    # mean exactly tau is not stable: e.g. K identical records at tau
    idx = hists.index(tuple([choices.index((0, tau))] * T))
    assert st.stable[0, idx] == 0
    if K == 1:   # K = 1: stable iff some step's prob exceeded tau
        assert np.array_equal(st.stable[0], (pr > tau).any(1).astype(np.uint8))


def test_missed_step_breaks_run(orc):
    L, K = 4, 3
    st = _state(orc, 1, L, 8)
    ones = np.ones((1, 1), np.float32)
    for s in range(7):
        if s == 2:
            pos = np.array([[1]], np.int32)      # position 0 not recomputed at step 2
        else:
            pos = np.array([[0]], np.int32)
        am = np.array([[5]], np.int32)
        orc.stability_step(st, s, pos, am, ones, ones * 0, K=K, tau=0.5, R=0, V=10)
        expect = 1 if s >= 5 else 0              # needs steps s, s-1, s-2 all present
        assert st.stable[0, 0] == expect, s


def test_confidence_closed_forms(orc):
    g = json.load(open(os.path.join(GOLD, "confidence_constants.json")))
    alpha, beta = g["alpha"], g["beta"]
    T = 16
    lam = g["lambda_times_T"] / T
    V = 512
    L = 6
    st = _state(orc, 1, L, 16)
    st.stable[:] = 1
    hmax = math.log(V)
    st.entropy_latest[0] = np.array([0.0, hmax, 0.0, hmax, 0.0, 0.0], np.float32)
    st.t_write[0] = np.array([10, 10, 0, 0, 9, 8], np.int32)
    pos, am, mp, en = _no_update(1)
    r = orc.stability_step(st, 10, pos, am, mp, en, K=3, tau=0.9, R=0, alpha=alpha, beta=beta,
                           lam=lam, conf_thresh=0.0, V=V)
    c = r["conf"][0]
    assert c[0] == alpha + beta == 1.0                  # certain and fresh
    assert abs(c[1] - beta) <= 1e-7                     # float32 ln V entropy: uniform, fresh
    # uniform and 10 steps old: only the decay term is left, e^-1.875 = 0.1534
    assert abs(c[3] - beta * 0.15335496684492847) <= 1e-7
    assert c[0] > c[4] > c[5] > c[2] > alpha            # decays with age, floor alpha at H = 0
    assert r["all_stable"][0] == 1 and r["mask"][0].tolist() == [1] * L


def test_confidence_age_clamp(orc):
    """the age s - t_write is clamped to [0, n_decay - 1]: a position 10 steps
    old with a 3-entry table scores as one 2 steps old with a table long
    enough, and a table longer than every age changes nothing"""
    V, L = 512, 3
    pos, am, mp, en = _no_update(1)

    def conf(step, t_write, n_decay):
        st = _state(orc, 1, L, 4)
        st.stable[:] = 1
        st.entropy_latest[0] = np.array([0.0, 1.5, 4.0], np.float32)
        st.t_write[0] = t_write
        return orc.stability_step(st, step, pos, am, mp, en, K=3, tau=0.9, R=0, alpha=0.7, beta=0.3,
                                  lam=0.25, conf_thresh=0.0, V=V, n_decay=n_decay)["conf"][0]
    assert np.array_equal(conf(10, 0, 3), conf(2, 0, 4096))
    assert np.array_equal(conf(10, 0, 11), conf(10, 0, 4096))
    assert not np.array_equal(conf(10, 0, 10), conf(10, 0, 4096))
    assert np.array_equal(conf(3, 7, 4096), conf(7, 7, 4096))     # negative age reads age 0
    # H = 0 at age 0 is alpha + beta exactly; the entropy term falls with H
    c = conf(5, 5, 1)
    assert c[0] == 0.7 + 0.3 and c[0] > c[1] > c[2]


def test_confidence_gate_refresh_timing(orc):
    """a certain (H = 0) stable position falls below 0.8 once
    0.7 + 0.3 exp(-3 dt / T) < 0.8, i.e. dt > T ln 3 / 3 (= 5.86 at T = 16)"""
    T, L = 16, 9
    st = _state(orc, 1, L, 16)
    st.stable[:] = 1
    pos, am, mp, en = _no_update(1)
    first_low = None
    for s in range(1, 12):
        r = orc.stability_step(st, s, pos, am, mp, en, K=3, tau=0.9, R=1, alpha=0.7, beta=0.3,
                               lam=3.0 / T, conf_thresh=0.8, V=512)
        if r["all_stable"][0] == 0 and first_low is None:
            first_low = s
            assert r["mask"][0].tolist() == [1] * L      # every position aged together
    assert first_low == math.floor(T * math.log(3) / 3) + 1 == 6


def test_low_confidence_seeds_window(orc):
    L = 12
    st = _state(orc, 1, L, 4)
    st.stable[:] = 1
    st.t_write[0] = 20
    st.t_write[0, 7] = 0                                # one old cache entry
    pos, am, mp, en = _no_update(1)
    r = orc.stability_step(st, 20, pos, am, mp, en, K=3, tau=0.9, R=2, alpha=0.7, beta=0.3,
                           lam=0.2, conf_thresh=0.8, V=512)
    assert np.flatnonzero(r["mask"][0]).tolist() == [5, 6, 7, 8, 9]
    assert r["all_stable"][0] == 0
    assert st.stable[0].tolist() == [1] * L            # low confidence does not unstick


def test_ring_depth_does_not_matter(orc):
    rng = np.random.default_rng(21)
    B, L, T, K = 2, 30, 12, 3
    tok = rng.integers(0, 2, (T, B, L)).astype(np.int32)
    pr = rng.choice(np.array([0.6, 0.8, 0.95, 1.0], np.float32), (T, B, L))
    ent = rng.uniform(0, 3, (T, B, L)).astype(np.float32)
    outs = []
    for D in (K, 5, 16):
        st = _state(orc, B, L, D)
        seq = []
        for s in range(T):
            r = orc.stability_step(st, s, None, tok[s], pr[s], ent[s], K=K, tau=0.85, R=1,
                                   alpha=0.7, beta=0.3, lam=0.25, conf_thresh=0.5, V=64)
            seq.append((st.stable.copy(), r["mask"].copy(), r["conf"].copy()))
        outs.append(seq)
    for seq in outs[1:]:
        for (a, m, c), (a0, m0, c0) in zip(seq, outs[0]):
            assert np.array_equal(a, a0) and np.array_equal(m, m0) and np.array_equal(c, c0)


def test_checkpoint_resume(orc):
    rng = np.random.default_rng(22)
    B, L, T, D = 2, 40, 10, 6
    tok = rng.integers(0, 3, (T, B, L)).astype(np.int32)
    pr = rng.choice(np.array([0.7, 0.9, 0.99], np.float32), (T, B, L))
    ent = rng.uniform(0, 2, (T, B, L)).astype(np.float32)
    kw = dict(K=2, tau=0.8, R=2, alpha=0.7, beta=0.3, lam=0.3, conf_thresh=0.6, V=128)
    st = _state(orc, B, L, D)
    full = [orc.stability_step(st, s, None, tok[s], pr[s], ent[s], **kw)["mask"] for s in range(T)]
    st2 = _state(orc, B, L, D)
    for s in range(4):
        orc.stability_step(st2, s, None, tok[s], pr[s], ent[s], **kw)
    saved = st2.copy()
    rest = [orc.stability_step(saved, s, None, tok[s], pr[s], ent[s], **kw)["mask"] for s in range(4, T)]
    for a, b in zip(full[4:], rest):
        assert np.array_equal(a, b)


def test_padding_positions_skipped(orc):
    B, L = 1, 6
    st = _state(orc, B, L, 3)
    pos = np.array([[2, -1, 4]], np.int32)
    am = np.array([[7, 9, 7]], np.int32)
    mp = np.ones((1, 3), np.float32)
    for s in range(3):
        orc.stability_step(st, s, pos, am, mp, mp * 0, K=3, tau=0.5, R=0, V=10)
    assert st.stable[0].tolist() == [0, 0, 1, 0, 1, 0]
    assert st.ring_step[:, 0, 1].tolist() == [-1, -1, -1]
