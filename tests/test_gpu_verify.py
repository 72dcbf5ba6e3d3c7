"""GPU parity of the self-verification (N4) against the oracle, bit-exact:
withdrawal flags, mask, stable and cached flags, next positions, counts and
the withdrawn list, on seeded decodes with conflicting pairs planted at
every distance of the window; lists longer than one 1024-entry chunk (the
halo of earlier entries); the vocab-sweep and long-context shapes; empty
and all-padding lists; and the documented rejection of a list that is not
ascending."""
import numpy as np
import pytest
import torch

import workloads as W_
from gpu_util import need_gpu, say

pytestmark = pytest.mark.gpu


def _case(rng, B, L, n, W, dense=0.15):
    """ascending decoded positions (a cluster, so pairs fall in the window),
    marginals like a step's max-probabilities, joints = product x a factor
    that is below 0.5 for about `dense` of the pairs"""
    dec = np.full((B, n), -1, np.int32)
    for b in range(B):
        k = int(rng.integers(0, n + 1)) if b % 3 == 2 else n
        span = min(L, max(k, int(k * rng.uniform(1.0, 3.0))))
        lo = int(rng.integers(0, L - span + 1))
        dec[b, :k] = np.sort(rng.choice(np.arange(lo, lo + span), size=k, replace=False))
    pm = rng.uniform(0.3, 1.0, (B, n)).astype(np.float32)
    pm[rng.random((B, n)) < 0.02] = 0.0
    fac = np.exp(rng.normal(0.0, 0.4, (B, n, W - 1)))
    fac[rng.random((B, n, W - 1)) < dense] *= 0.3
    pj = (pm[:, :, None] * pm[:, :, None] * fac).astype(np.float32)   # the partner's marginal differs: any value works
    return dec, pm, pj


def _run_case(orc, D, L, dec, pm, pj, W, tau, label, seed=0):
    B, n = dec.shape
    say("verify", label, "B", B, "L", L, "n", n, "W", W)
    rng = np.random.default_rng(seed)
    mask = (rng.random((B, L)) < 0.1).astype(np.uint8)
    stable = (rng.random((B, L)) < 0.7).astype(np.uint8)
    cached = (rng.random((B, L)) < 0.8).astype(np.uint8)
    st = D.StabilityState(B, L, 2)
    st.mask.copy_(torch.from_numpy(mask))
    st.stable.copy_(torch.from_numpy(stable))
    st.cached.copy_(torch.from_numpy(cached))
    nrb = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    rbp = torch.full((B, n), -7, dtype=torch.int32, device="cuda")
    rb = D.dllm_self_verify(st, torch.from_numpy(dec).cuda(), torch.from_numpy(pm).cuda(),
                            torch.from_numpy(pj).cuda(), W, tau, n_rollback=nrb, rb_pos=rbp)
    torch.cuda.synchronize()
    r = orc.self_verify(L, dec, pm, pj, W, tau, mask, stable, cached)
    assert np.array_equal(rb.cpu().numpy(), r["rollback"]), label
    assert np.array_equal(st.mask.cpu().numpy(), mask), label
    assert np.array_equal(st.stable.cpu().numpy(), stable), label
    assert np.array_equal(st.cached.cpu().numpy(), cached), label
    assert np.array_equal(st.count.cpu().numpy(), r["count"]), label
    assert np.array_equal(st.next_pos.cpu().numpy(), r["next_pos"]), label
    assert np.array_equal(nrb.cpu().numpy(), r["n_rollback"]), label
    assert np.array_equal(rbp.cpu().numpy(), r["rb_pos"]), label
    return r


def test_random_ragged(orc):
    D = need_gpu()
    rng = np.random.default_rng(31)
    total = 0
    for trial in range(24):
        L = int(rng.choice([1, 5, 63, 64, 65, 700, 1024, 1025, 2049]))
        W = int(rng.integers(2, 9))
        n = int(rng.integers(0, min(L, 300) + 1))
        B = int(rng.integers(1, 5))
        dec, pm, pj = _case(rng, B, L, n, W)
        tau = float(rng.choice([0.25, 0.5, 0.9]))
        r = _run_case(orc, D, L, dec, pm, pj, W, tau, f"random {trial}", seed=trial)
        total += int(r["n_rollback"].sum())
    assert total > 0


def test_long_lists_cross_chunks(orc):
    """3000 and 4097 decoded entries: conflicts across the 1024-entry chunk
    boundaries need the halo of W-1 earlier entries"""
    D = need_gpu()
    rng = np.random.default_rng(32)
    for L, n in [(8192, 3000), (4097, 4097)]:
        dec, pm, pj = _case(rng, 2, L, n, 8, dense=0.05)
        dec[0, :n] = np.sort(rng.choice(L, size=n, replace=False))
        r = _run_case(orc, D, L, dec, pm, pj, 8, 0.5, f"long L={L} n={n}")
        assert r["n_rollback"].sum() > 0


@pytest.mark.parametrize("shape", ["vocab", "longctx"])
def test_full_size(orc, shape):
    """the vocab sweep's 64 x 512 with 16 positions decoded per step (the
    early parallel width) and the long-context 4 x 32768 with its 64-position
    block decoded at once; window 4, tau 0.5"""
    D = need_gpu()
    cfg = W_.CONFIGS[shape]
    B, L = cfg.B, cfg.L
    n = 16 if shape == "vocab" else cfg.b
    rng = np.random.default_rng(33)
    dec, pm, pj = _case(rng, B, L, n, 4)
    if shape == "longctx":
        dec[:] = np.arange(L - n, L, dtype=np.int32)                 # the block at the end
    r = _run_case(orc, D, L, dec, pm, pj, 4, 0.5, f"full {shape}")
    assert r["n_rollback"].sum() > 0


def test_degenerate_lists(orc):
    D = need_gpu()
    rng = np.random.default_rng(34)
    L, W = 300, 5
    # no entries at all, only padding, one entry, and every pair in conflict
    _run_case(orc, D, L, np.zeros((2, 0), np.int32), np.zeros((2, 0), np.float32),
              np.zeros((2, 0, W - 1), np.float32), W, 0.5, "n = 0")
    _run_case(orc, D, L, np.full((2, 6), -1, np.int32), np.ones((2, 6), np.float32),
              np.zeros((2, 6, W - 1), np.float32), W, 0.5, "padding only")
    _run_case(orc, D, L, np.array([[7]], np.int32), np.ones((1, 1), np.float32),
              np.zeros((1, 1, W - 1), np.float32), W, 0.5, "one entry")
    dec = np.arange(100, 140, dtype=np.int32)[None, :]
    r = _run_case(orc, D, L, dec, np.full((1, 40), 0.9, np.float32), np.zeros((1, 40, W - 1), np.float32),
                  W, 0.5, "all conflict")
    assert r["n_rollback"][0] == 40


def test_unsorted_list_is_rejected(orc):
    """a sequence whose list is not ascending is left unchanged with count -1;
    the others are processed (the oracle rejects such a list outright)"""
    D = need_gpu()
    rng = np.random.default_rng(35)
    B, L, n, W = 3, 200, 8, 3
    dec, pm, pj = _case(rng, B, L, n, W, dense=0.5)
    dec[0] = np.arange(10, 10 + n)
    dec[1] = np.arange(10, 10 + n)[::-1]                              # descending
    dec[2] = np.arange(50, 50 + n)
    st = D.StabilityState(B, L, 2)
    st.mask.zero_()
    st.count.fill_(5)
    nrb = torch.zeros(B, dtype=torch.int32, device="cuda")
    say("verify unsorted")
    D.dllm_self_verify(st, torch.from_numpy(dec).cuda(), torch.from_numpy(pm).cuda(),
                       torch.from_numpy(pj).cuda(), W, 0.5, n_rollback=nrb)
    torch.cuda.synchronize()
    assert st.count[1].item() == -1 and nrb[1].item() == -1
    assert not st.mask[1].any().item()
    good = np.delete(np.arange(B), 1)
    mask = np.zeros((2, L), np.uint8)
    r = orc.self_verify(L, dec[good], pm[good], pj[good], W, 0.5, mask)
    assert np.array_equal(st.mask.cpu().numpy()[good], mask)
    assert np.array_equal(nrb.cpu().numpy()[good], r["n_rollback"])
