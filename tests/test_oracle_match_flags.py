"""Pins of the oracle's match outputs that decide what the GPU parity harness
forces: the relative distance `rel`, the near-threshold flag `near_tau` and
the near-tie flag `near_tie` of orc_step.

The pages define the match as the nearest recent pre-RoPE query under an L2
threshold (MAC-Attention paper card, Figure 2 (a)); the threshold is read as
relative, rel = ||q~_m - q~_p|| / ||q~_m|| <= tau.  The two flags mark the
decisions whose outcome fp32 rounding could flip: |rel - tau| < 1e-4, and a
second-nearest squared distance within a relative 1e-5 of the nearest.

Every value checked here comes from planted geometry, not from the oracle's
formula: the query is s * e_0 and a ring entry is q + t * e_k, so the squared
distance is exactly fp32(t)^2 and rel is |fp32(t)| / s in closed form.  The
margins planted (+-5e-5 against +-1.5e-4 and +-2e-4 of tau; relative gaps of
0, 2e-6 and 5e-6 against 3e-5 and 1e-4) sit far from the 1e-4 and 1e-5 cuts
compared with fp32 rounding (~1e-7), and the scales (s from 0.25 to 37,
distances from 1e-2 to 30) make an absolute margin, a squared-rel margin or an
unnormalised rel fail.
"""
import numpy as np
import pytest

import oracle

D = 8


def _decide(entries, q, tau, W=None):
    """One request, one head: insert each pre-RoPE query of `entries` (oldest
    first, positions 0, 1, ...) by one decode call, then decode `q` at the next
    position.  Returns the last call's result for the head."""
    n = len(entries) + 1
    W = W or n
    rng = np.random.default_rng(7)
    K = rng.standard_normal((n, D)).astype(np.float32)
    V = rng.standard_normal((n, D)).astype(np.float32)
    orc = oracle.Oracle(1, 1, 1, D, W, 1, tau, 500000.0, kv_fp32=True)
    for t, x in enumerate(entries):
        orc.step([K], [V], np.array([t + 1], np.int32),
                 np.asarray(x, np.float32).reshape(1, 1, D))
    res = orc.step([K], [V], np.array([n], np.int32), np.asarray(q, np.float32).reshape(1, 1, D))
    return {k: (v[0, 0] if isinstance(v, np.ndarray) and v.ndim >= 2 else v)
            for k, v in res.items()}


def _e(k, scale=1.0):
    x = np.zeros(D, np.float32)
    x[k] = scale
    return x


def pin_rel_and_near_tau():
    """rel in closed form and the 1e-4 band around tau, at several query
    norms and thresholds; the hit decision on the same plants."""
    for tau in (0.3, 0.05, 1.2):
        for s in (1.0, 3.0, 0.25, 37.0):
            for delta in (5e-5, -5e-5, 1.5e-4, -1.5e-4, 2e-4, -2e-4, 3e-3, -3e-3):
                q = _e(0, s)
                t = np.float32((tau + delta) * s)
                x = q + _e(1, float(t))
                assert x[1] == t                   # the planted offset is exact in fp32
                rel = abs(float(t)) / s            # the closed form
                r = _decide([x], q, tau)
                assert r["rel"] == pytest.approx(rel, rel=1e-14, abs=0), (tau, s, delta)
                assert bool(r["near_tau"]) == (abs(rel - tau) < 1e-4), (tau, s, delta)
                assert bool(r["near_tau"]) == (abs(delta) < 1e-4), (tau, s, delta)
                assert bool(r["hit"]) == (rel <= tau), (tau, s, delta)
                assert r["p"] == (0 if rel <= tau else -1)


def pin_near_tie():
    """Second-nearest squared distance within a relative 1e-5 of the nearest,
    at distances from 1e-2 to 30, with the nearer entry older or newer and a
    third entry farther away."""
    for a in (0.01, 1.0, 30.0):
        for eps in (0.0, 2e-6, 5e-6, 3e-5, 1e-4, 0.5):
            for s in (1.0, 50.0):
                q = _e(0, s)
                fa = np.float32(a)
                fb = np.float32(a * np.sqrt(1.0 + eps))
                xa, xb, xc = q + _e(1, float(fa)), q + _e(2, float(fb)), q + _e(3, 10 * a + 1)
                da, db = float(fa) ** 2, float(fb) ** 2     # exact in float64
                gap = (db - da) / da
                for order in ((xa, xb, xc), (xb, xa, xc), (xc, xa, xb), (xb, xc, xa)):
                    r = _decide(list(order), q, 1.0e9)      # tau huge: always a hit
                    assert bool(r["near_tie"]) == (gap <= 1e-5), (a, eps, s, gap)
                    assert r["rel"] == pytest.approx(float(fa) / s, rel=1e-14)
                    # the nearest entry wins; an exact tie goes to the newer one
                    pa = [i for i, x in enumerate(order) if x is xa][0]
                    pb = [i for i, x in enumerate(order) if x is xb][0]
                    want = (max(pa, pb) if db == da else pa)
                    assert r["p"] == want, (a, eps, s, pa, pb)
    # exact duplicates at different positions: a tie, decided for the newest
    q = _e(0, 2.0)
    x = q + _e(1, 0.3)
    r = _decide([x, _e(5, 9.0), x], q, 0.5)
    assert r["near_tie"] == 1 and r["p"] == 2 and r["hit"] == 1
    # one valid entry: no second distance, no tie
    r = _decide([x], q, 0.5)
    assert r["near_tie"] == 0 and r["hit"] == 1
    # empty ring (first call): no distance at all
    r = _decide([], q, 0.5)
    assert np.isnan(r["rel"]) and r["near_tau"] == 0 and r["near_tie"] == 0 and r["hit"] == 0


def pin_zero_query():
    """A zero query: rel is 0 for an exact zero entry (a hit at any tau >= 0)
    and infinite otherwise."""
    z = np.zeros(D, np.float32)
    r = _decide([_e(1, 0.5)], z, 0.3)
    assert r["rel"] == np.inf and r["hit"] == 0 and r["near_tau"] == 0
    r = _decide([_e(1, 0.5), z], z, 0.0)
    assert r["rel"] == 0.0 and r["hit"] == 1 and r["p"] == 1


def pin_random_rings():
    """Random rings (stale slots included): rel, the flags and the nearest
    entry recomputed in numpy from the stored fp32 queries."""
    rng = np.random.default_rng(99)
    for trial in range(60):
        W = int(rng.integers(2, 12))
        n = int(rng.integers(1, 2 * W))
        base = rng.standard_normal(D).astype(np.float32)
        entries = [(base + rng.standard_normal(D) * rng.uniform(0.05, 1.0)).astype(np.float32)
                   for _ in range(n)]
        q = (base + 0.1 * rng.standard_normal(D)).astype(np.float32)
        tau = float(rng.uniform(0.05, 1.0))
        r = _decide(entries, q, tau, W=W)
        live = entries[-W:]                      # FIFO: the last W insertions
        pos = list(range(n - len(live), n))
        dist = np.array([np.sum((x.astype(np.float64) - q.astype(np.float64)) ** 2)
                         for x in live])
        # nearest entry; equal distances go to the newest position
        j = min(range(len(live)), key=lambda i: (dist[i], -pos[i]))
        rel = np.sqrt(dist[j]) / np.linalg.norm(q.astype(np.float64))
        assert r["rel"] == pytest.approx(rel, rel=1e-12)
        assert bool(r["near_tau"]) == (abs(rel - tau) < 1e-4)
        srt = np.sort(dist)
        tie = len(srt) > 1 and (srt[1] - srt[0]) <= 1e-5 * srt[0]
        assert bool(r["near_tie"]) == tie
        assert bool(r["hit"]) == (dist[j] <= tau * tau * float(np.sum(q.astype(np.float64) ** 2)))
        assert r["p"] == (pos[j] if r["hit"] else -1)


PINS = [pin_rel_and_near_tau, pin_near_tie, pin_zero_query, pin_random_rings]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_match_outputs(pin):
    pin()
