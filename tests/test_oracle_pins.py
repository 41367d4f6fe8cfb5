"""Pins of the fp64 oracle against facts fixed outside the oracle itself.

MAC-Attention (arXiv 2604.00235) prints no worked example and no error bound,
so each oracle function is pinned by mathematics it must satisfy, checked
through a route that does not reuse the oracle's own formula:
  attend  -> scipy softmax / logsumexp; closed-form special cases
  rope    -> complex-number rotation; 80-bit extended-precision angles
  merge   -> split invariance against a single attend (Figure 2 (b) identity)
  remove  -> (X (+) Y) (-) Y = X (Figure 2 (c) identity)
  nearest -> numpy brute-force argmin with the tie rule
  step    -> an independent segment model of the whole policy (below), plus the
             invariants the pages fix: a miss is full attention; with p = m the
             reuse path reproduces full attention; on a hit the keys read do not
             depend on the context length (abstract).
"""
import math

import numpy as np
import pytest
from scipy.special import logsumexp, softmax

import oracle

RNG = np.random.default_rng(12345)


def _rand_kv(n, d, rng=RNG):
    return (rng.standard_normal((n, d)).astype(np.float32),
            rng.standard_normal((n, d)).astype(np.float32))


def _rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


# ------------------------------------------------------------------ attend

@pytest.mark.parametrize("n,d", [(1, 4), (7, 4), (33, 128), (300, 16)])
def test_attend_matches_scipy_softmax(n, d):
    k, v = _rand_kv(n, d)
    q = RNG.standard_normal(d)
    scale = 1.0 / math.sqrt(d)
    s = oracle.attend(q, k, v, 0, n - 1, scale)
    logits = (k.astype(np.float64) @ q) * scale
    o_ref = softmax(logits) @ v.astype(np.float64)
    assert _rel(s[:d], o_ref) < 1e-13
    # M + log(l) is the log-sum-exp of the logits whatever M is
    assert abs(s[d] + math.log(s[d + 1]) - logsumexp(logits)) < 1e-12
    assert s[d] == pytest.approx(logits.max(), rel=1e-14, abs=1e-15)


def test_attend_subrange_and_bf16_bits():
    n, d = 50, 8
    k, v = _rand_kv(n, d)
    # round to bf16 by truncating mantissa bits: the oracle must read the bit pattern exactly
    kb = (k.view(np.uint32) >> 16).astype(np.uint16)
    vb = (v.view(np.uint32) >> 16).astype(np.uint16)
    kf = (kb.astype(np.uint32) << 16).view(np.float32)
    vf = (vb.astype(np.uint32) << 16).view(np.float32)
    q = RNG.standard_normal(d)
    a, b = 11, 37
    s_bits = oracle.attend(q, kb, vb, a, b, 0.3)
    logits = (kf[a:b + 1].astype(np.float64) @ q) * 0.3
    o_ref = softmax(logits) @ vf[a:b + 1].astype(np.float64)
    assert _rel(s_bits[:d], o_ref) < 1e-13


def test_attend_special_cases():
    d = 16
    k, v = _rand_kv(9, d)
    q = RNG.standard_normal(d)
    # one key -> its value, l = 1, M = its logit
    s = oracle.attend(q, k, v, 4, 4, 0.5)
    assert np.array_equal(s[:d], v[4].astype(np.float64))
    assert s[d + 1] == 1.0
    # identical keys -> plain mean of the values
    kk = np.repeat(k[:1], 9, axis=0)
    s = oracle.attend(q, kk, v, 0, 8, 0.5)
    assert _rel(s[:d], v.astype(np.float64).mean(0)) < 1e-14
    # zero query -> plain mean too
    s = oracle.attend(np.zeros(d), k, v, 0, 8, 0.5)
    assert _rel(s[:d], v.astype(np.float64).mean(0)) < 1e-14
    # empty range -> EMPTY
    s = oracle.attend(q, k, v, 5, 4, 0.5)
    assert s[d] == -np.inf and s[d + 1] == 0.0 and not s[:d].any()
    # logits far beyond exp's range stay finite (max-shifted)
    s = oracle.attend(q * 1e4, k, v, 0, 8, 1.0)
    assert np.all(np.isfinite(s[:d])) and s[d + 1] >= 1.0


# -------------------------------------------------------------------- rope

def _rope_complex(x, m, theta):
    d = x.shape[0]
    h = d // 2
    z = x[:h].astype(np.float64) + 1j * x[h:].astype(np.float64)
    ang = m * theta ** (-2.0 * np.arange(h) / d)
    w = z * np.exp(1j * ang)
    return np.concatenate([w.real, w.imag])


@pytest.mark.parametrize("m", [0, 1, 17, 4096, 131327])
def test_rope_is_complex_rotation(m):
    x = RNG.standard_normal(128).astype(np.float32)
    got = oracle.rope(x, m, 500000.0)
    ref = _rope_complex(x, m, 500000.0)
    assert np.max(np.abs(got - ref)) < 1e-9
    assert abs(np.linalg.norm(got) - np.linalg.norm(x.astype(np.float64))) < 1e-12
    if m == 0:
        assert np.array_equal(got, x.astype(np.float64))


def test_rope_angles_in_extended_precision():
    """At m = 131327 an fp32 angle errs by ~3e-3 rad; the oracle must be near the
    80-bit result."""
    ld = np.longdouble
    x = RNG.standard_normal(128).astype(np.float32)
    m, theta, d = 131327, 500000.0, 128
    got = oracle.rope(x, m, theta)
    i = np.arange(64, dtype=ld)
    phi = ld(m) * np.power(ld(theta), -ld(2) * i / ld(d))
    c, s = np.cos(phi), np.sin(phi)
    a, b = x[:64].astype(ld), x[64:].astype(ld)
    ref = np.concatenate([a * c - b * s, b * c + a * s]).astype(np.float64)
    assert np.max(np.abs(got - ref)) < 1e-9
    # an fp32 angle would be visibly off
    phi32 = (np.float32(m) * (np.float32(theta) ** (-2 * np.arange(64, dtype=np.float32) / 128)))
    bad = np.concatenate([x[:64] * np.cos(phi32) - x[64:] * np.sin(phi32),
                          x[64:] * np.cos(phi32) + x[:64] * np.sin(phi32)])
    assert np.max(np.abs(bad - ref)) > 1e-4


def test_rope_relative_position():
    q = RNG.standard_normal(64).astype(np.float32)
    k = RNG.standard_normal(64).astype(np.float32)
    lhs = oracle.rope(q, 1000, 1e4) @ oracle.rope(k, 700, 1e4)
    rhs = oracle.rope(q, 300, 1e4) @ k.astype(np.float64)
    assert abs(lhs - rhs) < 1e-10


# ---------------------------------------------------------- merge / remove

def test_merge_split_invariance_every_split():
    n, d = 40, 8
    k, v = _rand_kv(n, d)
    q = RNG.standard_normal(d) * 2.0
    whole = oracle.attend(q, k, v, 0, n - 1, 0.7)
    for a in range(-1, n):
        left = oracle.attend(q, k, v, 0, a, 0.7)
        right = oracle.attend(q, k, v, a + 1, n - 1, 0.7)
        z = oracle.merge(left, right)
        assert _rel(z[:d], whole[:d]) < 1e-13
        assert abs((z[d] + math.log(z[d + 1])) - (whole[d] + math.log(whole[d + 1]))) < 1e-13


def test_merge_commutative_associative_identity():
    n, d = 30, 8
    k, v = _rand_kv(n, d)
    q = RNG.standard_normal(d)
    x = oracle.attend(q, k, v, 0, 9, 1.0)
    y = oracle.attend(q, k, v, 10, 19, 1.0)
    z = oracle.attend(q, k, v, 20, 29, 1.0)
    assert _rel(oracle.merge(x, y), oracle.merge(y, x)) < 1e-15
    l1 = oracle.merge(oracle.merge(x, y), z)
    l2 = oracle.merge(x, oracle.merge(y, z))
    assert _rel(l1[:d], l2[:d]) < 1e-14
    e = oracle.empty(d)
    assert np.array_equal(oracle.merge(x, e), x)
    assert np.array_equal(oracle.merge(e, x), x)


def test_remove_inverts_merge():
    n, d = 60, 16
    k, v = _rand_kv(n, d)
    for trial in range(20):
        q = RNG.standard_normal(d)
        a = int(RNG.integers(0, n - 2))
        b = int(RNG.integers(a + 1, n))
        x = oracle.attend(q, k, v, 0, a, 0.25)
        y = oracle.attend(q, k, v, a + 1, b - 1 if b - 1 > a else a + 1, 0.25)
        got = oracle.remove(oracle.merge(x, y), y)
        assert _rel(got[:d], x[:d]) < 1e-12
        assert abs(got[d] + math.log(got[d + 1]) - (x[d] + math.log(x[d + 1]))) < 1e-12


def test_remove_degenerate_and_identity():
    d = 8
    k, v = _rand_kv(10, d)
    q = RNG.standard_normal(d)
    y = oracle.attend(q, k, v, 0, 9, 1.0)
    assert oracle.remove(y, y)[d + 1] == 0.0        # nothing left -> EMPTY
    assert np.array_equal(oracle.remove(y, oracle.empty(d)), y)


# ------------------------------------------------------------------ match

def _brute_nearest(qt, ring_q, ring_pos, m):
    best, key = -1, None
    for j in range(len(ring_pos)):
        if ring_pos[j] < 0 or ring_pos[j] > m:
            continue
        D = float(np.sum((qt.astype(np.float64) - ring_q[j].astype(np.float64)) ** 2))
        kj = (D, -int(ring_pos[j]), -j)
        if key is None or kj < key:
            best, key = j, kj
    return best


def test_nearest_bruteforce_with_ties():
    d, W = 4, 8
    for trial in range(200):
        ring_q = RNG.integers(-2, 3, size=(W, d)).astype(np.float32)   # many exact ties
        ring_pos = RNG.integers(-1, 12, size=W).astype(np.int32)
        qt = RNG.integers(-2, 3, size=d).astype(np.float32)
        m = int(RNG.integers(0, 12))
        j, d1, d2 = oracle.nearest(qt, ring_q, ring_pos, m)
        assert j == _brute_nearest(qt, ring_q, ring_pos, m)
        valid = [(float(np.sum((qt - ring_q[i]) ** 2))) for i in range(W)
                 if 0 <= ring_pos[i] <= m]
        if valid:
            srt = sorted(valid)
            assert d1 == srt[0]
            assert d2 == (srt[1] if len(srt) > 1 else np.inf)
        else:
            assert j == -1


def test_nearest_bruteforce_large_window():
    """Windows of the pages' operating point (512-2048 entries, Table 7), with
    stale and future stamps and planted exact duplicates of the best entry."""
    d = 128
    for W in (513, 2048):
        ring_q = RNG.standard_normal((W, d)).astype(np.float32)
        ring_pos = RNG.integers(-1, 3000, size=W).astype(np.int32)
        qt = RNG.standard_normal(d).astype(np.float32)
        m = 2500
        j0 = _brute_nearest(qt, ring_q, ring_pos, m)
        for dup in RNG.choice(W, size=3, replace=False):
            ring_q[dup] = ring_q[j0]
        j, _, _ = oracle.nearest(qt, ring_q, ring_pos, m)
        assert j == _brute_nearest(qt, ring_q, ring_pos, m)


def test_nearest_duplicate_prefers_newest():
    d = 4
    ring_q = np.zeros((4, d), np.float32)
    ring_pos = np.array([5, 9, 7, 2], np.int32)
    j, _, _ = oracle.nearest(np.zeros(d, np.float32), ring_q, ring_pos, 10)
    assert j == 1
    j, _, _ = oracle.nearest(np.zeros(d, np.float32), ring_q, ring_pos, 8)   # pos 9 > m
    assert j == 2


# ------------------------------------------------------ bfloat16 ring queries

def test_round_bf16_matches_torch_conversion():
    """The oracle's bfloat16 rounding against torch's float32 -> bfloat16
    conversion (round to nearest, ties to even), with planted exact ties."""
    import torch
    x = RNG.standard_normal(4000).astype(np.float32) * np.float32(3.0)
    bits = x.view(np.uint32)
    ties = (bits[:1000] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)    # exactly half an ulp
    x[:1000] = ties.view(np.float32)
    x[1000:1010] = [0.0, -0.0, 1.0, -1.0, 65504.0, 1e-38, -1e-38, 3.3895314e38, 1e30, 7.0]
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    got = oracle.round_bf16(x)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_ring_bf16_stores_rounded_queries_and_matches_on_them():
    """With F_RING_BF16 the ring holds bfloat16-rounded pre-RoPE queries and
    the decision is the brute-force nearest over those stored values."""
    import torch
    B, Hq, Hkv, d, W, r = 1, 2, 1, 128, 8, 4
    n = 40
    K, V = _rand_kv(n, d)
    Kg, Vg = [K], [V]
    orc = oracle.Oracle(B, Hq, Hkv, d, W, r, 0.3, 5e5, flags=oracle.F_RING_BF16)
    plain = oracle.Oracle(B, Hq, Hkv, d, W, r, 0.3, 5e5)
    q = RNG.standard_normal((Hq, d))
    for t in range(20):
        q = 0.97 * q + math.sqrt(1 - 0.97 ** 2) * RNG.standard_normal((Hq, d))
        qf = q.astype(np.float32)[None]
        m = 10 + t
        # expected decisions from the stored entries, read before the step inserts
        expect = []
        for h in range(Hq):
            entries = [orc.ring_entry(0, h, j) for j in range(W)]
            ring_q = np.stack([e[1] for e in entries])
            ring_pos = np.array([e[0] for e in entries], np.int32)
            for e in entries:
                if e[0] >= 0:
                    assert np.array_equal(e[1], torch.from_numpy(e[1]).to(torch.bfloat16)
                                          .to(torch.float32).numpy())
            j = _brute_nearest(qf[0, h], ring_q, ring_pos, m)
            qd = qf[0, h].astype(np.float64)
            hit = j >= 0 and float(np.sum((qd - ring_q[j]) ** 2)) <= 0.09 * float(np.sum(qd * qd))
            expect.append((hit, int(ring_pos[j]) if hit else -1))
        res = orc.step(Kg, Vg, np.array([m + 1]), qf)
        for h, (hit, p) in enumerate(expect):
            assert bool(res["hit"][0, h]) == hit
            if hit:
                assert res["p"][0, h] == p
        plain.step(Kg, Vg, np.array([m + 1]), qf)
    # the plain oracle keeps the exact fp32 queries
    pos, qp, _ = plain.ring_entry(0, 0, (20 - 1) % W)
    pos_b, qb, _ = orc.ring_entry(0, 0, (20 - 1) % W)
    assert pos == pos_b and not np.array_equal(qp, qb)
    assert np.array_equal(qb, oracle.round_bf16(qp))
