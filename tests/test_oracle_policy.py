"""Pins of the oracle's decode policy (match -> complete -> amend).

The independent model below never uses (+) or (-).  It keeps each stored
summary AS_{1:p-r} as an explicit list of segments (query vector, first key,
last key): in exact arithmetic a hit's output is one softmax over the union of
the stored segments and the band+tail segment, and amend's result is that
union with the last r keys of the newest segment cut off (MAC-Attention,
Figure 2 (b), (c)).  The model evaluates every output as a single scipy
softmax over the concatenated logits, takes decisions by numpy brute force and
rotates queries with complex numbers, so a dropped term, a wrong band or range
end, a wrong tie rule or a wrong rotation in the oracle fails here.
"""
import math

import numpy as np
import pytest
from scipy.special import softmax

import oracle
from workloads import get_config, kv_logical, queries, scaled, bf16_bits


def _rope_complex(x, m, theta):
    d = x.shape[0]
    h = d // 2
    z = x[:h].astype(np.float64) + 1j * x[h:].astype(np.float64)
    w = z * np.exp(1j * m * theta ** (-2.0 * np.arange(h) / d))
    return np.concatenate([w.real, w.imag])


def _kvf(a):
    """float64 view of fp32 rows or bf16 bit rows."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


class SegmentModel:
    def __init__(self, B, Hq, Hkv, d, W, r, tau, theta, flags=0):
        self.B, self.Hq, self.Hkv, self.d, self.W = B, Hq, Hkv, d, W
        self.band = [int(x) for x in np.broadcast_to(np.asarray(r), (Hq,))]
        self.tau, self.theta, self.flags = tau, theta, flags
        self.scale = 1.0 / math.sqrt(d)
        self.ring = [[[None] * W for _ in range(Hq)] for _ in range(B)]
        self.calls = 0

    def _visible(self, e):
        """An entry inserted by call c takes part in call t's match when
        c <= t - 1, or c <= t - 2 for the stale-by-one ring."""
        lag = 2 if self.flags & oracle.F_STALE_RING else 1
        return e["call"] <= self.calls - lag

    def _value(self, segs, Kf, Vf):
        logits, rows = [], []
        for q, a, b in segs:
            idx = np.arange(a, b + 1)
            logits.append((Kf[idx] @ q) * self.scale)
            rows.append(Vf[idx])
        return softmax(np.concatenate(logits)) @ np.concatenate(rows)

    def step(self, Kg, Vg, seq_lens, q_pre, override=None):
        B, Hq, W = self.B, self.Hq, self.W
        G = Hq // self.Hkv
        slot_new = self.calls % W
        reuse = not (self.flags & oracle.F_DISABLE_REUSE) and self.tau >= 0
        out = np.zeros((B, Hq, self.d))
        hit = np.zeros((B, Hq), np.uint8)
        p_out = np.full((B, Hq), -1, np.int32)
        for b in range(B):
            m = int(seq_lens[b]) - 1
            if m < 0:
                continue
            for h in range(Hq):
                r = self.band[h]
                qt = q_pre[b, h]
                ring = self.ring[b][h]
                slot = -1
                if reuse:
                    key = None
                    for j in range(W):
                        e = ring[j]
                        if e is None or e["pos"] > m or not self._visible(e):
                            continue
                        D = float(np.sum((qt.astype(np.float64) - e["qt"].astype(np.float64)) ** 2))
                        kj = (D, -e["pos"], -j)
                        if key is None or kj < key:
                            key, best = kj, j
                    if key is not None:
                        qn2 = float(np.sum(qt.astype(np.float64) ** 2))
                        if key[0] <= self.tau ** 2 * qn2:
                            slot = best
                    if override is not None and override[b, h] != -2:
                        slot = -1
                        for j in range(W):
                            if ring[j] is not None and ring[j]["pos"] == override[b, h] \
                                    and ring[j]["pos"] <= m and self._visible(ring[j]):
                                slot = j
                q = _rope_complex(qt, m, self.theta)
                Kf, Vf = Kg[b * self.Hkv + h // G], Vg[b * self.Hkv + h // G]
                if slot >= 0:
                    p = ring[slot]["pos"]
                    start = max(p - r + 1, 0)
                    segs = list(ring[slot]["segs"]) + [(q, start, m)]
                    hit[b, h], p_out[b, h] = 1, p
                else:
                    start = 0
                    segs = [(q, 0, m)]
                out[b, h] = self._value(segs, Kf, Vf)
                # amend: the stored summary covers keys up to m-r
                if m - r < 0:
                    kept = []
                else:
                    kept = list(segs[:-1])
                    if start <= m - r:
                        kept.append((q, start, m - r))
                if reuse:
                    ring[slot_new] = {"pos": m, "qt": qt.copy(), "segs": kept, "call": self.calls}
        self.calls += 1
        return out, hit, p_out


def _setup(kv="fp32", B=2, Hq=4, Hkv=2, d=8, C=12, steps=40, W=4, r=3, rho=0.9, seed=3):
    w = scaled(get_config("cpu4k"), B=B, Hq=Hq, Hkv=Hkv, d=d, C=C, steps=steps, W=W, r=r,
               rho=("const", rho), kv=kv, seed=seed)
    k, v = kv_logical(w, "cpu")
    kb, vb = bf16_bits(k), bf16_bits(v)
    Kg = [kb[b, g] for b in range(B) for g in range(Hkv)]
    Vg = [vb[b, g] for b in range(B) for g in range(Hkv)]
    return w, Kg, Vg, queries(w)


_STALE = oracle.F_STALE_RING


@pytest.mark.parametrize("kv,tau,W,r,flags", [("fp32", 0.5, 4, 3, 0), ("bf16", 0.45, 4, 5, 0),
                                              ("fp32", 1e9, 3, 2, 0), ("bf16", 0.0, 2, 4, 0),
                                              ("fp32", 0.6, 1, 3, 0),
                                              # a ring longer than the run never evicts:
                                              # the unbounded window of the prefill reading
                                              ("fp32", 0.5, 64, 3, 0),
                                              ("fp32", 0.5, 4, 3, _STALE),
                                              ("bf16", 1e9, 3, 2, _STALE),
                                              ("fp32", 1e9, 1, 3, _STALE)])
def test_policy_matches_segment_model(kv, tau, W, r, flags):
    w, Kg, Vg, qs = _setup(kv=kv, W=W, r=r)
    theta = 10000.0
    orc = oracle.Oracle(w.B, w.Hq, w.Hkv, w.d, W, r, tau, theta, kv_fp32=(kv == "fp32"),
                        flags=flags)
    mod = SegmentModel(w.B, w.Hq, w.Hkv, w.d, W, r, tau, theta, flags=flags)
    KgF = [_kvf(a) for a in Kg]
    VgF = [_kvf(a) for a in Vg]
    nhit = 0
    for t in range(w.steps):
        seq = np.full(w.B, w.C + t + 1, np.int32)
        res = orc.step(Kg, Vg, seq, qs[t])
        out, hit, p = mod.step(KgF, VgF, seq, qs[t])
        assert np.array_equal(res["hit"], hit), t
        assert np.array_equal(res["p"], p), t
        np.testing.assert_allclose(res["out"], out, rtol=1e-10, atol=1e-12)
        nhit += int(hit.sum())
    if tau >= 1e9:
        # every call hits the newest visible entry; the stale ring sees none
        # in its first two calls, and none at all with a single slot
        first = 2 if flags & _STALE else 1
        want = 0 if (flags & _STALE and W == 1) else (w.steps - first) * w.B * w.Hq
        assert nhit == want
    elif tau > 0:
        assert 0 < nhit < w.steps * w.B * w.Hq      # the case mixes hits and misses


@pytest.mark.parametrize("kv,bands,W,flags", [("fp32", [1, 3, 6, 2], 4, 0),
                                              ("bf16", [5, 5, 2, 9], 3, 0),
                                              ("fp32", [2, 7, 1, 4], 4, _STALE)])
def test_per_head_bands_match_segment_model(kv, bands, W, flags):
    """Per-head band r_h (Figure 3 (b)): each head's hit span and amend band
    use its own r_h, including heads of one KV group with different bands."""
    w, Kg, Vg, qs = _setup(kv=kv, W=W, r=max(bands), rho=0.95)
    theta = 10000.0
    orc = oracle.Oracle(w.B, w.Hq, w.Hkv, w.d, W, bands, 0.5, theta, kv_fp32=(kv == "fp32"),
                        flags=flags)
    mod = SegmentModel(w.B, w.Hq, w.Hkv, w.d, W, bands, 0.5, theta, flags=flags)
    KgF = [_kvf(a) for a in Kg]
    VgF = [_kvf(a) for a in Vg]
    nhit = 0
    for t in range(w.steps):
        seq = np.full(w.B, w.C + t + 1, np.int32)
        res = orc.step(Kg, Vg, seq, qs[t])
        out, hit, p = mod.step(KgF, VgF, seq, qs[t])
        assert np.array_equal(res["hit"], hit), t
        assert np.array_equal(res["p"], p), t
        np.testing.assert_allclose(res["out"], out, rtol=1e-10, atol=1e-12)
        starts = np.where(hit != 0, np.maximum(p - np.asarray(bands)[None, :] + 1, 0), 0)
        assert np.array_equal(res["start"], starts), t
        nhit += int(hit.sum())
    assert 0 < nhit < w.steps * w.B * w.Hq


def test_tau_zero_hits_only_exact_repeats():
    w, Kg, Vg, qs = _setup(kv="fp32", W=4, r=3)
    orc = oracle.Oracle(w.B, w.Hq, w.Hkv, w.d, 4, 3, 0.0, 1e4, kv_fp32=True)
    mod = SegmentModel(w.B, w.Hq, w.Hkv, w.d, 4, 3, 0.0, 1e4)
    KgF = [_kvf(a) for a in Kg]
    VgF = [_kvf(a) for a in Vg]
    for t in range(6):
        q = qs[t // 2]                          # every query appears twice in a row
        seq = np.full(w.B, w.C + t + 1, np.int32)
        res = orc.step(Kg, Vg, seq, q)
        out, hit, _ = mod.step(KgF, VgF, seq, q)
        assert res["hit"].all() == (t % 2 == 1) and res["hit"].any() == (t % 2 == 1)
        if t % 2 == 1:
            assert (res["p"] == w.C + t - 1).all()
        np.testing.assert_allclose(res["out"], out, rtol=1e-10, atol=1e-12)


def _full(w, Kg, Vg, seq, q):
    ref = oracle.Oracle(w.B, w.Hq, w.Hkv, w.d, w.W, w.r, w.tau, 1e4, kv_fp32=(w.kv == "fp32"),
                        flags=oracle.F_DISABLE_REUSE)
    return ref.step(Kg, Vg, seq, q)["out"]


def test_miss_and_disable_reuse_equal_full_attention():
    w, Kg, Vg, qs = _setup(kv="bf16", W=4, r=3)
    orc = oracle.Oracle(w.B, w.Hq, w.Hkv, w.d, 4, 3, 0.5, 1e4, flags=oracle.F_DISABLE_REUSE)
    mix = oracle.Oracle(w.B, w.Hq, w.Hkv, w.d, 4, 3, 0.5, 1e4)
    KgF = [_kvf(a) for a in Kg]
    VgF = [_kvf(a) for a in Vg]
    for t in range(20):
        seq = np.full(w.B, w.C + t + 1, np.int32)
        res = orc.step(Kg, Vg, seq, qs[t], want_full=True)
        assert not res["hit"].any()
        assert np.array_equal(res["out"], res["full"])
        # full attention itself against one scipy softmax per head
        for b in range(w.B):
            for h in range(w.Hq):
                g = b * w.Hkv + h // w.G
                q = _rope_complex(qs[t][b, h], w.C + t, 1e4)
                o = softmax(KgF[g][:w.C + t + 1] @ q / math.sqrt(w.d)) @ VgF[g][:w.C + t + 1]
                np.testing.assert_allclose(res["full"][b, h], o, rtol=1e-11, atol=1e-13)
        # in a mixed run every miss equals full attention
        mr = mix.step(Kg, Vg, seq, qs[t], want_full=True)
        miss = mr["hit"] == 0
        np.testing.assert_allclose(mr["out"][miss], mr["full"][miss], rtol=1e-12, atol=1e-14)


def test_band_covering_context_equals_full_attention():
    """r >= m+1: the stored prefix is always EMPTY and a hit reads [0, m]."""
    w, Kg, Vg, qs = _setup(kv="fp32", W=4, r=3, C=12, steps=20)
    orc = oracle.Oracle(w.B, w.Hq, w.Hkv, w.d, 4, 64, 1e9, 1e4, kv_fp32=True)
    for t in range(20):
        seq = np.full(w.B, w.C + t + 1, np.int32)
        res = orc.step(Kg, Vg, seq, qs[t], want_full=True)
        if t > 0:
            assert res["hit"].all() and (res["start"] == 0).all()
        np.testing.assert_allclose(res["out"], res["full"], rtol=1e-12, atol=1e-14)


def test_forced_redecode_at_own_position_equals_full_attention():
    w, Kg, Vg, qs = _setup(kv="bf16", W=4, r=3)
    orc = oracle.Oracle(w.B, w.Hq, w.Hkv, w.d, 4, 3, 0.5, 1e4)
    for t in range(8):
        seq = np.full(w.B, w.C + t + 1, np.int32)
        miss = np.full((w.B, w.Hq), -1, np.int32)
        first = orc.step(Kg, Vg, seq, qs[t], override=miss, want_full=True)
        force = np.full((w.B, w.Hq), w.C + t, np.int32)
        again = orc.step(Kg, Vg, seq, qs[t], override=force, want_full=True)
        assert again["hit"].all() and (again["p"] == w.C + t).all()
        np.testing.assert_allclose(again["out"], first["full"], rtol=1e-11, atol=1e-13)


def test_all_hit_keys_read_do_not_depend_on_context():
    """Abstract: on a hit, compute and bytes are constant in the context length."""
    tok = []
    for C in (40, 400):
        w, Kg, Vg, qs = _setup(kv="fp32", W=4, r=3, C=C, steps=12)
        orc = oracle.Oracle(w.B, w.Hq, w.Hkv, w.d, 4, 3, 1e9, 1e4, kv_fp32=True)
        rows = []
        for t in range(12):
            seq = np.full(w.B, C + t + 1, np.int32)
            res = orc.step(Kg, Vg, seq, qs[t])
            if t > 0:
                m = C + t
                p = res["p"].reshape(w.B, w.Hkv, w.G)
                assert np.array_equal(res["kv_tokens"], m - p.min(axis=2) + 3)
                rows.append(res["kv_tokens"].copy())
            else:
                assert (res["kv_tokens"] == C + 1).all()
        tok.append(np.array(rows))
    assert np.array_equal(tok[0], tok[1])


def test_override_to_absent_position_is_a_counted_miss():
    w, Kg, Vg, qs = _setup(kv="fp32", W=4, r=3)
    orc = oracle.Oracle(w.B, w.Hq, w.Hkv, w.d, 4, 3, 1e9, 1e4, kv_fp32=True)
    for t in range(3):
        orc.step(Kg, Vg, np.full(w.B, w.C + t + 1, np.int32), qs[t])
    ov = np.full((w.B, w.Hq), -2, np.int32)
    ov[0, 1] = 3                                # no entry stored at position 3
    ov[1, 2] = -1                               # forced miss
    res = orc.step(Kg, Vg, np.full(w.B, w.C + 4, np.int32), qs[3], override=ov, want_full=True)
    assert res["override_invalid"] == 1
    assert res["hit"][0, 1] == 0 and res["hit"][1, 2] == 0
    assert res["hit"].sum() == w.B * w.Hq - 2
    np.testing.assert_allclose(res["out"][0, 1], res["full"][0, 1], rtol=1e-12)


def test_idle_request_and_zero_query():
    w, Kg, Vg, qs = _setup(kv="fp32", W=4, r=3)
    orc = oracle.Oracle(w.B, w.Hq, w.Hkv, w.d, 4, 3, 0.3, 1e4, kv_fp32=True)
    z = np.zeros_like(qs[0])
    seq = np.array([w.C + 1, 0], np.int32)      # request 1 idle
    res = orc.step(Kg, Vg, seq, z)
    assert not res["out"][1].any() and (res["kv_tokens"][1] == 0).all()
    pos, _, _ = orc.ring_entry(1, 0, 0)
    assert pos == -1                            # idle request stores nothing
    res = orc.step(Kg, Vg, np.array([w.C + 2, 0], np.int32), z)
    assert res["hit"][0].all()                  # zero query vs stored zero: D = 0
    z2 = z.copy()
    z2[0, :, 0] = 1.0
    res = orc.step(Kg, Vg, np.array([w.C + 3, 0], np.int32), z2)
    assert not res["hit"][0].any()              # nonzero query: relative distance 1


def test_reset_empties_rings():
    w, Kg, Vg, qs = _setup(kv="fp32", W=4, r=3)
    orc = oracle.Oracle(w.B, w.Hq, w.Hkv, w.d, 4, 3, 1e9, 1e4, kv_fp32=True)
    for t in range(3):
        res = orc.step(Kg, Vg, np.full(w.B, w.C + t + 1, np.int32), qs[t])
    assert res["hit"].all()
    orc.reset()
    res = orc.step(Kg, Vg, np.full(w.B, w.C + 4, np.int32), qs[3])
    assert not res["hit"].any()


def test_stale_ring_hides_only_the_previous_call():
    """Stale-by-one ring: call t's match and override skip the entry of call
    t-1 and see every older one still stored.  The query repeats, so every
    stored entry is at distance 0 and the tie rule picks the newest visible
    one, call t-2's.  After a reset the first two calls miss."""
    w, Kg, Vg, qs = _setup(kv="fp32", W=4, r=3)
    orc = oracle.Oracle(w.B, w.Hq, w.Hkv, w.d, 4, 3, 1e9, 1e4, kv_fp32=True,
                        flags=oracle.F_STALE_RING)
    for rnd in range(2):
        for t in range(6):
            m = w.C + t
            res = orc.step(Kg, Vg, np.full(w.B, m + 1, np.int32), qs[0])
            if t < 2:
                assert not res["hit"].any()
            else:
                assert res["hit"].all() and (res["p"] == m - 2).all()
        m = w.C + 6
        ov = np.full((w.B, w.Hq), -2, np.int32)
        ov[0, 0] = m - 1                        # the previous call's entry: hidden
        ov[0, 1] = m - 2
        ov[1, 0] = m - 4                        # oldest entry still stored (W = 4)
        res = orc.step(Kg, Vg, np.full(w.B, m + 1, np.int32), qs[0], override=ov)
        assert res["override_invalid"] == 1
        assert res["hit"][0, 0] == 0
        assert res["p"][0, 1] == m - 2 and res["p"][1, 0] == m - 4
        orc.reset()
