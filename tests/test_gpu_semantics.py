"""GPU checks of the decode step's semantics through the C ABI.

- async amend on its own stream and amend on the decode stream give bit-identical
  outputs over many steps (amend(m-1) -> match(m) ordering; MAC-Attention
  Figure 2 (c), "async cache update");
- a paged cache with a permuted table gives the same bits as a contiguous one;
- a forced hit at the query's own position after a miss reproduces full
  attention; an override naming no stored position is a counted miss;
- mac_reset empties the rings; idle requests produce zeros and store nothing;
- sequence lengths and page ids out of range are caught on the device;
- the counters agree with the oracle's decisions and key counts;
- misaligned device pointers are refused on the host;
- overrides of every kind through both long-ring match forms;
- calls moving between two streams with no host synchronisation.
"""
import numpy as np
import pytest
import torch

import kv_reuse_amd as mac
import oracle
from workloads import get_config, kv_logical, page_table, queries, scaled, to_paged

pytestmark = pytest.mark.gpu


def _case(**kw):
    base = dict(B=3, C=900, steps=40, rho=("const", 0.965))
    base.update(kw)
    return scaled(get_config("b16_128k"), **base)


class Plain:
    """The library alone (no oracle): for GPU-vs-GPU bit comparisons."""

    def __init__(self, w, paged, flags=0, K=None, V=None):
        self.w = w
        dev = "cuda"
        if K is None:
            K, V = kv_logical(w, dev)
        self.K, self.V = K, V
        if paged:
            tab = page_table(w)
            self.kc, self.vc = to_paged(K, tab), to_paged(V, tab)
            self.tab = torch.as_tensor(tab, device=dev)
        else:
            self.kc, self.vc, self.tab = K.clone(), V.clone(), None
        self.seq = torch.zeros(w.B, dtype=torch.int32, device=dev)
        self.cfg = mac.make_config(batch=w.B, num_q_heads=w.Hq, num_kv_heads=w.Hkv, ring_size=w.W,
                                   band=w.r, tau=w.tau, rope_theta=w.theta,
                                   layout=mac.MAC_KV_PAGED if paged else mac.MAC_KV_CONTIGUOUS,
                                   kv_dtype=mac.MAC_BF16, max_seq_len=w.n_cap,
                                   flags=flags | mac.MAC_F_RECORD_DEBUG)
        self.layer = mac.MacLayer(self.cfg)
        self.view = mac.make_kv_view(self.kc, self.vc, self.seq, self.tab,
                                     num_pages=self.kc.shape[0] if paged else 0)
        self.out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device=dev)

    def step(self, seq_h, q, override=None):
        self.seq.copy_(torch.as_tensor(np.asarray(seq_h, np.int32)))
        ov = None if override is None else torch.as_tensor(override, device="cuda")
        self.layer.decode_step(self.view, torch.as_tensor(q, device="cuda"), self.out, ov)
        return self.out.clone()


@pytest.mark.parametrize("stale", [False, True])
def test_async_amend_bit_identical_to_sync(stale):
    """Steps issued back to back without synchronisation.  With the
    stale-by-one ring, amend(t-1) may still run during call t's match and
    complete; the bits must still equal those of amend on the decode stream."""
    w = _case(steps=160, W=8, r=64)
    base = mac.MAC_F_STALE_RING if stale else 0
    a = Plain(w, paged=True, flags=base)
    s = Plain(w, paged=True, flags=base | mac.MAC_F_SYNC_AMEND, K=a.K, V=a.V)
    qs = queries(w)
    for t in range(w.steps):
        seq = np.full(w.B, w.C + t + 1)
        oa = a.step(seq, qs[t])
        os_ = s.step(seq, qs[t])
        assert torch.equal(oa, os_), t
    ha = a.layer.stats()["hits"]
    assert ha == s.layer.stats()["hits"] and ha > 0


@pytest.mark.parametrize("stale", [False, True])
def test_async_amend_bit_identical_to_sync_no_host_waits(stale):
    """The same with every step enqueued back to back: inputs staged on the
    device beforehand, each output copied on the device, one synchronisation
    at the end.  The second stream's amend and the next call's match then
    overlap whatever the host does, so the hand-offs between the streams
    alone keep the ring entries whole."""
    w = _case(steps=96, W=8, r=64)
    base = mac.MAC_F_STALE_RING if stale else 0
    forms = [Plain(w, paged=True, flags=base)]
    forms.append(Plain(w, paged=True, flags=base | mac.MAC_F_SYNC_AMEND, K=forms[0].K,
                       V=forms[0].V))
    q_dev = torch.as_tensor(queries(w), device="cuda")
    seq_dev = torch.as_tensor(np.stack([np.full(w.B, w.C + t + 1, np.int32)
                                        for t in range(w.steps)]), device="cuda")
    outs = []
    for f in forms:
        torch.cuda.synchronize()
        got = []
        for t in range(w.steps):
            f.seq.copy_(seq_dev[t])
            f.layer.decode_step(f.view, q_dev[t], f.out)
            got.append(f.out.clone())
        outs.append(torch.stack(got))
    torch.cuda.synchronize()
    for t in range(w.steps):
        assert torch.equal(outs[0][t], outs[1][t]), t
    ha = forms[0].layer.stats()["hits"]
    assert ha == forms[1].layer.stats()["hits"] and ha > 0


def test_paged_bit_identical_to_contiguous():
    w = _case(steps=24)
    pg = Plain(w, paged=True)
    ct = Plain(w, paged=False, K=pg.K, V=pg.V)
    qs = queries(w)
    for t in range(w.steps):
        seq = np.full(w.B, w.C + t + 1)
        assert torch.equal(pg.step(seq, qs[t]), ct.step(seq, qs[t])), t


def test_forced_redecode_at_own_position_is_full_attention():
    from gpu_harness import Lockstep
    w = _case(steps=6)
    ls = Lockstep(w)
    try:
        for t in range(4):
            ls.step(t)
        miss = np.full((w.B, w.Hq), -1, np.int32)
        first = ls.step(4, override=miss)
        # re-decode the same position, forced onto the entry stored just now
        own = np.full((w.B, w.Hq), w.C + 4, np.int32)
        again = ls.step(4, override=own)
        assert again["hit_gpu"].all()
        np.testing.assert_allclose(again["out_gpu"], first["out_gpu"], atol=2e-6, rtol=0)
    finally:
        ls.close()


def test_override_to_absent_position_is_counted_miss():
    from gpu_harness import Lockstep
    w = _case(steps=5)
    ls = Lockstep(w)
    try:
        for t in range(4):
            ls.step(t)
        before = ls.layer.stats()["override_invalid"]
        ov = np.full((w.B, w.Hq), -2, np.int32)
        ov[0, 3] = 5          # nothing stored at position 5
        info = ls.step(4, override=ov)
        assert info["hit_gpu"][0, 3] == 0
        assert info["res"]["override_invalid"] == 1
        assert ls.layer.stats()["override_invalid"] == before + 1
    finally:
        ls.close()


def test_stale_ring_override_of_previous_call_is_counted_miss():
    """With MAC_F_STALE_RING the previous call's entry is hidden from the
    override too; the entry before it is not."""
    from gpu_harness import Lockstep
    w = _case(steps=6)
    ls = Lockstep(w, flags=mac.MAC_F_STALE_RING, oracle_flags=oracle.F_STALE_RING)
    try:
        for t in range(5):
            ls.step(t)
        m = w.C + 5
        ov = np.full((w.B, w.Hq), -2, np.int32)
        ov[0, 3] = m - 1          # inserted by the previous call: hidden
        ov[1, 2] = m - 2
        info = ls.step(5, override=ov)
        assert info["res"]["override_invalid"] == 1
        assert info["hit_gpu"][0, 3] == 0
        assert info["hit_gpu"][1, 2] == 1 and info["p_gpu"][1, 2] == m - 2
        assert ls.layer.stats()["override_invalid"] == 1
    finally:
        ls.close()


def test_reset_then_all_misses_equal_full_attention():
    from gpu_harness import Lockstep
    w = _case(steps=12)
    ls = Lockstep(w)
    try:
        for t in range(6):
            ls.step(t)
        ls.layer.reset()
        ls.orc.reset()
        info = ls.step(6)
        assert not info["hit_gpu"].any()
        for t in range(7, 12):
            ls.step(t)
    finally:
        ls.close()


def test_idle_request_outputs_zero_and_stores_nothing():
    from gpu_harness import Lockstep
    w = _case(steps=10)
    ls = Lockstep(w)
    try:
        for t in range(10):
            seq = np.full(w.B, w.C + t + 1, np.int32)
            if t % 3 == 1:
                seq[1] = 0                  # request 1 idle this step
            info = ls.step(t, seq_lens=seq)
            if t % 3 == 1:
                assert not info["out_gpu"][1].any()
    finally:
        ls.close()


def test_all_requests_idle_then_resume():
    """A step with every request idle has no work at all (no pages for the
    complete grid): outputs are zero, nothing enters the rings, and the next
    steps continue as the oracle does."""
    from gpu_harness import Lockstep
    w = _case(steps=8)
    ls = Lockstep(w)
    try:
        for t in range(8):
            seq = np.full(w.B, w.C + t + 1, np.int32)
            if t in (0, 3):
                seq[:] = 0
            info = ls.step(t, seq_lens=seq)
            if t in (0, 3):
                assert not info["out_gpu"].any() and not info["hit_gpu"].any()
    finally:
        ls.close()


def test_tau_zero_hits_only_exact_repeats():
    """tau = 0: a hit needs distance exactly 0.  Repeating the previous step's
    query hits it (span [m-1-r+1, m]); a fresh query misses.  Distances of
    exactly zero are exact in fp32, so nothing is forced: every decision,
    exact ties included, is the GPU's own."""
    from gpu_harness import Lockstep
    w = _case(steps=10)
    ls = Lockstep(w, tau=0.0, force=False)
    try:
        q = ls.q
        # steps 4 and 5 repeat step 3's query, step 8 repeats step 7's
        src = {4: 3, 5: 3, 8: 7}
        for t in range(10):
            info = ls.step(t, q=q[src.get(t, t)])
            if t in src:
                # distance 0 to the entries holding that query; ties go to the
                # newest, the previous step's (p = m - 1)
                assert info["hit_gpu"].all() and (info["p_gpu"] == w.C + t - 1).all()
            else:
                assert not info["hit_gpu"].any()
    finally:
        ls.close()


@pytest.mark.parametrize("fused", [False, True])
def test_stats_match_oracle_counts(fused):
    """Counters against the oracle's decisions and key counts; amend re-reads
    r keys per active group and step (none when it is fused into the reduce)."""
    from gpu_harness import Lockstep
    w = _case(steps=20)
    ls = Lockstep(w, flags=mac.MAC_F_FUSED_AMEND if fused else 0)
    try:
        hits = toks = 0
        for t in range(20):
            info = ls.step(t)
            hits += int(info["res"]["hit"].sum())
            toks += int(info["res"]["kv_tokens"].sum())
        st = ls.layer.stats()
        assert st["steps"] == 20 and st["decisions"] == 20 * w.B * w.Hq
        assert st["hits"] == hits and st["misses"] == 20 * w.B * w.Hq - hits
        assert st["kv_tokens_critical"] == toks
        assert st["kv_bytes_critical"] == toks * 2 * w.d * 2
        amend_toks = 0 if fused else 20 * w.B * w.Hkv * w.r   # every step has m >= r here
        assert st["kv_tokens_amend"] == amend_toks
        assert st["bad_input"] == 0 and st["aux_bytes"] > 0
        n_cu = torch.cuda.get_device_properties(0).multi_processor_count
        assert st["aux_bytes"] <= mac.mac_aux_bytes(ls.cfg, n_cu)   # the bound the header states
    finally:
        ls.close()


def test_device_bounds_checks_idle_bad_requests():
    """seq_len past the cache capacity, and a page id outside the pool, are
    caught by the kernels' own checks: counted, never dereferenced."""
    w = _case(B=2, steps=2)
    pl = Plain(w, paged=True)
    qs = queries(w)
    out = pl.step(np.full(w.B, w.C + 1), qs[0])
    before = pl.layer.stats()["bad_input"]
    out = pl.step(np.array([w.n_cap + 5, w.C + 2]), qs[1])     # request 0 beyond capacity
    torch.cuda.synchronize()
    assert not out[0].any() and out[1].abs().sum() > 0
    assert pl.layer.stats()["bad_input"] == before + 1
    tab = pl.tab.clone()
    m = w.C + 2
    pl.tab[1, m // 16] = 1 << 28          # page holding the query position: always read
    out = pl.step(np.array([m + 1, m + 1]), qs[1])
    torch.cuda.synchronize()
    assert pl.layer.stats()["bad_input"] > before + 1
    assert torch.isfinite(out).all()
    pl.tab.copy_(tab)


def test_timing_flag_reports_kernel_times():
    w = _case(B=2, steps=3)
    pl = Plain(w, paged=True, flags=mac.MAC_F_TIMING)
    qs = queries(w)
    for t in range(3):
        pl.step(np.full(w.B, w.C + t + 1), qs[t])
    st = pl.layer.stats()
    assert st["last_us_attention"] > 0 and st["last_us_complete"] > 0
    assert st["last_us_amend"] > 0


def test_misaligned_pointers_rejected_on_host():
    """Queries, outputs and cache rows move as 16-byte vectors: a pointer off
    by one float is refused before any launch, and the handle stays usable."""
    w = _case(B=2, steps=2)
    pl = Plain(w, paged=True)
    qs = queries(w)
    q = torch.as_tensor(qs[0], device="cuda")
    qbuf = torch.zeros(q.numel() + 4, dtype=torch.float32, device="cuda")
    qbuf[1:1 + q.numel()].copy_(q.reshape(-1))
    q_bad = qbuf[1:1 + q.numel()].view_as(q)
    pl.seq.fill_(w.C + 1)
    with pytest.raises(mac.MacError) as ei:
        pl.layer.decode_step(pl.view, q_bad, pl.out)
    assert ei.value.status == mac.MAC_EINVAL
    obuf = torch.zeros(pl.out.numel() + 4, dtype=torch.float32, device="cuda")
    with pytest.raises(mac.MacError) as ei:
        pl.layer.decode_step(pl.view, q, obuf[2:2 + pl.out.numel()].view_as(pl.out))
    assert ei.value.status == mac.MAC_EINVAL
    out = pl.step(np.full(w.B, w.C + 1), qs[0])
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and out.abs().sum() > 0
    assert pl.layer.stats()["steps"] == 1


@pytest.mark.parametrize("form", ["async", "fused", "stale", "sync"])
def test_alternating_streams_match_oracle(form):
    """Calls of one handle on two streams, enqueued back to back with no host
    synchronisation: each call must wait for the previous one's work on the
    other stream (its match rewrites the decisions and partials the previous
    reduce reads), in every amend form; all outputs against the oracle."""
    from gpu_harness import Lockstep
    flags, oflags = {"async": (0, 0), "fused": (mac.MAC_F_FUSED_AMEND, 0),
                     "stale": (mac.MAC_F_STALE_RING, oracle.F_STALE_RING),
                     "sync": (mac.MAC_F_SYNC_AMEND, 0)}[form]
    w = _case(B=4, C=3000, steps=24, rho=("const", 0.985 if form == "stale" else 0.965))
    ls = Lockstep(w, flags=flags, oracle_flags=oflags)
    s0, s1 = torch.cuda.Stream(), torch.cuda.Stream()
    try:
        hits = 0
        for t in range(4):                      # warm the ring up, synchronised
            hits += ls.step(t)["hits"]
        hits += ls.run_unsynced(4, w.steps - 4, [s0, s1])
    finally:
        torch.cuda.synchronize()
        ls.close()
    print("  hits", hits, ls.forced_summary(), flush=True)
    assert hits > 0


@pytest.mark.parametrize("B", [2, 16])
def test_overrides_with_long_rings_match_oracle(B):
    """Overrides (forced reuse of a named position, a forced miss, a position
    not in the ring) with a 200-entry ring, through both long-ring match forms:
    the tile kernel (2 x 32 heads) and the one-launch kernel (16 x 32 heads).
    Every decision and output against the oracle given the same overrides."""
    from gpu_harness import Lockstep
    w = _case(B=B, C=400, steps=36, W=200)
    rng = np.random.default_rng(11 + B)
    ls = Lockstep(w)
    try:
        for t in range(w.steps):
            ov = None
            if t >= 12:
                m = w.C + t
                ov = np.full((w.B, w.Hq), -2, np.int32)
                kind = rng.integers(0, 4, size=(w.B, w.Hq))
                back = rng.integers(1, t + 1, size=(w.B, w.Hq))   # steps 0 .. t-1 are stored
                ov[kind == 1] = (m - back)[kind == 1]
                ov[kind == 2] = -1
                ov[kind == 3] = m + 3                              # never stored
            info = ls.step(t, override=ov)
            if ov is not None:
                assert info["res"]["override_invalid"] == int((ov == w.C + t + 3).sum())
    finally:
        ls.close()
