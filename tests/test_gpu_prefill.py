"""GPU parity of mac_prefill (MAC-Attention over the prompt with an unbounded
window, the pages' Table 8 ablation) through the C ABI.

The oracle takes the prompt as decode calls in order, one per token, with a
ring as long as the prompt: no entry is ever evicted, which is the unbounded
window.  Decisions (matched positions) bit-exact; outputs within max-abs 2e-3
and per-row relative 1e-2.  Near-threshold and near-tie decisions are forced
to the oracle's through the override input, as in the decode tests.
"""
import os

import numpy as np
import pytest
import torch

from gpu_harness import MAX_ABS, ROW_REL, check_forced_share, force_near
from workloads import bf16_bits, get_config, kv_logical, page_table, queries, scaled, to_paged

pytestmark = pytest.mark.gpu


def _prefill_case(w, lens=None, bands=None, flags=0, oflags=0):
    import kv_reuse_amd as mac
    import oracle
    N, B, Hq, d = w.steps, w.B, w.Hq, w.d
    lens = np.full(B, N, np.int32) if lens is None else np.asarray(lens, np.int32)
    print("prefill case", w.name, "B", B, "Hq", Hq, "Hkv", w.Hkv, "N", N, "lens", lens.tolist(),
          w.kv, w.layout, "flags", flags, flush=True)
    K, V = kv_logical(w, "cuda")
    paged = w.layout == "paged"
    if paged:
        tab = page_table(w)
        kc, vc, table = to_paged(K, tab), to_paged(V, tab), torch.as_tensor(tab, device="cuda")
    else:
        kc, vc, table = K, V, None
    q = queries(w, steps=N)                                  # [N][B][Hq][d]
    Kg = [bf16_bits(K[b, g]) for b in range(B) for g in range(w.Hkv)]
    Vg = [bf16_bits(V[b, g]) for b in range(B) for g in range(w.Hkv)]
    orc = oracle.Oracle(B, Hq, w.Hkv, d, N, w.r if bands is None else bands, w.tau, w.theta,
                        kv_fp32=(w.kv == "fp32"), flags=oflags)
    ov = np.full((B, N, Hq), -2, np.int32)
    want_p = np.full((B, N, Hq), -1, np.int32)
    want_o = np.zeros((B, N, Hq, d))
    keys = n_tau = n_tie = 0
    for t in range(N):
        seq = np.where(t < lens, t + 1, 0).astype(np.int32)
        res = orc.step(Kg, Vg, seq, q[t])
        ov[:, t], _, a, b = force_near(res)
        n_tau += a
        n_tie += b
        want_p[:, t] = np.where(res["hit"] != 0, res["p"], -1)
        want_o[:, t] = res["out"]
        keys += int(res["kv_tokens"].sum())
    cfg = mac.make_config(batch=B, num_q_heads=Hq, num_kv_heads=w.Hkv, ring_size=w.W, band=w.r,
                          tau=w.tau, rope_theta=w.theta,
                          layout=mac.MAC_KV_PAGED if paged else mac.MAC_KV_CONTIGUOUS,
                          kv_dtype=mac.MAC_FP32 if w.kv == "fp32" else mac.MAC_BF16,
                          max_seq_len=w.n_cap, flags=flags, band_per_head=bands)
    layer = mac.MacLayer(cfg)
    try:
        seq_d = torch.as_tensor(lens, device="cuda")
        view = mac.make_kv_view(kc, vc, seq_d, table, num_pages=kc.shape[0] if paged else 0)
        qd = torch.as_tensor(np.ascontiguousarray(q.transpose(1, 0, 2, 3)), device="cuda")
        out = torch.full((B, N, Hq, d), float("nan"), device="cuda")
        pout = torch.full((B, N, Hq), -7, dtype=torch.int32, device="cuda")
        layer.prefill(view, N, qd, out, torch.as_tensor(ov, device="cuda"), pout)
        torch.cuda.synchronize()
        st = layer.stats()
    finally:
        layer.close()
    p_g = pout.cpu().numpy()
    o_g = out.cpu().numpy().astype(np.float64)
    assert np.array_equal(p_g, want_p), np.argwhere(p_g != want_p)[:8]
    live = np.arange(N)[None, :] < lens[:, None]              # [B][N]
    assert not o_g[~live].any(), "rows past a prompt must be zero"
    g, o = o_g[live], want_o[live]
    assert np.all(np.isfinite(g))
    err = np.abs(g - o)
    rel = np.linalg.norm(g - o, axis=-1) / np.maximum(np.linalg.norm(o, axis=-1), 1e-30)
    hits = int((want_p >= 0).sum())
    print("  hits", hits, "of", int(lens.sum()) * Hq, "forced", int((ov != -2).sum()),
          "(near tau %d, near tie %d)" % (n_tau, n_tie),
          "max-abs %.2e row-rel %.2e" % (err.max(), rel.max()), flush=True)
    check_forced_share(n_tau + n_tie, int(lens.sum()) * Hq, w.name)
    assert err.max() <= MAX_ABS and rel.max() <= ROW_REL
    assert st["prefill_tokens"] == lens.sum()
    assert st["prefill_decisions"] == lens.sum() * Hq
    assert st["prefill_hits"] == hits
    assert st["prefill_kv_tokens"] == keys
    assert st["prefill_override_invalid"] == 0 and st["bad_input"] == 0
    return hits


def _w(base, **kw):
    return scaled(get_config(base), C=0, **kw)


def test_prefill_paged_mixed_rho(gpu_lib):
    """128K workload's head shape and paged cache, per-request rho 0.95..0.995
    over a 700-token prompt: hits chain back over many tokens, misses too."""
    w = _w("b16_128k", B=2, steps=700, rho=("per_request_uniform", 0.95, 0.995))
    hits = _prefill_case(w)
    assert 0 < hits < 2 * 700 * 32


def test_prefill_moe_heads(gpu_lib):
    """32q/4kv (8 query heads per KV head), per-head rho 0.5..0.99, r = 64."""
    w = _w("moe_122k", B=1, steps=600, r=64)
    assert _prefill_case(w) > 0


def test_prefill_fp32_contiguous(gpu_lib):
    w = _w("cpu4k", steps=500, r=64, rho=("const", 0.97))
    assert _prefill_case(w) > 0


def test_prefill_ragged_prompts(gpu_lib):
    """Prompts of 300, 151 and 1 tokens in one call of 300 rows."""
    w = _w("b16_128k", B=3, steps=300, rho=("const", 0.98))
    assert _prefill_case(w, lens=[300, 151, 1]) > 0


def test_prefill_per_head_bands(gpu_lib):
    w = _w("b16_128k", B=1, steps=400, rho=("const", 0.98))
    bands = [(16, 64, 256, 3)[h % 4] for h in range(w.Hq)]
    assert _prefill_case(w, bands=bands) > 0


def test_prefill_ring_bf16(gpu_lib):
    import kv_reuse_amd as mac
    import oracle
    w = _w("b16_128k", B=1, steps=400, rho=("const", 0.98))
    assert _prefill_case(w, flags=mac.MAC_F_RING_BF16, oflags=oracle.F_RING_BF16) > 0


def test_prefill_disable_reuse_is_causal_attention(gpu_lib):
    import kv_reuse_amd as mac
    import oracle
    w = _w("b16_128k", B=1, steps=300, rho=("const", 0.98))
    assert _prefill_case(w, flags=mac.MAC_F_DISABLE_REUSE, oflags=oracle.F_DISABLE_REUSE) == 0


@pytest.mark.parametrize("n", [1, 64, 65])
def test_prefill_tile_edges(gpu_lib, n):
    """One token (no earlier query: a miss), and prompts ending on and just past
    the match kernel's 64-token tiles."""
    w = _w("b16_128k", B=1, steps=n, rho=("const", 0.98))
    _prefill_case(w)


def _small_layer(w, flags=0):
    import kv_reuse_amd as mac
    K, V = kv_logical(w, "cuda")
    tab = page_table(w)
    kc, vc, table = to_paged(K, tab), to_paged(V, tab), torch.as_tensor(tab, device="cuda")
    cfg = mac.make_config(batch=w.B, num_q_heads=w.Hq, num_kv_heads=w.Hkv, ring_size=w.W,
                          band=w.r, tau=w.tau, rope_theta=w.theta, layout=mac.MAC_KV_PAGED,
                          kv_dtype=mac.MAC_BF16, max_seq_len=w.n_cap, flags=flags)
    return mac.MacLayer(cfg), kc, vc, table


def test_prefill_bad_lengths_and_overrides_are_counted(gpu_lib):
    """A prompt length beyond the rows given idles its request (zero output,
    counted in bad_input); an override naming the token itself or a later one
    is a counted miss; the other requests are unaffected."""
    import kv_reuse_amd as mac
    w = _w("b16_128k", B=2, steps=80, rho=("const", 0.98))
    N = 64
    layer, kc, vc, table = _small_layer(w)
    try:
        seq = torch.tensor([N + 5, N], dtype=torch.int32, device="cuda")   # request 0: too long
        view = mac.make_kv_view(kc, vc, seq, table, num_pages=kc.shape[0])
        q = queries(w, steps=N)
        qd = torch.as_tensor(np.ascontiguousarray(q.transpose(1, 0, 2, 3)), device="cuda")
        out = torch.full((w.B, N, w.Hq, w.d), float("nan"), device="cuda")
        ov = torch.full((w.B, N, w.Hq), -2, dtype=torch.int32, device="cuda")
        ov[1, 10, 3] = 10          # the token itself: no earlier entry
        ov[1, 11, 4] = 40          # a later token
        ov[1, 12, 5] = 3           # a valid earlier token: forced hit
        pout = torch.full((w.B, N, w.Hq), -7, dtype=torch.int32, device="cuda")
        layer.prefill(view, N, qd, out, ov, pout)
        torch.cuda.synchronize()
        st = layer.stats()
        assert st["bad_input"] == 1 and st["prefill_tokens"] == N
        assert st["prefill_override_invalid"] == 2
        assert not out[0].any() and (pout[0] == -1).all()
        assert torch.isfinite(out[1]).all()
        assert pout[1, 10, 3] == -1 and pout[1, 11, 4] == -1 and pout[1, 12, 5] == 3
    finally:
        layer.close()


def test_prefill_host_checks(gpu_lib):
    import kv_reuse_amd as mac
    w = _w("b16_128k", B=1, steps=16)
    layer, kc, vc, table = _small_layer(w)
    try:
        seq = torch.tensor([16], dtype=torch.int32, device="cuda")
        view = mac.make_kv_view(kc, vc, seq, table, num_pages=kc.shape[0])
        q = torch.zeros((1, 16, w.Hq, w.d), device="cuda")
        out = torch.zeros_like(q)
        for n in (0, 32769):
            with pytest.raises(mac.MacError) as ei:
                layer.prefill(view, n, q, out)
            assert ei.value.status == mac.MAC_EINVAL
        qm = torch.zeros(1 * 16 * w.Hq * w.d + 1, device="cuda")[1:]   # 4-byte offset
        with pytest.raises(mac.MacError) as ei:
            layer.prefill(view, 16, qm, out)
        assert ei.value.status == mac.MAC_EINVAL
    finally:
        layer.close()


def _prefill_draw(i, rng):
    gqa = [(8, 8), (8, 4), (16, 4), (8, 2), (32, 8), (8, 1), (32, 4)]
    Hq, Hkv = gqa[rng.integers(len(gqa))]
    B = int(rng.choice([1, 2, 3]))
    N = int(rng.integers(17, 500))
    rho = float(rng.uniform(0.93, 0.995))
    bands = None
    if rng.random() < 0.3:
        bands = [int(x) for x in rng.choice([1, 16, 64, 300], size=Hq)]
    lens = [int(x) for x in rng.integers(1, N + 1, size=B)]
    lens[int(rng.integers(B))] = N          # one prompt fills the call
    return dict(i=i, B=B, Hq=Hq, Hkv=Hkv, N=N, rho=rho, bands=bands, lens=lens,
                r=int(rng.choice([1, 16, 64, 300])),
                tau=round(float(rng.uniform(0.85, 1.4)) * np.sqrt(2 * (1 - rho)), 3),
                kv="fp32" if rng.random() < 0.3 else "bf16",
                layout="paged" if rng.random() < 0.6 else "contiguous",
                ring_bf16=bool(rng.random() < 0.35))


# a longer or different draw on demand: MAC_PREFILL_SWEEP_CASES=60 MAC_PREFILL_SWEEP_SEED=7
_PF_N = int(os.environ.get("MAC_PREFILL_SWEEP_CASES", "8"))
_PF_SEED = int(os.environ.get("MAC_PREFILL_SWEEP_SEED", "4242"))
_PF_SWEEP = [_prefill_draw(i, rng) for rng in [np.random.default_rng(_PF_SEED)] for i in range(_PF_N)]
_PF_IDS = ["p%d-B%d-%dq%dkv-N%d" % (c["i"], c["B"], c["Hq"], c["Hkv"], c["N"]) for c in _PF_SWEEP]


@pytest.mark.parametrize("c", _PF_SWEEP, ids=_PF_IDS)
def test_prefill_random_configuration(gpu_lib, c):
    """Seeded random prefill cases: shape, ragged prompt lengths (every chunk
    and tile boundary of the match), band or per-head bands, rho with a tau
    near the nearest earlier query's distance, KV dtype and layout, fp32 or
    bf16 candidate queries."""
    import kv_reuse_amd as mac
    import oracle
    w = _w("b16_128k", name="pfsweep%d" % c["i"], B=c["B"], Hq=c["Hq"], Hkv=c["Hkv"],
           steps=c["N"], r=c["r"], tau=c["tau"], rho=("const", c["rho"]), kv=c["kv"],
           layout=c["layout"], seed=200 + c["i"])
    flags = mac.MAC_F_RING_BF16 if c["ring_bf16"] else 0
    oflags = oracle.F_RING_BF16 if c["ring_bf16"] else 0
    print("tau", c["tau"], "rho %.4f" % c["rho"], "bands", c["bands"], "ring_bf16", c["ring_bf16"],
          flush=True)
    _prefill_case(w, lens=c["lens"], bands=c["bands"], flags=flags, oflags=oflags)
