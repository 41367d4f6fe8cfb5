"""GPU parity: the HIP decode path through the C ABI against the fp64 oracle.

Decisions (hit/miss and matched position) bit-exact; outputs within max-abs
2e-3 and per-row relative 1e-2 (bf16 or fp32 KV, fp32 accumulation).
"""
import sys

import numpy as np
import pytest

from workloads import get_config, scaled

pytestmark = pytest.mark.gpu


def _run(w, steps, **kw):
    from gpu_harness import Lockstep
    print("case", w.name, "B", w.B, "Hq", w.Hq, "Hkv", w.Hkv, "C", w.C, "steps", steps,
          w.kv, w.layout, kw, flush=True)
    ls = Lockstep(w, **kw)
    hits = 0
    try:
        for t in range(steps):
            info = ls.step(t)
            hits += info["hits"]
    finally:
        ls.close()
    emax = max(e for e, _ in ls.stats)
    rmax = max(r for _, r in ls.stats)
    print("  hits", hits, "of", steps * w.B * w.Hq, ls.forced_summary(),
          "max-abs %.2e row-rel %.2e" % (emax, rmax), flush=True)
    return hits, ls


def test_cpu_sized_workload_all_steps(gpu_lib):
    """1 request, 8q/2kv, fp32 KV, 4096 + 256 steps, rho 0.95, ring 16, r 64."""
    w = get_config("cpu4k")
    hits, _ = _run(w, w.steps)
    assert 0 < hits < w.steps * w.B * w.Hq


def test_llama_shape_32k_contiguous_bf16(gpu_lib):
    w = get_config("llama32k")
    hits, _ = _run(w, 96)
    assert hits > 0.5 * 95 * w.Hq


@pytest.mark.parametrize("C", [3000, 4096])
def test_paged_batch_mixed_rho(gpu_lib, C):
    """The 128K batch workload's recipe at a small context: paged (permuted
    table), per-request rho in [0.8, 0.99], a ragged prefill length."""
    w = scaled(get_config("b16_128k"), B=4, C=C, steps=48)
    _run(w, w.steps)


@pytest.mark.parametrize("r", [64, 256, 1024])
def test_moe_heads_per_head_rho(gpu_lib, r):
    """32q/4kv (8 query heads per KV head), per-head rho 0.5..0.99, r swept."""
    w = scaled(get_config("moe_122k"), B=2, C=2500, steps=40)
    _run(w, w.steps, r=r)


@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (16, 8), (8, 1)])
def test_group_sizes(gpu_lib, Hq, Hkv):
    w = scaled(get_config("b16_128k"), B=2, Hq=Hq, Hkv=Hkv, C=1000, steps=24,
               rho=("const", 0.96))
    _run(w, w.steps)


def test_small_window_and_band(gpu_lib):
    w = scaled(get_config("cpu4k"), C=300, steps=40, W=1, r=1, kv="bf16")
    _run(w, w.steps)


def test_ragged_contexts(gpu_lib):
    """Requests of different lengths in one batch: positions at every offset
    within a page, one request shorter than the band (its stored prefixes are
    EMPTY), rows past each request's position NaN."""
    w = scaled(get_config("b16_128k"), B=6, C=1200, steps=40, rho=("const", 0.96))
    hits, _ = _run(w, w.steps, prefill=[1200, 1199, 1185, 1024, 777, 17])
    assert hits > 0


def test_context_shorter_than_band(gpu_lib):
    """m grows from 3 past r = 64: hits before m = r merge an EMPTY prefix."""
    w = scaled(get_config("b16_128k"), B=2, C=3, steps=100, W=16, r=64, rho=("const", 0.96))
    hits, _ = _run(w, w.steps)
    assert hits > 0


@pytest.mark.parametrize("W", [24, 48])
def test_windows_not_power_of_two(gpu_lib, W):
    w = scaled(get_config("b16_128k"), B=2, C=500, steps=70, W=W, rho=("const", 0.96))
    _run(w, w.steps)


@pytest.mark.parametrize("Hq,Hkv", [(32, 8), (8, 8)])
def test_maximum_group_count(gpu_lib, Hq, Hkv):
    """B * Hkv = 4096 GQA groups, the most a handle takes: the plan of every
    complete block covers all of them."""
    w = scaled(get_config("b16_128k"), B=4096 // Hkv, Hq=Hq, Hkv=Hkv, C=40, steps=6, W=4, r=16,
               rho=("const", 0.96))
    _run(w, w.steps)


@pytest.mark.parametrize("W,steps", [(65, 90), (100, 150), (512, 140), (2048, 140)])
def test_large_windows(gpu_lib, W, steps):
    """Rings longer than one 64-slot tile (the pages' windows reach 2048
    entries, Table 7): a ragged last tile, wrap-around eviction (W = 65, 100)
    and several filled tiles next to empty ones (W = 512, 2048)."""
    w = scaled(get_config("b16_128k"), B=2, C=600, steps=steps, W=W, rho=("const", 0.96))
    hits, _ = _run(w, w.steps)
    assert hits > 0


_WIDE_CASES = {
    # (B, W, steps, ring queries, stale-by-one ring); B x 32 query heads
    "b16_w200": (16, 200, 60, "fp32", False),
    "b16_w1000_bf16": (16, 1000, 24, "bf16", False),
    "b32_w100_wraps": (32, 100, 130, "fp32", False),
    "b32_w300_bf16_stale": (32, 300, 40, "bf16", True),
}


@pytest.mark.parametrize("case", sorted(_WIDE_CASES))
def test_large_windows_many_heads(gpu_lib, case):
    """Rings over one 64-slot tile with enough heads to give every CU two
    blocks (512 and 1024 query heads): one launch per step whose waves (up to
    8 per head) split each ring into 16-slot sub-tiles and meet in LDS; a
    ragged last sub-tile (W = 100, 200, 300, 1000), the ring wrapping (W = 100
    over 130 steps), both ring precisions and the slot the stale-by-one ring
    hides."""
    import kv_reuse_amd as mac
    import oracle
    B, W, steps, ring, stale = _WIDE_CASES[case]
    w = scaled(get_config("b16_128k"), B=B, C=300, steps=steps, W=W,
               rho=("const", 0.985 if stale else 0.96))
    flags = (mac.MAC_F_RING_BF16 if ring == "bf16" else 0) | (mac.MAC_F_STALE_RING if stale else 0)
    oflags = (oracle.F_RING_BF16 if ring == "bf16" else 0) | (oracle.F_STALE_RING if stale else 0)
    hits, _ = _run(w, w.steps, flags=flags, oracle_flags=oflags)
    assert hits > 0


_FUSED_CASES = {
    "cpu4k_fp32": (lambda: scaled(get_config("cpu4k"), steps=120), {}),
    "paged_mixed": (lambda: scaled(get_config("b16_128k"), B=4, C=3000, steps=48), {}),
    "moe_g8": (lambda: scaled(get_config("moe_122k"), B=2, C=2500, steps=40), {"r": 1024}),
    "ragged": (lambda: scaled(get_config("b16_128k"), B=6, C=1200, steps=40, rho=("const", 0.96)),
               {"prefill": [1200, 1199, 1185, 1024, 777, 17]}),
    "shorter_than_band": (lambda: scaled(get_config("b16_128k"), B=2, C=3, steps=100, W=16, r=64,
                                         rho=("const", 0.96)), {}),
    "window_100": (lambda: scaled(get_config("b16_128k"), B=2, C=600, steps=150, W=100,
                                  rho=("const", 0.96)), {}),
    "band_of_one": (lambda: scaled(get_config("cpu4k"), C=300, steps=40, W=1, r=1, kv="bf16"), {}),
}


@pytest.mark.parametrize("case", sorted(_FUSED_CASES))
def test_fused_amend_matches_oracle(gpu_lib, case):
    """MAC_F_FUSED_AMEND: the reduce stores AS_{1:m-r} as the stored prefix
    merged with the part of the span before the band; the oracle amends with
    the log-domain removal.  Same decisions, outputs within tolerance."""
    import kv_reuse_amd as mac
    make, kw = _FUSED_CASES[case]
    w = make()
    _run(w, w.steps, flags=mac.MAC_F_FUSED_AMEND, **kw)


_RING_BF16_CASES = {
    "paged_mixed_w32": (lambda: scaled(get_config("b16_128k"), B=4, C=3000, steps=48), {}),
    "window_100": (lambda: scaled(get_config("b16_128k"), B=2, C=600, steps=150, W=100,
                                  rho=("const", 0.96)), {}),
    "window_2048": (lambda: scaled(get_config("b16_128k"), B=2, C=600, steps=140, W=2048,
                                   rho=("const", 0.96)), {}),
    "window_24_g8": (lambda: scaled(get_config("moe_122k"), B=2, C=2500, steps=40, W=24), {}),
    "cpu4k_fp32_fused": (lambda: scaled(get_config("cpu4k"), steps=120), {"fused": True}),
}


@pytest.mark.parametrize("case", sorted(_RING_BF16_CASES))
def test_ring_bf16_matches_oracle(gpu_lib, case):
    """MAC_F_RING_BF16: ring queries stored as bfloat16, against the oracle
    with the same rounding (F_RING_BF16); decisions bit-exact."""
    import kv_reuse_amd as mac
    import oracle
    make, kw = _RING_BF16_CASES[case]
    w = make()
    flags = mac.MAC_F_RING_BF16 | (mac.MAC_F_FUSED_AMEND if kw.get("fused") else 0)
    _run(w, w.steps, flags=flags, oracle_flags=oracle.F_RING_BF16)


_STALE_CASES = {
    "cpu4k_fp32": (lambda: scaled(get_config("cpu4k"), steps=120, rho=("const", 0.985)), {}),
    "paged_mixed": (lambda: scaled(get_config("b16_128k"), B=4, C=3000, steps=48,
                                   rho=("per_request_uniform", 0.95, 0.995)), {}),
    "moe_g8": (lambda: scaled(get_config("moe_122k"), B=2, C=2500, steps=40), {"r": 64}),
    "ragged": (lambda: scaled(get_config("b16_128k"), B=6, C=1200, steps=40, rho=("const", 0.985)),
               {"prefill": [1200, 1199, 1185, 1024, 777, 17]}),
    "window_100": (lambda: scaled(get_config("b16_128k"), B=2, C=600, steps=150, W=100,
                                  rho=("const", 0.985)), {}),
    "window_2": (lambda: scaled(get_config("b16_128k"), B=2, C=600, steps=30, W=2,
                                rho=("const", 0.985)), {}),
    "window_1": (lambda: scaled(get_config("cpu4k"), C=300, steps=20, W=1, r=1, kv="bf16"), {}),
    "ring_bf16": (lambda: scaled(get_config("b16_128k"), B=2, C=600, steps=60, W=48,
                                 rho=("const", 0.985)), {"bf16": True}),
}


@pytest.mark.parametrize("case", sorted(_STALE_CASES))
def test_stale_ring_matches_oracle(gpu_lib, case):
    """MAC_F_STALE_RING: call t's match skips the slot call t-1 inserts, as
    the oracle with F_STALE_RING; decisions bit-exact (W = 1 never hits).
    The nearest visible entry is two calls back, so the AR(1) queries use
    rho = 0.985 (relative distance ~ sqrt(2 (1 - rho^2)) ~ 0.24 < tau)."""
    import kv_reuse_amd as mac
    import oracle
    make, kw = _STALE_CASES[case]
    w = make()
    bf16 = kw.pop("bf16", False)
    flags = mac.MAC_F_STALE_RING | (mac.MAC_F_RING_BF16 if bf16 else 0)
    oflags = oracle.F_STALE_RING | (oracle.F_RING_BF16 if bf16 else 0)
    hits, _ = _run(w, w.steps, flags=flags, oracle_flags=oflags, **kw)
    if w.W == 1:
        assert hits == 0
    else:
        assert hits > 0


_UNBALANCED_CASES = {
    "cpu4k_fp32": (lambda: scaled(get_config("cpu4k"), steps=60), 0),
    "paged_mixed": (lambda: scaled(get_config("b16_128k"), B=4, C=3000, steps=48), 0),
    "moe_g8": (lambda: scaled(get_config("moe_122k"), B=2, C=2500, steps=40), 0),
    "ragged_fused": (lambda: scaled(get_config("b16_128k"), B=6, C=1200, steps=40,
                                    rho=("const", 0.96)), 1),
    "allhit_short": (lambda: scaled(get_config("b16_128k"), B=3, C=40, steps=30,
                                    rho=("const", 0.99)), 0),
}


@pytest.mark.parametrize("case", sorted(_UNBALANCED_CASES))
def test_unbalanced_plan_matches_oracle(gpu_lib, case):
    """MAC_F_UNBALANCED_PLAN (the baseline of Figure 8 (b)): every group gets
    the same number of waves; spans shorter than that get one wave per page.
    Same decisions, outputs within tolerance."""
    import kv_reuse_amd as mac
    make, fused = _UNBALANCED_CASES[case]
    w = make()
    kw = {"prefill": [1200, 1199, 1185, 1024, 777, 17]} if case.startswith("ragged") else {}
    flags = mac.MAC_F_UNBALANCED_PLAN | (mac.MAC_F_FUSED_AMEND if fused else 0)
    _run(w, w.steps, flags=flags, **kw)


def _bands(Hq, choices):
    return [choices[h % len(choices)] for h in range(Hq)]


_BAND_CASES = {
    # bands differ inside every KV group
    "paged_mixed": (lambda: scaled(get_config("b16_128k"), B=4, C=3000, steps=48),
                    (64, 256, 1024, 16), 0),
    "moe_g8": (lambda: scaled(get_config("moe_122k"), B=2, C=2500, steps=40),
               (64, 256, 1024, 1, 700, 33, 256, 2048), 0),
    "cpu4k_fp32": (lambda: scaled(get_config("cpu4k"), steps=80), (8, 64, 300, 1), 0),
    # short prefill: heads cross m - r_h >= 0 at different steps
    "shorter_than_band": (lambda: scaled(get_config("b16_128k"), B=2, C=3, steps=100, W=16,
                                         rho=("const", 0.96)), (4, 16, 64, 90), 0),
    "stale_ring": (lambda: scaled(get_config("b16_128k"), B=2, C=600, steps=50,
                                  rho=("const", 0.985)), (16, 128, 512, 5), 1),
    # fused amend: one band per KV group
    "fused_per_group": (lambda: scaled(get_config("b16_128k"), B=4, C=3000, steps=48),
                        (64, 64, 64, 64, 256, 256, 256, 256, 1024, 1024, 1024, 1024,
                         16, 16, 16, 16), 2),
}


@pytest.mark.parametrize("case", sorted(_BAND_CASES))
def test_per_head_bands_match_oracle(gpu_lib, case):
    """Per-head band r_h (band_per_head, Figure 3 (b)) against the oracle with
    the same bands: spans, amend bands and fused cuts follow each head's r_h."""
    import kv_reuse_amd as mac
    import oracle
    make, choices, mode = _BAND_CASES[case]
    w = make()
    bands = _bands(w.Hq, choices)
    flags = {0: 0, 1: mac.MAC_F_STALE_RING, 2: mac.MAC_F_FUSED_AMEND}[mode]
    oflags = oracle.F_STALE_RING if mode == 1 else 0
    hits, _ = _run(w, w.steps, flags=flags, oracle_flags=oflags, bands=bands)
    assert hits > 0


def test_disable_reuse_is_full_attention(gpu_lib):
    import kv_reuse_amd as mac
    import oracle
    w = scaled(get_config("b16_128k"), B=2, C=2000, steps=12)
    hits, _ = _run(w, w.steps, flags=mac.MAC_F_DISABLE_REUSE, oracle_flags=oracle.F_DISABLE_REUSE)
    assert hits == 0
