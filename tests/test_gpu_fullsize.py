"""Parity at full size, in the configurations the benchmark times:
- batch 16 x 131072-token context, 32q/8kv, paged bf16 KV with a permuted
  page table (with the pages' amend, the fused amend, the stale-by-one ring
  and bf16 ring queries);
- batch 8 x 122880, 32q/4kv (8 query heads per KV head), per-head rho
  0.5..0.99, paged bf16.

Decisions are checked for every head (the oracle's match is cheap); outputs
are checked on a sample of whole GQA groups the oracle tracks in full (each
head's state is independent of the others, so the sample is exact).
"""
import numpy as np
import pytest

from workloads import get_config

pytestmark = pytest.mark.gpu


def _sampled(w, steps, n_groups, seed, **kw):
    from gpu_harness import Lockstep
    track = np.zeros((w.B, w.Hq), np.uint8)
    rng = np.random.default_rng(seed)
    for b in rng.choice(w.B, size=n_groups, replace=False):
        g = int(rng.integers(0, w.Hkv))
        track[b, g * w.G:(g + 1) * w.G] = 1        # whole GQA groups
    print("tracked", np.argwhere(track).tolist(), kw, flush=True)
    ls = Lockstep(w, track=track, **kw)
    hits = 0
    try:
        for t in range(steps):
            info = ls.step(t)
            hits += info["hits"]
            print("step", t, "hits", info["hits"], "forced", info["forced"], flush=True)
    finally:
        ls.close()
    return hits


@pytest.mark.parametrize("form", ["pages", "fused", "stale", "ring_bf16"])
def test_batch16_128k_paged_sampled_heads(gpu_lib, form):
    """The headline workload in the pages' form (async amend) and each option
    the library offers for it, against the oracle with the same option."""
    import kv_reuse_amd as mac
    import oracle
    flags, oflags = {"pages": (0, 0),
                     "fused": (mac.MAC_F_FUSED_AMEND, 0),
                     "stale": (mac.MAC_F_STALE_RING, oracle.F_STALE_RING),
                     "ring_bf16": (mac.MAC_F_RING_BF16, oracle.F_RING_BF16)}[form]
    w = get_config("b16_128k")
    hits = _sampled(w, 24, 4, 7, flags=flags, oracle_flags=oflags)
    assert hits > 0


def test_moe_8x122k_paged_sampled_groups(gpu_lib):
    w = get_config("moe_122k")
    assert _sampled(w, 16, 2, 11) > 0
