"""Parity at full size: batch 16 x 131072-token context, 32q/8kv, paged bf16 KV
with a permuted page table -- the configuration the benchmark times.

Decisions are checked for every head (the oracle's match is cheap); outputs
are checked on a sample of (request, head) pairs the oracle tracks in full
(each head's state is independent of the others, so the sample is exact).
"""
import numpy as np
import pytest

from workloads import get_config

pytestmark = pytest.mark.gpu


def test_batch16_128k_paged_sampled_heads(gpu_lib):
    from gpu_harness import Lockstep
    w = get_config("b16_128k")
    steps = 24
    track = np.zeros((w.B, w.Hq), np.uint8)
    rng = np.random.default_rng(7)
    for b in rng.choice(w.B, size=4, replace=False):
        g = int(rng.integers(0, w.Hkv))
        track[b, g * w.G:(g + 1) * w.G] = 1        # whole GQA groups
    print("tracked", np.argwhere(track).tolist(), flush=True)
    ls = Lockstep(w, track=track)
    hits = 0
    try:
        for t in range(steps):
            info = ls.step(t)
            hits += info["hits"]
            print("step", t, "hits", info["hits"], "forced", info["forced"], flush=True)
    finally:
        ls.close()
    assert hits > 0
