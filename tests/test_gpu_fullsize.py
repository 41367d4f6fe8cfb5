"""Parity at full size, in the configurations the benchmark times:
- batch 16 x 131072-token context, 32q/8kv, paged bf16 KV with a permuted
  page table: every one of the 128 (request, KV group) units output-checked
  for 8 steps with the pages' amend and with the fused amend; the
  stale-by-one ring and bf16 ring queries on sampled groups;
- batch 8 x 122880, 32q/4kv (8 query heads per KV head), per-head rho
  0.5..0.99, paged bf16, sampled groups;
- batch 16 x 8192, 32q/8kv, and batch 8 x 16384 with one query head per KV
  head (the vector worker): every group at a size where the complete
  kernel's plan weights its shares by dispatch round (the step's pages reach
  16 per wave of the persistent grid), asserted through the grid size the
  library reports.

Decisions are checked for every head (the oracle's match is cheap); where a
sample of whole GQA groups is tracked, each head's state is independent of
the others, so the sample is exact.  Sampled runs always include the first
and the last group of the work list and use a different seed per form.
"""
import numpy as np
import pytest

from workloads import get_config, scaled

pytestmark = pytest.mark.gpu


def _track(w, n_random, seed):
    """Whole GQA groups: the first and last (request, KV head) of the work
    list and n_random others drawn with `seed`."""
    track = np.zeros((w.B, w.Hq), np.uint8)
    groups = {(0, 0), (w.B - 1, w.Hkv - 1)}
    rng = np.random.default_rng(seed)
    while len(groups) < 2 + n_random:
        groups.add((int(rng.integers(0, w.B)), int(rng.integers(0, w.Hkv))))
    for b, g in groups:
        track[b, g * w.G:(g + 1) * w.G] = 1
    return track, sorted(groups)


def _run(w, steps, track=None, **kw):
    from gpu_harness import Lockstep
    print("case", w.name, "B", w.B, "C", w.C, "steps", steps,
          "all groups" if track is None else "groups %s" % (track[1],), kw, flush=True)
    ls = Lockstep(w, track=None if track is None else track[0], **kw)
    hits, pages = 0, []
    try:
        for t in range(steps):
            info = ls.step(t)
            hits += info["hits"]
            pages.append(_step_pages(w, info["res"], ls.prefill + t, kw.get("flags", 0)))
            print("step", t, "hits", info["hits"], "forced tau", info["forced_tau"], "tie",
                  info["forced_tie"], "pages", pages[-1], flush=True)
        st = ls.layer.stats()
    finally:
        ls.close()
    print("  hits", hits, ls.forced_summary(), "complete waves", st["complete_waves"], flush=True)
    return hits, pages, st


def _step_pages(w, res, m, flags):
    """Pages of the step's work list, from the oracle's span starts: each
    group's union span [min start, m], cut at m - r + 1 with fused amend."""
    import kv_reuse_amd as mac
    st = res["start"].reshape(w.B, w.Hkv, w.G).min(axis=2)
    mm = np.asarray(m)[:, None]
    if flags & mac.MAC_F_FUSED_AMEND:
        cut = np.maximum(st, mm - w.r + 1)
        p0 = np.where(cut - 1 >= st, (cut - 1) // 16 - st // 16 + 1, 0)
        p1 = mm // 16 - cut // 16 + 1
        return int(p0.sum() + p1.sum())
    return int((mm // 16 - st // 16 + 1).sum())


@pytest.mark.parametrize("form", ["pages", "fused"])
def test_batch16_128k_paged_every_group(gpu_lib, form):
    """The headline workload, every GQA group output-checked for 8 steps."""
    import kv_reuse_amd as mac
    flags = {"pages": 0, "fused": mac.MAC_F_FUSED_AMEND}[form]
    w = get_config("b16_128k")
    hits, _, _ = _run(w, 8, flags=flags)
    assert hits > 0


@pytest.mark.parametrize("form,seed", [("stale", 21), ("ring_bf16", 22)])
def test_batch16_128k_paged_sampled_groups(gpu_lib, form, seed):
    """The stale-by-one ring and bf16 ring queries at full size, against the
    oracle with the same option, on sampled groups."""
    import kv_reuse_amd as mac
    import oracle
    flags, oflags = {"stale": (mac.MAC_F_STALE_RING, oracle.F_STALE_RING),
                     "ring_bf16": (mac.MAC_F_RING_BF16, oracle.F_RING_BF16)}[form]
    w = get_config("b16_128k")
    hits, _, _ = _run(w, 24, track=_track(w, 4, seed), flags=flags, oracle_flags=oflags)
    assert hits > 0


def test_moe_8x122k_paged_sampled_groups(gpu_lib):
    w = get_config("moe_122k")
    hits, _, _ = _run(w, 16, track=_track(w, 2, 11))
    assert hits > 0


@pytest.mark.parametrize("form", ["pages", "fused"])
def test_dispatch_round_weighted_plan_every_group(gpu_lib, form):
    """16 x 8192: with mostly missing groups the step holds ~57K pages, over 16
    per wave of a grid with three dispatch rounds, so the plan's shares are
    weighted by round (the start and owner of every share computed by the
    weighted split) and every segment is output-checked."""
    import torch
    import kv_reuse_amd as mac
    flags = {"pages": 0, "fused": mac.MAC_F_FUSED_AMEND}[form]
    w = scaled(get_config("b16_128k"), C=8192, steps=16)
    hits, pages, st = _run(w, w.steps, flags=flags)
    waves = st["complete_waves"]
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    assert waves >= 3 * 4 * n_cu, "fewer than three dispatch rounds of 4-wave blocks"
    weighted = sum(p >= 16 * waves for p in pages)
    print("steps with a round-weighted plan:", weighted, "of", len(pages), flush=True)
    assert weighted == len(pages)
    assert hits > 0


def test_g1_vector_worker_weighted_plan_every_group(gpu_lib):
    """One query head per KV head (G = 1; bf16 runs the vector worker there):
    8 x 16384 with 8 heads gives 64 groups of ~1025 pages, over 16 per wave of
    three dispatch rounds, so every step takes the round-weighted split;
    every group is output-checked."""
    import torch
    w = scaled(get_config("b16_128k"), B=8, Hq=8, Hkv=8, C=16384, steps=12)
    hits, pages, st = _run(w, w.steps)
    waves = st["complete_waves"]
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    assert waves >= 3 * 4 * n_cu, "fewer than three dispatch rounds of 4-wave blocks"
    assert all(p >= 16 * waves for p in pages)
    assert hits > 0
