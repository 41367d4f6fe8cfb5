"""The oracle's pins catch plausible mistakes.

Each case plants one slip in a copy of oracle/mac_oracle.c (an off-by-one
range or band, a sign, a weight, the tie rule, the threshold's square, the
normalisation or width of the near-threshold and near-tie margins), builds
the copy on the CPU and runs the pins that guard that part of the oracle: at
least one of them must fail.  The unmodified source must pass the same pins
(checked once, first), so a failure here means a pin has gone blind.
"""
import os

import pytest

import oracle
from oracle import build as oracle_build

import test_oracle_match_flags as MF
import test_oracle_pins as PN
import test_oracle_policy as PL

SRC = os.path.join(os.path.dirname(oracle.__file__), "mac_oracle.c")


def _segment_model():
    PL.test_policy_matches_segment_model("fp32", 0.5, 4, 3, 0)


def _segment_model_bf16():
    PL.test_policy_matches_segment_model("bf16", 0.45, 4, 5, 0)


def _attend():
    PN.test_attend_matches_scipy_softmax(33, 128)


def _rope():
    PN.test_rope_is_complex_rotation(17)


# name: (text in mac_oracle.c, its mistaken form, pins that must catch it)
MUTANTS = {
    "attend_drops_last_key": ("int64_t n = b - a + 1;", "int64_t n = b - a;", [_attend]),
    "attend_unscaled_logits": ("logit[i] = scale * acc;", "logit[i] = acc;", [_attend]),
    "rope_sign": ("out[i] = a * c - b * s;", "out[i] = a * c + b * s;", [_rope]),
    "merge_exponent_sign": ("double a = x[d + 1] * exp(x[d] - M);",
                            "double a = x[d + 1] * exp(M - x[d]);",
                            [PN.test_merge_split_invariance_every_split]),
    "remove_weighting": ("tmp[j] = (z[d + 1] * z[j] - c * y[j]) / l;",
                         "tmp[j] = (z[j] - c * y[j]) / l;", [PN.test_remove_inverts_merge]),
    "tie_prefers_oldest": ("(D == b1 && ring_pos[j] >= ring_pos[best])",
                           "(D == b1 && ring_pos[j] < ring_pos[best])",
                           [PN.test_nearest_duplicate_prefers_newest, MF.pin_near_tie]),
    "hit_span_one_short": ("int64_t st = slot >= 0 ? (int64_t)p - r + 1 : 0;",
                           "int64_t st = slot >= 0 ? (int64_t)p - r : 0;",
                           [_segment_model, _segment_model_bf16]),
    "amend_band_one_long": ("orc_attend(q, kg, vg, c->kv_fp32, d, m - r + 1, m, c->scale, tmp);",
                            "orc_attend(q, kg, vg, c->kv_fp32, d, m - r, m, c->scale, tmp);",
                            [_segment_model, _segment_model_bf16]),
    "threshold_not_squared": ("if (d1 <= c->tau * c->tau * qn2)", "if (d1 <= c->tau * qn2)",
                              [MF.pin_rel_and_near_tau, MF.pin_random_rings]),
    "rel_unnormalised": ("double rr = qn2 > 0.0 ? sqrt(d1 / qn2)", "double rr = qn2 > 0.0 ? sqrt(d1)",
                         [MF.pin_rel_and_near_tau, MF.pin_random_rings]),
    "rel_squared": ("double rr = qn2 > 0.0 ? sqrt(d1 / qn2)", "double rr = qn2 > 0.0 ? (d1 / qn2)",
                    [MF.pin_rel_and_near_tau, MF.pin_random_rings]),
    "near_tau_on_squares": ("near_tau[bh] = fabs(rr - c->tau) < 1e-4;",
                            "near_tau[bh] = fabs(rr * rr - c->tau * c->tau) < 1e-4;",
                            [MF.pin_rel_and_near_tau]),
    "near_tau_too_wide": ("near_tau[bh] = fabs(rr - c->tau) < 1e-4;",
                          "near_tau[bh] = fabs(rr - c->tau) < 1e-3;", [MF.pin_rel_and_near_tau]),
    "near_tie_absolute": ("near_tie[bh] = (d2 - d1) <= 1e-5 * d1;",
                          "near_tie[bh] = (d2 - d1) <= 1e-5;", [MF.pin_near_tie]),
    "near_tie_too_wide": ("near_tie[bh] = (d2 - d1) <= 1e-5 * d1;",
                          "near_tie[bh] = (d2 - d1) <= 1e-4 * d1;", [MF.pin_near_tie]),
}


@pytest.fixture(scope="module")
def mutant_dir(tmp_path_factory):
    d = tmp_path_factory.mktemp("oracle_mutants")
    yield d
    oracle._use_library(None)


def _build(text, out):
    path = str(out) + ".c"
    with open(path, "w") as f:
        f.write(text)
    oracle_build.build(src=path, out=str(out) + ".so")
    return str(out) + ".so"


def test_unmodified_oracle_passes_every_guarding_pin(mutant_dir):
    lib = _build(open(SRC).read(), mutant_dir / "original")
    oracle._use_library(lib)
    try:
        seen = set()
        for _, _, pins in MUTANTS.values():
            for pin in pins:
                if pin not in seen:
                    seen.add(pin)
                    pin()
    finally:
        oracle._use_library(None)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(mutant_dir, name):
    old, new, pins = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, "the mutated text must occur exactly once: %r" % old
    lib = _build(src.replace(old, new), mutant_dir / name)
    oracle._use_library(lib)
    failed = []
    try:
        for pin in pins:
            try:
                pin()
            except (AssertionError, FloatingPointError, ValueError):
                failed.append(pin.__name__)
    finally:
        oracle._use_library(None)
    assert failed, "no pin caught the planted mistake %s" % name
