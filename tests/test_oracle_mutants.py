"""The oracle's pins must catch plausible mistakes.

Each case below compiles a copy of ``oracle/oracle.c`` with one deliberate
mistake planted in it (on the CPU, in a temporary directory), points the
oracle module at that copy and runs the pins of ``test_oracle.py`` (forward)
or ``test_oracle_bwd.py`` (backward).  At least
one pin must fail for every mistake; the real oracle is restored afterwards.
"""
import os
import subprocess

import pytest

import oracle
import test_oracle as pins
import test_oracle_bwd as bwd_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (name, text in oracle.c, replacement) -- each a mistake someone could make.
MUTANTS = [
    ("exp sign", "double p = exp(s[j] - m);", "double p = exp(m - s[j]);"),
    ("dropped max shift", "double p = exp(s[j] - m);", "double p = exp(s[j]);"),
    ("dropped scale", "s[j] = scale * dot;", "s[j] = dot;"),
    ("interleaved gqa", "const int64_t hk = hq / group;", "const int64_t hk = hq % Hkv;"),
    ("top-left mask", "int64_t last = i + (Skv - Sq);", "int64_t last = i;"),
    ("mask off by one", "return last + 1;", "return last;"),
    ("lse drops max", "m + log(l);", "log(l);"),
    ("no normalisation", "orow[d] = acc[d] / l;", "orow[d] = acc[d];"),
    ("bhsd q layout", "q + ((b * Sq + i) * Hq + hq) * D;", "q + ((b * Hq + hq) * Sq + i) * D;"),
    ("v uses k", "const double* vrow = v + ", "const double* vrow = k + "),
    ("merge weight sign", "double c = exp(m2[r] - m);", "double c = exp(m - m2[r]);"),
    ("merge drops l2", "l_out[r] = l1[r] * a + l2[r] * c;", "l_out[r] = l1[r] * a;"),
]

PIN_CALLS = [
    lambda: pins.test_single_key_gives_v0(False),
    lambda: pins.test_identical_keys_give_mean_of_visible_v(True),
    lambda: pins.test_causal_row0_and_last_row(),
    lambda: pins.test_bottom_right_offset(),
    lambda: pins.test_scale_zero_gives_uniform_weights(True),
    lambda: pins.test_v_ones_gives_ones_and_weights_sum_to_one(),
    lambda: pins.test_no_visible_key_rows(),
    lambda: pins.test_golden_worked_example(),
    lambda: pins.test_merge_of_partials_equals_one_shot(True),
    lambda: pins.test_merge_identity_commutes_and_associates(),
    lambda: pins.test_gqa_contiguous_grouping(),
    lambda: pins.test_against_softmax_definition(True),
    lambda: pins.test_against_torch_sdpa_float64(2, 9, 31, 4, 2, 64, True, 0.0884),
]


# mistakes in the backward pass, caught by the pins of test_oracle_bwd.py
BWD_MUTANTS = [
    ("bwd drops delta", "double ds = p * (dp - delta[r]);", "double ds = p * dp;"),
    ("bwd delta sign", "double ds = p * (dp - delta[r]);", "double ds = p * (dp + delta[r]);"),
    ("bwd dk without scale", "dkrow[d] += scale * ds * qrow[d];", "dkrow[d] += ds * qrow[d];"),
    ("bwd dv from ds", "dvrow[d] += p * dorow[d];", "dvrow[d] += ds * dorow[d];"),
    ("bwd dq sign", "dqrow[d] += scale * ds * krow[d];", "dqrow[d] -= scale * ds * krow[d];"),
    ("bwd one q-head per group", "for (int64_t hq = hk * group; hq < (hk + 1) * group; ++hq)",
     "for (int64_t hq = hk; hq < hk + 1; ++hq)"),
    ("bwd mask off by one", "if (j >= visible_end(i, Sq, Skv, causal)) continue;",
     "if (j > visible_end(i, Sq, Skv, causal)) continue;"),
    ("bwd delta unnormalised", "dl += dorow[d] * (acc[d] / l);", "dl += dorow[d] * acc[d];"),
    ("bwd dv from q", "dvrow[d] += p * dorow[d];", "dvrow[d] += p * qrow[d];"),
]

BWD_PIN_CALLS = [
    lambda: bwd_pins.test_finite_differences(True, 5, 11, 4, 2),
    lambda: bwd_pins.test_golden_worked_example(),
    lambda: bwd_pins.test_single_key(True),
    lambda: bwd_pins.test_scale_zero(True),
    lambda: bwd_pins.test_invariants(True),
    lambda: bwd_pins.test_against_torch_autograd_float64(2, 9, 31, 4, 2, 64, True, 0.0884),
]


def _caught(tmp_path, old, new, calls):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site {old!r} not found in oracle.c"
    mutated = src.replace(old, new)
    c_path = tmp_path / "mutant.c"
    so_path = tmp_path / "libmutant.so"
    c_path.write_text(mutated)
    subprocess.run(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    "-std=c11", "-o", str(so_path), str(c_path), "-lm"], check=True)
    old_handle = oracle.use_library(str(so_path))
    failures = 0
    try:
        for call in calls:
            try:
                call()
            except (AssertionError, ValueError, FloatingPointError):
                failures += 1
    finally:
        oracle.restore_library(old_handle)
    return failures


@pytest.mark.parametrize("name,old,new", BWD_MUTANTS, ids=[m[0] for m in BWD_MUTANTS])
def test_bwd_pins_catch_mutant(tmp_path, name, old, new):
    assert _caught(tmp_path, old, new, BWD_PIN_CALLS) > 0, f"no pin caught the mutant {name!r}"


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    count = src.count(old)
    assert count >= 1, f"mutation site for {name!r} not found in oracle.c"
    mutated = src.replace(old, new)
    c_path = tmp_path / "mutant.c"
    so_path = tmp_path / "libmutant.so"
    c_path.write_text(mutated)
    subprocess.run(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    "-std=c11", "-o", str(so_path), str(c_path), "-lm"], check=True)
    old_handle = oracle.use_library(str(so_path))
    failures = 0
    try:
        for call in PIN_CALLS:
            try:
                call()
            except (AssertionError, ValueError, FloatingPointError):
                failures += 1
    finally:
        oracle.restore_library(old_handle)
    assert failures > 0, f"no pin caught the mutant {name!r}"
