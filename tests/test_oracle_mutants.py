"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that
the pins catch every one of them."""
import os
import shutil
import subprocess

import pytest

import oracle
from tests import test_oracle as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    # forward
    "dropped_scale": ("s[j] = scale * acc;", "s[j] = acc;"),
    "causal_excludes_diagonal": ("long n = i + Lk - Lq + 1;", "long n = i + Lk - Lq;"),
    "causal_sees_one_future_key": ("long n = i + Lk - Lq + 1;", "long n = i + Lk - Lq + 2;"),
    "causal_top_left_aligned": ("long n = i + Lk - Lq + 1;", "long n = i + 1;"),
    "padding_rows_not_masked": ("if (i >= Lq) return 0; /* padding row */", "/* padding rows not masked */"),
    "key_lengths_ignored": ("long Lq = lq ? lq[b] : Nq, Lk = lk ? lk[b] : Nk;", "long Lq = lq ? lq[b] : Nq, Lk = Nk;"),
    "no_max_subtraction": ("s[j] = exp(s[j] - m); /* unnormalised weight */", "s[j] = exp(s[j]); /* unnormalised weight */"),
    "lse_without_max": ("*lse = m + log(l);", "*lse = log(l);"),
    "value_transposed": ("o[c] += p * V[j * d + c];", "o[c] += p * V[c * d + j % d];"),
    # backward
    "softmax_grad_sign": ("dSi[j] = Pi[j] * (dSi[j] - D);", "dSi[j] = Pi[j] * (dSi[j] + D);"),
    "dk_uses_k": ("acc += J->dS[i * Nk + j] * J->q[i * d + c];", "acc += J->dS[i * Nk + j] * J->k[i * d + c];"),
    "dq_missing_scale": ("J->dq[i * d + c] = J->scale * acc;", "J->dq[i * d + c] = acc;"),
    "dv_uses_transposed_p": ("double w = J->P[i * Nk + j];", "double w = J->P[j * Nk + i];"),
    # dropout
    "dropout_scale_missing": ("return byte >= dr->p8 ? 256.0 / (256.0 - (double)dr->p8) : 0.0;",
                              "return byte >= dr->p8 ? 1.0 : 0.0;"),
    "dropout_dv_unmasked": ("if (J->Z) w *= J->Z[i * Nk + j];", "/* dV without the mask */"),
    "dropout_dp_unmasked": ("if (J->Z) acc *= J->Z[i * Nk + j];", "/* dP without the mask */"),
    "philox_key_not_advanced": ("k[0] += 0x9E3779B9u;", "k[0] += 0u;"),
}

PINS = [
    lambda: pins.test_golden_forward_noncausal(),
    lambda: pins.test_golden_forward_causal(),
    lambda: pins.test_golden_backward_noncausal(),
    lambda: pins.test_identical_keys_give_mean_of_values(True),
    lambda: pins.test_causal_row0_is_v0(),
    lambda: pins.test_probability_rows_sum_to_one(True),
    lambda: pins.test_lse_and_output_match_50_digit_brute_force(5, True, 12.0, 0.5),
    lambda: pins.test_lse_and_output_match_50_digit_brute_force(5, True, 1.0, -0.8),
    lambda: pins.test_zero_scale_gives_mean_of_visible_values(True),
    lambda: pins.test_negative_scale_equals_negated_keys(True),
    lambda: pins.test_huge_scores_stay_finite(),
    lambda: pins.test_backward_central_differences(True, 5, 4),
    lambda: pins.test_backward_invariants(True),
    lambda: pins.test_padded_matches_torch_masked_reference(0, True),
    lambda: pins.test_padded_matches_torch_masked_reference(1, False),
    lambda: pins.test_bottom_right_causal_closed_forms(),
    lambda: pins.test_philox_known_answers(),
    lambda: pins.test_dropout_matches_torch_masked_reference(True),
    lambda: pins.test_dropout_is_unbiased(),
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path, monkeypatch):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mutant = tmp_path / "oracle_mutant.c"
    mutant.write_text(src.replace(old, new))
    lib = tmp_path / "liboracle_mutant.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", str(mutant), "-o", str(lib), "-lm"])
    saved_lib, saved_path = oracle._lib, oracle._LIB
    monkeypatch.setattr(oracle, "_lib", None)
    monkeypatch.setattr(oracle, "_LIB", str(lib))
    monkeypatch.setattr(oracle, "build", lambda force=False: str(lib))
    caught = []
    for pin in PINS:
        try:
            pin()
        except (AssertionError, RuntimeError, FloatingPointError, ValueError, OverflowError):
            caught.append(pin)
    assert caught, f"no pin caught mutant {name}"
