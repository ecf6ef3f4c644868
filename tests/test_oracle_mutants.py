"""Planted mistakes: each plausible slip in the oracle must fail at least one pin.

Every mutant is a text substitution in a private copy of ``oracle/gdn_oracle.c``,
compiled on the CPU into a temporary directory; the committed oracle is never
changed.  The pins of ``test_oracle_pins`` then run against the mutant.
"""
import os
import subprocess

import pytest

import oracle
from oracle import build as obuild
from tests import test_oracle_pins as P
from tests import test_oracle_pins_variants as V

MUTANTS = {
    "drop_decay_in_update": ("hs[(size_t)i * dv + j] = at * hs[(size_t)i * dv + j]",
                             "hs[(size_t)i * dv + j] = hs[(size_t)i * dv + j]"),
    "sign_of_correction": ("u[j] = bt * (vt[j] - at * kv[j])", "u[j] = bt * (vt[j] + at * kv[j])"),
    "decay_missing_in_correction": ("u[j] = bt * (vt[j] - at * kv[j])", "u[j] = bt * (vt[j] - kv[j])"),
    "transposed_state_read": ("kv[j] += kt[i] * hs[(size_t)i * dv + j]",
                              "kv[j] += kt[i] * hs[(size_t)j * dv + i]"),
    "query_used_as_key": ("const double *kt = k +", "const double *kt = q +"),
    "output_scale_dropped": ("ot[j] = scale * acc;", "ot[j] = acc;"),
    "gqa_head_map": ("(int)((long long)h * Hk / Hv)", "(int)(h % Hk)"),
    "conv_taps_reversed": ("acc += w[(size_t)c * K + j] * xv", "acc += w[(size_t)c * K + (K - 1 - j)] * xv"),
    "conv_silu_missing": ("yt[c] = silu(acc);", "yt[c] = acc;"),
    "conv_state_not_advanced": ("memcpy(rs, tmp, sizeof(double) * (size_t)R * C);", "(void)tmp;"),
    "l2_eps_outside_sqrt": ("1.0 / sqrt(ss + l2_eps)", "1.0 / (sqrt(ss) + l2_eps)"),
    "rmsnorm_sum_not_mean": ("sqrt(ss / dv + eps)", "sqrt(ss + eps)"),
    "gate_sigmoid_not_silu": (": silu(zrow[j]))", ": sigmoid(zrow[j]))"),
    "sigmoid_gate_is_silu": ("(gate_sigmoid ? sigmoid(zrow[j])", "(gate_sigmoid ? silu(zrow[j])"),
    "binary16_ties_away_from_zero": ("ldexp(nearbyint(ldexp(x, -q)), q)", "ldexp(round(ldexp(x, -q)), q)"),
    "binary16_one_bit_short": ("int q = e - 11;", "int q = e - 10;"),
    "binary16_no_subnormal_floor": ("if (q < -24) q = -24;", "(void)0;"),
    "f16_state_never_rounded": ("if (state_round == 1 ||", "if (state_round == 9 ||"),
    "u_record_holds_kv": ("memcpy(u_out + ((size_t)t * nh + hi) * (size_t)dv, u,",
                          "memcpy(u_out + ((size_t)t * nh + hi) * (size_t)dv, kv,"),
}

BATTERY = [
    lambda: P.test_bruteforce_exact_rational(0),
    P.test_identity_a1_b0,
    P.test_reset_a0,
    P.test_retrieval_b1_unit_k,
    P.test_orthonormal_keys_closed_form,
    P.test_pure_decay_b0,
    P.test_single_token_from_zero,
    P.test_linearity_in_v_and_gqa_sharing,
    lambda: P.test_chunked_form_agrees(7),
    P.test_conv_matches_numpy_convolve_and_torch_conv1d,
    P.test_conv_delta_tap_is_identity_and_split_calls_continue,
    P.test_l2_norm_value,
    P.test_gated_rmsnorm_library_and_closed_form,
    P.test_verify_intermediates_equal_decode_steps_and_commit,
    V.test_round_binary16_matches_numpy_float16,
    V.test_f16_state_is_rounded_where_it_is_stored,
    V.test_f16_every_token_equals_step_by_step_numpy_half,
    V.test_sigmoid_gated_norm_library_and_closed_form,
    V.test_woa_stash_u_equals_exact_rank1_update,
    lambda: V.test_fold_of_stash_equals_recorded_states("f16"),
    V.test_decode_tokens_equals_chunked_form_and_single_decodes,
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    src = open(obuild.SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) >= 1, "mutation site drifted: " + name
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", str(mutated), "-o",
                    str(lib), "-lm"], check=True)
    caught = []
    with oracle.use_library(str(lib)):
        for pin in BATTERY:
            try:
                pin()
            except AssertionError:
                caught.append(pin)
    assert caught, "no pin caught the planted mistake " + name


def test_unmutated_battery_passes():
    for pin in BATTERY:
        pin()
    assert os.path.exists(obuild.LIB)
