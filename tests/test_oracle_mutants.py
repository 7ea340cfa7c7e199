"""The oracle's pins must catch plausible mistakes.

Each case copies ``oracle/kda_oracle.c``, plants one mistake by text
substitution (a dropped term, a wrong sign, a wrong index, a swapped operand),
compiles the copy into a temporary library and runs the pin suite against it.
At least one pin must fail for every mutant.  All mutants stay in bounds.
CPU only.
"""
import os
import subprocess

import numpy as np
import pytest

import oracle
import tests.test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "kda_oracle.c")
BWD = os.path.join(os.path.dirname(oracle.__file__), "kda_oracle_bwd.c")   # linked unchanged

MUTANTS = {
    "decay_by_value_axis": ("S[(size_t)i * dv + j] *= e;", "S[(size_t)i * dv + j] *= exp(gt[j % dk]);"),
    "delta_sign": ("d[j] = beta[t] * (v[j] - p[j]);", "d[j] = beta[t] * (v[j] + p[j]);"),
    "delta_drops_beta": ("d[j] = beta[t] * (v[j] - p[j]);", "d[j] = (v[j] - p[j]);"),
    "read_with_key": ("ot[j] += q[i] * S[(size_t)i * dv + j];", "ot[j] += k[i] * S[(size_t)i * dv + j];"),
    "write_drops_key": ("S[(size_t)i * dv + j] += k[i] * d[j];", "S[(size_t)i * dv + j] += d[j];"),
    "predict_with_query": ("p[j] += k[i] * S[(size_t)i * dv + j];", "p[j] += q[i] * S[(size_t)i * dv + j];"),
    "conv_taps_reversed": ("y += w[(size_t)c * 4 + j] * xv;", "y += w[(size_t)c * 4 + (3 - j)] * xv;"),
    "conv_history_reversed": ("conv_in[(size_t)(3 + tt) * Ctot", "conv_in[(size_t)(-1 - tt) * Ctot"),
    "no_silu": ("val = y * orc_sigmoid(y);", "val = y;"),
    "k_normed_by_q": ("kh[(size_t)t * dk + i] /= nk;", "kh[(size_t)t * dk + i] /= nq;"),
    "eps_outside_sqrt": ("const double nq = sqrt(sq + eps), nk = sqrt(sk + eps);",
                         "const double nq = sqrt(sq) + eps, nk = sqrt(sk) + eps;"),
    "gate_sign": ("gi = -a * orc_softplus(", "gi = a * orc_softplus("),
    "no_clamp": ("if (gi < lb) gi = lb;", ""),
    "softplus_tail": ("log1p(exp(-fabs(x)))", "log1p(exp(-x))"),
    "beta_no_sigmoid": ("(flags & ORC_FLAG_RAW_BETA) ? bb : orc_sigmoid(bb)", "bb"),
    "dt_bias_head0": ("dt_bias[(size_t)h * dk + i]", "dt_bias[i]"),
    "A_log_head0": ("const double a = exp(A_log[h]);", "const double a = exp(A_log[0]);"),
    "scale_on_k": ("for (int i = 0; i < dk; ++i) qh[(size_t)t * dk + i] *= scale;",
                   "for (int i = 0; i < dk; ++i) kh[(size_t)t * dk + i] *= scale;"),
    "conv_out_shift": ("const int tt = L - 3 + m;", "const int tt = L - 4 + m;"),
    "onorm_sum_not_mean": ("const double rms = sqrt(ss / dv + eps);", "const double rms = sqrt(ss + eps);"),
    "onorm_eps_outside": ("const double rms = sqrt(ss / dv + eps);", "const double rms = sqrt(ss / dv) + eps;"),
    "onorm_weight_ch0": ("orow[j] / rms * w[j] * orc_sigmoid(grow[j]);", "orow[j] / rms * w[0] * orc_sigmoid(grow[j]);"),
    "ogate_sign": ("orow[j] / rms * w[j] * orc_sigmoid(grow[j]);", "orow[j] / rms * w[j] * orc_sigmoid(-grow[j]);"),
    "ogate_row0": ("const double *grow = gate + (size_t)r * dv;", "const double *grow = gate;"),
    "ogate_silu": ("orow[j] / rms * w[j] * orc_sigmoid(grow[j]);", "orow[j] / rms * w[j] * grow[j] * orc_sigmoid(grow[j]);"),
    "skip_conv_applies_silu": ("val = x[(size_t)t * row + c];",
                               "val = x[(size_t)t * row + c] * orc_sigmoid(x[(size_t)t * row + c]);"),
    "raw_gate_clamped": ("gi = al;", "gi = al < lb ? lb : al;"),
    "raw_beta_sigmoid": ("(flags & ORC_FLAG_RAW_BETA) ? bb : orc_sigmoid(bb)", "orc_sigmoid(bb)"),
    "state_not_loaded": ("memcpy(S, J->S0 + ((size_t)n * H + h) * dk * dv, sizeof(double) * (size_t)dk * dv);",
                         "memset(S, 0, sizeof(double) * (size_t)dk * dv);"),
}

CHECKS = [
    lambda: pins.test_recurrence_matches_unrolled_products(None, 0, 5, 3),
    lambda: pins.test_recurrence_matches_unrolled_products(None, 1, 4, 6),
    lambda: pins.test_one_token_closed_form(None),
    lambda: pins.test_beta_zero_only_decays(None),
    lambda: pins.test_orthonormal_keys_recall(None),
    lambda: pins.test_repeated_key_last_write_wins(None),
    lambda: pins.test_chunked_form_matches_token_loop(None, 100, 16),
    lambda: pins.test_conv_silu_matches_torch_conv1d(None),
    lambda: pins.test_conv_single_channel_numpy_convolve(None),
    lambda: pins.test_conv_identity_taps_and_history(None),
    lambda: pins.test_l2norm_unit_and_direction(None),
    lambda: pins.test_scale_multiplies_q_only(None),
    lambda: pins.test_gate_special_values(None),
    lambda: pins.test_beta_is_sigmoid(None),
    lambda: pins.test_conv_state_out_short_sequences(None),
    lambda: pins.test_skip_conv_passes_raw_inputs(None),
    lambda: pins.test_raw_gate_is_alpha_unclamped(None),
    lambda: pins.test_raw_beta_is_b(None),
    lambda: pins.test_forward_equals_preprocess_then_recurrence(None),
    lambda: pins.test_output_gate_unit_rms_and_scale_invariance(None),
    lambda: pins.test_output_gate_eps_inside_the_root(None),
    lambda: pins.test_output_gate_logistic_gate_and_channel_weights(None),
    lambda: pins.test_output_gate_rows_are_independent(None),
]


@pytest.fixture
def restore_oracle():
    yield
    oracle._lib = None


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(tmp_path, monkeypatch, restore_oracle, name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique"
    mut = tmp_path / "mut.c"
    mut.write_text(src.replace(old, new))
    lib = tmp_path / "libmut.so"
    subprocess.check_call(["gcc", "-O1", "-fPIC", "-shared", "-std=c11", "-o", str(lib), str(mut), BWD,
                           "-lm", "-lpthread"])
    monkeypatch.setattr(oracle, "build", lambda force=False: str(lib))
    oracle._lib = None
    failed = []
    for i, chk in enumerate(CHECKS):
        try:
            with np.errstate(all="ignore"):
                chk()
        except AssertionError:
            failed.append(i)
    assert failed, f"mutant {name} passed every pin"
