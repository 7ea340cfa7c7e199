"""The gradient oracle's pins must catch plausible mistakes.

Each case copies ``oracle/kda_oracle_bwd.c``, plants one mistake (a dropped
term, a wrong sign, a wrong operand or index), builds it with the forward
oracle into a temporary library and runs the gradient pins against it.  At
least one pin must fail for every mutant.  All mutants stay in bounds.  CPU
only.
"""
import os
import subprocess

import numpy as np
import pytest

import oracle
import tests.test_oracle_bwd_pins as pins

HERE = os.path.dirname(oracle.__file__)
SRC = os.path.join(HERE, "kda_oracle_bwd.c")
FWD = os.path.join(HERE, "kda_oracle.c")

MUTANTS = {
    "dg_from_adjoint_before_write": ("s += dSt[(size_t)i * dv + j] * Stil[(size_t)i * dv + j];",
                                     "s += dS[(size_t)i * dv + j] * Stil[(size_t)i * dv + j];"),
    "adjoint_not_decayed": ("dS[(size_t)i * dv + j] = e * dSt[(size_t)i * dv + j];",
                            "dS[(size_t)i * dv + j] = dSt[(size_t)i * dv + j];"),
    "dk_drops_prediction_term": ("dkk[(size_t)t * dk + i] += s;", "dkk[(size_t)t * dk + i] += 0.0 * s;"),
    "dp_sign": ("dp[j] = -beta[t] * dd[j];", "dp[j] = beta[t] * dd[j];"),
    "dbeta_drops_prediction": ("db += dd[j] * (vt[j] - p[j]);", "db += dd[j] * vt[j];"),
    "dq_reads_old_state": ("s += Snew[(size_t)i * dv + j] * dot[j];", "s += Sprev[(size_t)i * dv + j] * dot[j];"),
    "dv_drops_beta": ("dvv[(size_t)t * dv + j] = beta[t] * dd[j];", "dvv[(size_t)t * dv + j] = dd[j];"),
    "adjoint_write_uses_query": ("dSt[(size_t)i * dv + j] = dS[(size_t)i * dv + j] + kt[i] * dp[j];",
                                 "dSt[(size_t)i * dv + j] = dS[(size_t)i * dv + j] + qt[i] * dp[j];"),
    "l2_drops_projection": ("dut[i] = s * (gt[i] / n - ut[i] * dot / (n * n * n));", "dut[i] = s * gt[i] / n;"),
    "l2_scale_on_k": ("const double s = grp == 0 ? scale : 1.0;", "const double s = scale;"),
    "silu_derivative_sigmoid_only": ("const double dy = dut * sg * (1.0 + yy * (1.0 - sg));",
                                     "const double dy = dut * sg;"),
    "conv_taps_reversed": ("dx[(size_t)tt * row + c] += w[(size_t)c * 4 + j] * dy;",
                           "dx[(size_t)tt * row + c] += w[(size_t)c * 4 + (3 - j)] * dy;"),
    "conv_weight_grad_current_token": ("pw[(size_t)i * 4 + j] += dy * xv;",
                                       "pw[(size_t)i * 4 + j] += dy * x[(size_t)t * row + c];"),
    "history_grad_dropped": ("if (dconv_in) dconv_in[(size_t)(3 + tt) * Ctot + ctot_off + c] += w[(size_t)c * 4 + j] * dy;",
                             ""),
    "clamp_passes_gradient": ("if (graw >= lb) {", "if (1) {"),
    "dA_log_dropped": ("dAl += dgi * graw;", "dAl += 0.0 * graw;"),
    "gate_derivative_sign": ("da = -dgi * a * orb_sigmoid(z);", "da = dgi * a * orb_sigmoid(z);"),
    "dt_bias_grad_dropped": ("pdtb[i] += da;", "pdtb[i] += 0.0 * da;"),
    "beta_sigmoid_derivative_dropped": ("dbv = dbeta[t] * sg * (1.0 - sg);", "dbv = dbeta[t];"),
    "beta_x2_ignored": ("if (flags & ORB_FLAG_BETA_X2) dbv *= 2.0;", ""),
    "final_state_grad_ignored": ("if (dST) memcpy(dS, dST, sizeof(double) * SZ); else memset(dS, 0, sizeof(double) * SZ);",
                                 "memset(dS, 0, sizeof(double) * SZ);"),
    "checkpoint_skips_segment": ("memcpy(seg, ckpt + (size_t)sgi * SZ, sizeof(double) * SZ);",
                                 "memcpy(seg, ckpt + (size_t)(sgi > 0 ? sgi - 1 : 0) * SZ, sizeof(double) * SZ);"),
}

CHECKS = [
    lambda: pins.test_gradient_matches_finite_differences(None, "default"),
    lambda: pins.test_gradient_matches_finite_differences(None, "beta_x2"),
    lambda: pins.test_gradient_matches_finite_differences(None, "hooks"),
    lambda: pins.test_gradient_without_clamp_and_with_scale(None),
    lambda: pins.test_beta_zero_closed_form(None),
]


@pytest.fixture
def restore_oracle():
    yield
    oracle._lib = None


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_gradient_pins_catch_mutant(tmp_path, monkeypatch, restore_oracle, name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique"
    mut = tmp_path / "mut_bwd.c"
    mut.write_text(src.replace(old, new))
    lib = tmp_path / "libmut.so"
    subprocess.check_call(["gcc", "-O1", "-fPIC", "-shared", "-std=c11", "-o", str(lib), FWD, str(mut),
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
