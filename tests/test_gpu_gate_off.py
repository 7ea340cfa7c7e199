"""GPU parity of the recurrent-form prefill against the fp64 oracle.

A gate lower bound below the chunked form's floor (-5.4), -inf included,
routes kda_prefill / kda_varlen_prefill to the token-by-token recurrence.
The inputs here make many log decays fall below -5.4 (and some below -30,
where e^g underflows to 0 in fp32), which the chunked form cannot hold; the
oracle is run with the same bound.  Bounds as for the chunked path: 1e-5 for
all-fp32 runs, 2e-3 RMS / 1e-3 state for bf16 inputs.
"""
import numpy as np
import pytest
import torch

import oracle
from kda_inputs import BF16, FP32, as_f64, make_problem
from tests.test_gpu_parity import assert_parity, kda, run_varlen  # noqa: F401  (fixture)

pytestmark = pytest.mark.gpu

NO_CLAMP = float("-inf")


def strong_gates(p, A_logs):
    """Per-head A_log values; returns the fraction of unclamped log decays
    below -5.4 (the inputs must reach past the chunked form's floor)."""
    p.A_log = np.resize(np.asarray(A_logs, dtype=np.float32), p.H)
    a = as_f64(p.alpha, p.io).reshape(-1, p.H, p.dk) + p.dt_bias.reshape(p.H, p.dk)
    g = -np.exp(p.A_log.astype(np.float64))[None, :, None] * np.logaddexp(0.0, a)
    return float(np.mean(g < -5.4)) if g.size else 0.0


@pytest.mark.parametrize("D", [16, 32, 64, 128])
def test_fp32_varlen_ragged_no_clamp(kda, D):
    p = make_problem(900 + D, [1, 2, 70, 64, 0, 129, 3], 3, D, D, FP32, state_seqs=[0, 2, 3, 5],
                     state_std=0.5, conv_state=True)
    assert strong_gates(p, [2.5, 0.0, 1.4]) > 0.05
    o, S, cs = run_varlen(kda, p, gate_lower_bound=NO_CLAMP)
    assert_parity(p, o, S, cs, oracle_kw={"lower_bound": NO_CLAMP})


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("out_bf16", [False, True])
def test_bf16_varlen_ragged_no_clamp(kda, D, out_bf16):
    p = make_problem(920 + D + out_bf16, [5, 200, 1, 64, 65, 2, 300], 4, D, D, BF16, state_seqs=[1, 3, 6],
                     conv_state=True)
    assert strong_gates(p, [3.0, 1.5, -0.5, 2.0]) > 0.1
    out = torch.bfloat16 if out_bf16 else torch.float32
    o, S, cs = run_varlen(kda, p, out_dtype=out, gate_lower_bound=NO_CLAMP)
    assert_parity(p, o, S, cs, oracle_kw={"lower_bound": NO_CLAMP}, out_bf16=out_bf16)


def test_uniform_prefill_no_clamp(kda):
    B, T, H, D = 2, 300, 4, 128
    p = make_problem(940, [T] * B, H, D, D, BF16, state_seqs=[1], conv_state=True)
    assert strong_gates(p, [2.5, 0.5]) > 0.05
    dev = torch.device("cuda:0")
    from kda_inputs.torch_io import problem_to_device
    cfg, t = problem_to_device(p, dev, out_dtype=torch.float32, gate_lower_bound=NO_CLAMP)
    S = torch.full((B, H, D, D), float("nan"), device=dev)
    cs = torch.full((B, 3, p.ctot), float("nan"), device=dev, dtype=torch.bfloat16)
    o, _, _ = kda.kda_prefill(cfg, t["q"].view(B, T, -1), t["k"].view(B, T, -1), t["v"].view(B, T, -1),
                              t["alpha"].view(B, T, H, D), t["b"].view(B, T, H), t["initial_state"],
                              t["conv_state"], final_state=S, conv_state_out=cs)
    torch.cuda.synchronize()
    assert_parity(p, o.view(B * T, H, D), S, cs, oracle_kw={"lower_bound": NO_CLAMP})


def test_finite_bound_below_floor(kda):
    # lower bound -8: clamped gates the chunked form still cannot hold
    p = make_problem(950, [130, 64, 3], 2, 128, 128, BF16, state_seqs=[0], conv_state=True)
    assert strong_gates(p, [3.0, 2.0]) > 0.3
    o, S, cs = run_varlen(kda, p, gate_lower_bound=-8.0)
    assert_parity(p, o, S, cs, oracle_kw={"lower_bound": -8.0})


def test_raw_gate_hooks_no_clamp(kda):
    # g given directly, down to -30 (e^g ~ 1e-13), q, k, v taken as given
    p = make_problem(960, [90, 17], 2, 64, 64, FP32, state_seqs=[0])
    r = np.random.default_rng(3)
    p.alpha = (-r.random(p.alpha.shape) ** 3 * 30).astype(np.float32)
    p.b = r.random(p.b.shape).astype(np.float32)
    flags = oracle.FLAG_SKIP_CONV | oracle.FLAG_RAW_GATE | oracle.FLAG_RAW_BETA
    o, S, _ = run_varlen(kda, p, flags=flags, gate_lower_bound=NO_CLAMP)
    assert_parity(p, o, S, None, flags=flags, oracle_kw={"lower_bound": NO_CLAMP})


def test_long_sequence_no_clamp(kda):
    # hundreds of staged token blocks per workgroup, with mild decays so that
    # the state carries information across the whole sequence
    p = make_problem(970, [6000, 77], 2, 128, 128, BF16, state_seqs=[0, 1], conv_state=True)
    strong_gates(p, [-1.0, 1.8])
    o, S, cs = run_varlen(kda, p, gate_lower_bound=NO_CLAMP)
    assert_parity(p, o, S, cs, oracle_kw={"lower_bound": NO_CLAMP})


def test_recurrent_form_matches_chunked_above_floor(kda):
    """Where both forms apply (every gate >= -5), the recurrent form, reached
    through a bound below the floor on gates that never go below -5, and
    the chunked form must agree with each other as they do with the
    oracle."""
    p = make_problem(980, [150, 64, 9], 4, 128, 128, FP32, state_seqs=[0, 2], conv_state=True)
    p.A_log = np.full_like(p.A_log, -3.0)   # |g| <= e^-3 softplus(.) stays far above -5
    assert strong_gates(p, [-3.0]) == 0.0
    o_c, S_c, _ = run_varlen(kda, p)
    o_r, S_r, _ = run_varlen(kda, p, gate_lower_bound=-100.0)
    assert_parity(p, o_r, S_r, None)
    scale = float(torch.sqrt(torch.mean(o_c.double() ** 2)))
    assert float((o_r - o_c).abs().max()) <= 2e-5 * scale


@pytest.mark.parametrize("lower_bound", [-5.0, NO_CLAMP])
def test_state_and_conv_history_updated_in_place(kda, lower_bound):
    """final_state may alias initial_state and conv_state_out may alias
    conv_state_in (both prefill forms): the call continues in place."""
    from kda_inputs.torch_io import problem_to_device
    p = make_problem(990, [300, 1, 70, 0, 129], 4, 128, 128, BF16, state_seqs=[0, 1, 2, 3, 4], state_std=0.3,
                     conv_state=True)
    strong_gates(p, [2.5, 0.0, 1.4, -1.0])
    dev = torch.device("cuda:0")
    cfg, t = problem_to_device(p, dev, out_dtype=torch.float32, gate_lower_bound=lower_bound)
    S, cs = t["initial_state"], t["conv_state"]
    o, _, _ = kda.kda_varlen_prefill(cfg, t["cu_seqlens"], t["q"], t["k"], t["v"], t["alpha"], t["b"], S, cs,
                                     final_state=S, conv_state_out=cs)
    torch.cuda.synchronize()
    assert_parity(p, o, S, cs, oracle_kw={"lower_bound": lower_bound})
