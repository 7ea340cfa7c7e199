"""GPU parity of the variants the pages name, on every path that accepts them.

- beta = 2 sigmoid(b): `kda_allow_negative_eigenvalues` (AliceAI page,
  section 二, where it is false by default);
- the gate without its safe lower bound (Ling-3.0-flash-VL page, section
  "KDA 层的安全门"): gate_lower_bound = -inf.

Covered here: the decode step and the serving decode with either variant and
both; the bf16 row prep of the chunked prefill with beta x2 alone (its
production instantiation); the recurrent form (unclamped gate) with beta x2.
Each case first checks on the oracle that the variant changes the result, so
no case passes vacuously.  Bounds: 1e-5 / 1e-5 all-fp32, 2e-3 RMS / 1e-3
bf16 inputs with fp32 state.
"""
import numpy as np
import pytest
import torch

import oracle
from kda_inputs import BF16, FP32, as_f64, make_problem, make_tokens, workload_decode
from kda_inputs.torch_io import decode_to_device, from_torch_bf16, tokens_to_device
from tests.helpers import max_over_rms, rel_fro
from tests.test_gpu_parity import BOUNDS, assert_parity, kda, run_varlen  # noqa: F401  (fixture)

pytestmark = pytest.mark.gpu

NO_CLAMP = float("-inf")
VARIANTS = {
    "no_clamp": dict(lower_bound=NO_CLAMP, flags=0),
    "beta_x2": dict(lower_bound=-5.0, flags=oracle.FLAG_BETA_X2),
    "both": dict(lower_bound=NO_CLAMP, flags=oracle.FLAG_BETA_X2),
}


def strong_decay(params_holder):
    """Make every head decay fast enough that many log-decays fall below -5
    (A_log = 1.5: -e^1.5 softplus(alpha + dt_bias) reaches -10 and beyond)."""
    params_holder.A_log = np.full_like(params_holder.A_log, 1.5)


def conv_host(cs, io):
    return as_f64(from_torch_bf16(cs), BF16) if io == BF16 else cs.double().cpu().numpy()


@pytest.mark.parametrize("variant", sorted(VARIANTS))
@pytest.mark.parametrize("io,d", [(FP32, 16), (FP32, 128), (BF16, 128), (BF16, 64)])
def test_decode_step_variants(kda, variant, io, d):
    kw = VARIANTS[variant]
    N, H, steps = 6, 4, 8
    dp = workload_decode(N=N, H=H, d=d, steps=steps, io=io, workload_id=4100 + d + (io == FP32))
    strong_decay(dp)
    dev = torch.device("cuda:0")
    cfg, S, cs = decode_to_device(dp, dev, out_dtype=torch.float32, gate_lower_bound=kw["lower_bound"],
                                  flags=kw["flags"])
    params = (dp.w_q, dp.w_k, dp.w_v, dp.A_log, dp.dt_bias)
    S_ref, c_ref = dp.state.astype(np.float64), dp.conv_state
    S_def, c_def = S_ref, c_ref
    bo, bs = BOUNDS[io]
    o_refs, o_defs = [], []
    for step in range(steps):
        toks = dp.tokens(step)
        o = kda.kda_decode_step(cfg, *tokens_to_device(toks, io, dev), S, cs)
        torch.cuda.synchronize()
        o_ref, S_ref, c_ref = oracle.decode_reference(S_ref, c_ref, toks, params, H, d, d, io,
                                                      lower_bound=kw["lower_bound"], flags=kw["flags"])
        # the default method on the same inputs, to show that the variant matters
        o_def, S_def, c_def = oracle.decode_reference(S_def, c_def, toks, params, H, d, d, io)
        o_refs.append(o_ref)
        o_defs.append(o_def)
        assert max_over_rms(o.double().cpu().numpy(), o_ref) <= bo
        assert np.array_equal(conv_host(cs, io), c_ref)
    es = rel_fro(S.double().cpu().numpy(), S_ref)
    assert es <= bs, f"state error {es:.3e}"
    assert max_over_rms(np.stack(o_defs), np.stack(o_refs)) > 10 * bo, "the variant did not change the result"


@pytest.mark.parametrize("variant", sorted(VARIANTS))
@pytest.mark.parametrize("io,d", [(FP32, 32), (BF16, 128)])
def test_decode_multi_variants(kda, variant, io, d):
    kw = VARIANTS[variant]
    N, K, P, H = 5, 3, 8, 4
    pool = workload_decode(N=P, H=H, d=d, steps=1, io=io, workload_id=4200 + d)
    strong_decay(pool)
    dev = torch.device("cuda:0")
    cfg, S, cs = decode_to_device(pool, dev, out_dtype=torch.float32, gate_lower_bound=kw["lower_bound"],
                                  flags=kw["flags"])
    toks = make_tokens(4201 + d, N * K, H, d, d, io)
    q, k, v, alpha, b = tokens_to_device(toks, io, dev)
    params = (pool.w_q, pool.w_k, pool.w_v, pool.A_log, pool.dt_bias)
    slots = [6, -1, 0, 3, 7]
    commit = [3, 0, 1, 2, 0]
    it = lambda x: torch.tensor(x, dtype=torch.int32, device=dev)
    o = kda.kda_decode_multi(cfg, q.view(N, K, -1), k.view(N, K, -1), v.view(N, K, -1), alpha.view(N, K, H, d),
                             b.view(N, K, H), S, cs, slots=it(slots), n_commit=it(commit))
    torch.cuda.synchronize()
    o_ref, S_ref, c_ref = oracle.decode_multi_reference(pool.state, pool.conv_state, np.array(slots), toks, params,
                                                        H, d, d, io, K, n_commit=commit,
                                                        lower_bound=kw["lower_bound"], flags=kw["flags"])
    o_def, _, _ = oracle.decode_multi_reference(pool.state, pool.conv_state, np.array(slots), toks, params,
                                                H, d, d, io, K, n_commit=commit)
    bo, bs = BOUNDS[io]
    active = [n for n in range(N) if slots[n] >= 0]
    og = o.double().cpu().numpy()
    assert max_over_rms(og[active], o_ref[active]) <= bo
    assert max_over_rms(o_def[active], o_ref[active]) > 5 * bo, "the variant did not change the result"
    touched = [slots[n] for n in active if commit[n] > 0]
    assert rel_fro(S.double().cpu().numpy()[touched], S_ref[touched]) <= bs
    untouched = [r for r in range(P) if r not in touched]
    assert np.array_equal(S.cpu().numpy()[untouched], pool.state[untouched])
    assert np.array_equal(conv_host(cs, io), c_ref)


@pytest.mark.parametrize("d", [64, 128])
def test_bf16_chunked_prefill_beta_x2(kda, d):
    """beta x2 alone, bf16, d in {64, 128}: the chunked form through the row
    prep's production instantiation (no other hook)."""
    p = make_problem(4300 + d, [100, 64, 1, 190, 0, 130], 4, d, d, BF16, state_seqs=[0, 2, 3], conv_state=True)
    o, S, cs = run_varlen(kda, p, flags=oracle.FLAG_BETA_X2)
    assert_parity(p, o, S, cs, flags=oracle.FLAG_BETA_X2)
    o_def, _, _, _ = oracle.forward(p)
    o_x2, _, _, _ = oracle.forward(p, flags=oracle.FLAG_BETA_X2)
    assert max_over_rms(o_def, o_x2) > 0.1


@pytest.mark.parametrize("io,d", [(FP32, 32), (BF16, 128)])
def test_recurrent_form_beta_x2(kda, io, d):
    """The gate without clamp (the recurrent form) with beta x2, on strongly
    decaying heads."""
    p = make_problem(4400 + d, [70, 1, 0, 200, 64], 3, d, d, io, state_seqs=[0, 3], conv_state=True)
    strong_decay(p)
    kw = dict(lower_bound=NO_CLAMP)
    o, S, cs = run_varlen(kda, p, gate_lower_bound=NO_CLAMP, flags=oracle.FLAG_BETA_X2)
    assert_parity(p, o, S, cs, flags=oracle.FLAG_BETA_X2, oracle_kw=kw)
    o_clamped, _, _, _ = oracle.forward(p, flags=oracle.FLAG_BETA_X2)
    o_free, _, _, _ = oracle.forward(p, flags=oracle.FLAG_BETA_X2, lower_bound=NO_CLAMP)
    assert max_over_rms(o_clamped, o_free) > (1e-4 if io == FP32 else 1e-5)
