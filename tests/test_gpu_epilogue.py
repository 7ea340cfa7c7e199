"""GPU parity of the output epilogue (o_norm x sigmoid gate) against the oracle.

Stand-alone: the same stored o, gate and weight go to kda_output_gate and to
oracle.output_gate; the only differences are fp32 arithmetic and the final
rounding, so the bound is 1e-5 of RMS(y) (+ half a bf16 ulp for bf16 y).
Composed with a prefill or a decode step, the core's bound on o -- per
element E_k = 2e-3 RMS(o) for bf16 inputs, plus half a bf16 ulp of o_k when o
is stored in bf16 -- is carried through the row normalisation to first order.
With r the row's RMS and s_j the gate's sigmoid, y_j = w_j s_j o_j / r moves
under a perturbation |d_k| <= E_k by at most
  |w_j s_j| (E_j / r + |o_j| sum_k |o_k| E_k / (dv r^3))
(the direct term and the change of r); half a bf16 ulp is added for a bf16 y.
Rows whose RMS is far below the global one get proportionally looser bounds.
"""
import numpy as np
import pytest
import torch

import oracle
from kda_inputs import BF16, FP32, as_f64, make_epilogue_o, make_output_gate_inputs, make_problem
from kda_inputs.torch_io import from_torch_bf16, make_config, to_torch
from tests.helpers import check_bf16_output, max_over_rms
from tests.test_gpu_parity import kda, run_varlen  # noqa: F401  (fixture)

pytestmark = pytest.mark.gpu


def epilogue_cfg(H, d, io, out):
    dev = torch.device("cuda:0")
    import gated_delta_rule_03_amd as m
    # the epilogue reads only the head geometry and the dtypes of the config
    return m.Config(A_log=torch.zeros(H, device=dev), dt_bias=torch.zeros(H * d, device=dev), conv_w_q=None,
                    conv_w_k=None, conv_w_v=None, num_heads=H, head_k_dim=d, head_v_dim=d,
                    io_dtype=torch.bfloat16 if io == BF16 else torch.float32,
                    out_dtype=torch.bfloat16 if out == BF16 else torch.float32)


def y_to_f64(y):
    return as_f64(from_torch_bf16(y), BF16) if y.dtype == torch.bfloat16 else y.double().cpu().numpy()


def check(y, y_ref, bound):
    if y.dtype == torch.bfloat16:
        ok, e = check_bf16_output(y_to_f64(y), y_ref, bound)
        assert ok, f"bf16 y error {e:.3e} x RMS beyond bound + half ulp"
    else:
        e = max_over_rms(y_to_f64(y), y_ref)
        assert e <= bound, f"y error {e:.3e} x RMS > {bound}"


def check_composed(y, o_ref, gate64, w, core_bound, o_bf16):
    from tests.helpers import bf16_half_ulp
    y_ref = oracle.output_gate(o_ref, gate64, w)
    E = np.full_like(o_ref, core_bound * float(np.sqrt(np.mean(o_ref ** 2))))
    if o_bf16:
        E = E + bf16_half_ulp(np.abs(o_ref) + E)
    dv = o_ref.shape[-1]
    r = np.sqrt(np.mean(o_ref ** 2, axis=-1, keepdims=True))
    s = 1.0 / (1.0 + np.exp(-gate64))
    lim = np.abs(w * s) * (E / r + np.abs(o_ref) * np.sum(np.abs(o_ref) * E, axis=-1, keepdims=True) / (dv * r ** 3))
    yg = y_to_f64(y)
    if y.dtype == torch.bfloat16:
        lim = lim + bf16_half_ulp(np.abs(y_ref) + lim)
    excess = np.abs(yg - y_ref) - lim
    assert float(np.max(excess)) <= 0.0, f"y off by {float(np.max(np.abs(yg - y_ref))):.3e} beyond the propagated bound"


@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("io,out", [(BF16, BF16), (BF16, FP32), (FP32, FP32), (FP32, BF16)])
def test_output_gate_matches_oracle(kda, d, io, out):
    # 37 tokens x 3 heads = 111 rows: the last 16-lane groups of a wave idle
    n, H = 37, 3
    dev = torch.device("cuda:0")
    cfg = epilogue_cfg(H, d, io, out)
    o = make_epilogue_o(1000 + d, n, H, d, out)
    gate, w = make_output_gate_inputs(1000 + d, n, H, d, io)
    y = kda.kda_output_gate(cfg, to_torch(o, out, dev), to_torch(gate, io, dev), torch.from_numpy(w).to(dev),
                            eps=1e-6)
    torch.cuda.synchronize()
    y_ref = oracle.output_gate(as_f64(o, out), as_f64(gate, io), w, eps=1e-6)
    check(y, y_ref, 1e-5)


def test_output_gate_in_place_and_eps(kda):
    n, H, d = 300, 4, 128
    dev = torch.device("cuda:0")
    cfg = epilogue_cfg(H, d, BF16, BF16)
    o = make_epilogue_o(1100, n, H, d, BF16)
    gate, w = make_output_gate_inputs(1100, n, H, d, BF16)
    for eps in (0.0, 1e-6, 0.5):
        ot = to_torch(o, BF16, dev)
        y = kda.kda_output_gate(cfg, ot, to_torch(gate, BF16, dev), torch.from_numpy(w).to(dev), eps=eps, y=ot)
        torch.cuda.synchronize()
        assert y.data_ptr() == ot.data_ptr()
        check(y, oracle.output_gate(as_f64(o, BF16), as_f64(gate, BF16), w, eps=eps), 1e-5)


def test_output_gate_full_size_sampled(kda):
    """B=4 x 32768 tokens x 32 heads x 128 (bf16), the shape of the 32K
    prefill's output: every row computed, 4096 sampled rows checked."""
    n, H, d = 4 * 32768, 32, 128
    dev = torch.device("cuda:0")
    cfg = epilogue_cfg(H, d, BF16, BF16)
    o = make_epilogue_o(1200, n, H, d, BF16)
    gate, w = make_output_gate_inputs(1200, n, H, d, BF16)
    y = kda.kda_output_gate(cfg, to_torch(o, BF16, dev), to_torch(gate, BF16, dev), torch.from_numpy(w).to(dev))
    torch.cuda.synchronize()
    rows = np.random.default_rng(5).choice(n * H, size=4096, replace=False)
    y_rows = from_torch_bf16(y).reshape(n * H, d)[rows]
    ref = oracle.output_gate(as_f64(o.reshape(n * H, d)[rows], BF16), as_f64(gate.reshape(n * H, d)[rows], BF16), w)
    ok, e = check_bf16_output(as_f64(y_rows, BF16), ref, 1e-5)
    assert ok, f"bf16 y error {e:.3e}"


def test_output_gate_after_prefill(kda):
    p = make_problem(1300, [200, 1, 64, 130], 4, 128, 128, BF16, state_seqs=[0, 3], conv_state=True)
    dev = torch.device("cuda:0")
    o, _, _ = run_varlen(kda, p, out_dtype=torch.bfloat16)
    gate, w = make_output_gate_inputs(1300, p.total_T, p.H, p.dv, BF16)
    cfg = make_config(p, dev, out_dtype=torch.bfloat16)
    y = kda.kda_output_gate(cfg, o, to_torch(gate, BF16, dev), torch.from_numpy(w).to(dev), y=o)
    torch.cuda.synchronize()
    o_ref, _, _, _ = oracle.forward(p)
    check_composed(y, o_ref, as_f64(gate, BF16), w, 2e-3, o_bf16=True)


def test_output_gate_after_decode(kda):
    from kda_inputs import workload_decode
    from kda_inputs.torch_io import decode_to_device, tokens_to_device
    dp = workload_decode(N=8, H=4, d=128, steps=1, workload_id=1400)
    dev = torch.device("cuda:0")
    cfg, S, cs = decode_to_device(dp, dev, out_dtype=torch.bfloat16)
    toks = dp.tokens(0)
    o = kda.kda_decode_step(cfg, *tokens_to_device(toks, dp.io, dev), S, cs)
    gate, w = make_output_gate_inputs(1400, 8, 4, 128, BF16)
    y = kda.kda_output_gate(cfg, o, to_torch(gate, BF16, dev), torch.from_numpy(w).to(dev))
    torch.cuda.synchronize()
    params = (dp.w_q, dp.w_k, dp.w_v, dp.A_log, dp.dt_bias)
    o_ref, _, _ = oracle.decode_reference(dp.state, dp.conv_state, toks, params, dp.H, dp.dk, dp.dv, dp.io)
    check_composed(y, o_ref, as_f64(gate, BF16), w, 2e-3, o_bf16=True)


def test_output_gate_grid_stride(kda):
    """17.3 M rows of 16 (270000 tokens x 64 heads): more rows than the
    launch's 2^20 workgroups cover at once, so groups stride over rows."""
    n, H, d = 270000, 64, 16
    assert n * H > (1 << 20) * 16
    dev = torch.device("cuda:0")
    cfg = epilogue_cfg(H, d, BF16, BF16)
    o = make_epilogue_o(1250, n, H, d, BF16)
    gate, w = make_output_gate_inputs(1250, n, H, d, BF16)
    y = kda.kda_output_gate(cfg, to_torch(o, BF16, dev), to_torch(gate, BF16, dev), torch.from_numpy(w).to(dev))
    torch.cuda.synchronize()
    rows = np.concatenate([np.random.default_rng(6).choice(n * H, size=4096, replace=False),
                           np.arange(n * H - 64, n * H), np.arange((1 << 20) * 16 - 32, (1 << 20) * 16 + 32)])
    y_rows = from_torch_bf16(y).reshape(n * H, d)[rows]
    ref = oracle.output_gate(as_f64(o.reshape(n * H, d)[rows], BF16), as_f64(gate.reshape(n * H, d)[rows], BF16), w)
    ok, e = check_bf16_output(as_f64(y_rows, BF16), ref, 1e-5)
    assert ok, f"bf16 y error {e:.3e}"


# ---- the epilogue fused into the decode step and the serving decode: o never
# leaves the workgroup; y is checked against the oracle's output epilogue
# applied to the oracle's decode output, at the composed bound above, and the
# state and conv history must equal the plain call's bit for bit.

@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("io,out", [(BF16, BF16), (BF16, FP32), (FP32, FP32)])
def test_decode_step_gated(kda, d, io, out):
    from kda_inputs import workload_decode
    from kda_inputs.torch_io import decode_to_device, tokens_to_device
    N, H, steps = 7, 3, 3
    dp = workload_decode(N=N, H=H, d=d, steps=steps, io=io, workload_id=1500 + d)
    dev = torch.device("cuda:0")
    cfg, S, cs = decode_to_device(dp, dev, out_dtype=torch.bfloat16 if out == BF16 else torch.float32)
    _, S2, cs2 = decode_to_device(dp, dev)
    params = (dp.w_q, dp.w_k, dp.w_v, dp.A_log, dp.dt_bias)
    S_ref, c_ref = dp.state.astype(np.float64), dp.conv_state
    core = 2e-3 if io == BF16 else 1e-5
    for step in range(steps):
        toks = dp.tokens(step)
        gate, w = make_output_gate_inputs(1500 + d, N, H, d, io, step=step)
        dt = tokens_to_device(toks, io, dev)
        y = kda.kda_decode_step_gated(cfg, *dt, S, cs, to_torch(gate, io, dev), torch.from_numpy(w).to(dev),
                                      eps=1e-6)
        kda.kda_decode_step(cfg, *dt, S2, cs2)
        torch.cuda.synchronize()
        o_ref, S_ref, c_ref = oracle.decode_reference(S_ref, c_ref, toks, params, H, d, d, io)
        check_composed(y, o_ref, as_f64(gate, io), w, core, o_bf16=False)
        assert torch.equal(S, S2) and torch.equal(cs, cs2)


@pytest.mark.parametrize("d", [32, 128])
@pytest.mark.parametrize("io", [BF16, FP32])
def test_decode_multi_gated(kda, d, io):
    from kda_inputs import make_tokens, workload_decode
    from kda_inputs.torch_io import decode_to_device, tokens_to_device
    N, K, P, H = 5, 3, 8, 4
    pool = workload_decode(N=P, H=H, d=d, steps=1, io=io, workload_id=1600 + d)
    dev = torch.device("cuda:0")
    cfg, S, cs = decode_to_device(pool, dev, out_dtype=torch.bfloat16)
    _, S2, cs2 = decode_to_device(pool, dev)
    toks = make_tokens(1601 + d, N * K, H, d, d, io)
    q, k, v, alpha, b = tokens_to_device(toks, io, dev)
    dt = (q.view(N, K, -1), k.view(N, K, -1), v.view(N, K, -1), alpha.view(N, K, H, d), b.view(N, K, H))
    gate, w = make_output_gate_inputs(1602 + d, N * K, H, d, io)
    slots, commit = [6, -1, 0, 3, 7], [3, 0, 1, 2, 0]
    it = lambda x: torch.tensor(x, dtype=torch.int32, device=dev)
    y = kda.kda_decode_multi_gated(cfg, *dt, S, cs, to_torch(gate, io, dev).view(N, K, H, d),
                                   torch.from_numpy(w).to(dev), slots=it(slots), n_commit=it(commit))
    kda.kda_decode_multi(cfg, *dt, S2, cs2, slots=it(slots), n_commit=it(commit))
    torch.cuda.synchronize()
    params = (pool.w_q, pool.w_k, pool.w_v, pool.A_log, pool.dt_bias)
    o_ref, _, _ = oracle.decode_multi_reference(pool.state, pool.conv_state, np.array(slots), toks, params,
                                                H, d, d, io, K, n_commit=commit)
    active = [n for n in range(N) if slots[n] >= 0]
    g64 = as_f64(gate, io).reshape(N, K, H, d)
    check_composed(y[active], o_ref[active], g64[active], w, 2e-3 if io == BF16 else 1e-5, o_bf16=False)
    assert torch.equal(S, S2) and torch.equal(cs, cs2)
