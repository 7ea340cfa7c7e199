"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (bf16 outputs), against the fp64 oracle.

The 4K prefill is checked everywhere; the larger workloads on sampled
(sequence, head) pairs that the oracle computes one at a time from the exact
stored input bytes, plus whole-output properties (finite everywhere, exact
conv history).  Bounds: bf16 inputs / fp32 state, max|o - o_ref| <= 2e-3
RMS(o_ref) (+ half a bf16 ulp for the bf16 store) and relative Frobenius
state error <= 1e-3.
"""
import numpy as np
import pytest
import torch

import oracle
from kda_inputs import BF16, VARLEN_LENGTHS, as_f64, workload_decode, workload_prefill_4k
from kda_inputs.torch_io import decode_to_device, from_torch_bf16, problem_to_device, tokens_to_device
from tests.helpers import check_bf16_output, max_over_rms, rel_fro

pytestmark = [pytest.mark.gpu, pytest.mark.slow]
H, D = 32, 128


@pytest.fixture(scope="module")
def kda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_03_amd as m
    return m


def _bf16_check(o_gpu, o_ref, what):
    ok, e = check_bf16_output(o_gpu, o_ref, 2e-3)
    print(f"{what}: max|o - o_ref| = {e:.3e} x RMS (bf16 store)")
    assert ok, f"{what}: bf16 output beyond 2e-3 RMS + half ulp ({e:.3e} x RMS)"


@pytest.mark.parametrize("out", ["fp32", "bf16"])
def test_prefill_4k_every_head(kda, out):
    p = workload_prefill_4k()
    dev = torch.device("cuda:0")
    cfg, t = problem_to_device(p, dev, out_dtype=torch.float32 if out == "fp32" else torch.bfloat16)
    S = torch.empty((1, H, D, D), device=dev)
    cs = torch.empty((1, 3, p.ctot), dtype=torch.bfloat16, device=dev)
    sh = lambda x: x.view(1, 4096, *x.shape[1:])
    o, _, _ = kda.kda_prefill(cfg, sh(t["q"]), sh(t["k"]), sh(t["v"]), sh(t["alpha"]), sh(t["b"]),
                              final_state=S, conv_state_out=cs)
    torch.cuda.synchronize()
    o_ref, S_ref, c_ref, _ = oracle.forward(p)
    og = o[0].double().cpu().numpy()
    if out == "fp32":
        e = max_over_rms(og, o_ref)
        print(f"4K prefill fp32 o: {e:.3e} x RMS")
        assert e <= 2e-3
    else:
        _bf16_check(og, o_ref, "4K prefill")
    es = rel_fro(S.double().cpu().numpy(), S_ref)
    print(f"4K prefill state: {es:.3e}")
    assert es <= 1e-3
    assert np.array_equal(as_f64(from_torch_bf16(cs), BF16), c_ref)


def _sampled_check(dp, o, S_out, items, label, **oracle_kw):
    o_all, ref_all = [], []
    cu = dp.cu_seqlens
    for n, h in items:
        hp = dp.head_problem(n, h)
        o_ref, S_ref, _, _ = oracle.forward(hp, with_conv_out=False, **oracle_kw)
        og = o[cu[n]:cu[n + 1], h].double().cpu().numpy()
        o_all.append(og)
        ref_all.append(o_ref[:, 0])
        es = rel_fro(S_out[n, h].double().cpu().numpy(), S_ref[0, 0])
        print(f"{label} seq {n} head {h} ({hp.seqlens[0]} tokens): state {es:.3e}")
        assert es <= 1e-3
    _bf16_check(np.concatenate(o_all), np.concatenate(ref_all), label)


def test_prefill_32k_sampled(kda):
    from kda_inputs.device_gen import DeviceProblem
    dev = torch.device("cuda:0")
    B, T = 4, 32768
    dp = DeviceProblem(3, [T] * B, H, D, D, BF16, dev, state_seqs=list(range(B)))
    cfg = dp.config(out_dtype=torch.bfloat16)
    tz = dp.tensors
    o = torch.empty((B, T, H, D), dtype=torch.bfloat16, device=dev)
    S = torch.empty((B, H, D, D), device=dev)
    cs = torch.empty((B, 3, dp.ctot), dtype=torch.bfloat16, device=dev)
    kda.kda_prefill(cfg, tz["q"].view(B, T, -1), tz["k"].view(B, T, -1), tz["v"].view(B, T, -1),
                    tz["alpha"].view(B, T, H, D), tz["b"].view(B, T, H), tz["initial_state"], tz["conv_state"],
                    o=o, final_state=S, conv_state_out=cs)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()
    _sampled_check(dp, o.view(B * T, H, D), S, [(0, 0), (1, 13), (2, 22), (3, 31)], "32K prefill")
    # conv history: the last three raw inputs of every sequence, exactly
    for n in range(B):
        last = torch.cat([tz["q"][(n + 1) * T - 3:(n + 1) * T], tz["k"][(n + 1) * T - 3:(n + 1) * T],
                          tz["v"][(n + 1) * T - 3:(n + 1) * T]], dim=1)
        assert torch.equal(cs[n], last)


def test_prefill_32k_no_clamp_sampled(kda):
    """The 32K prefill with the gate's clamp off (lower bound -inf), in the
    launch configuration the benchmark times: the recurrent form."""
    from kda_inputs.device_gen import DeviceProblem
    dev = torch.device("cuda:0")
    B, T = 4, 32768
    dp = DeviceProblem(3, [T] * B, H, D, D, BF16, dev, state_seqs=list(range(B)))
    cfg = dp.config(out_dtype=torch.bfloat16, gate_lower_bound=float("-inf"))
    tz = dp.tensors
    o = torch.empty((B, T, H, D), dtype=torch.bfloat16, device=dev)
    S = torch.empty((B, H, D, D), device=dev)
    kda.kda_prefill(cfg, tz["q"].view(B, T, -1), tz["k"].view(B, T, -1), tz["v"].view(B, T, -1),
                    tz["alpha"].view(B, T, H, D), tz["b"].view(B, T, H), tz["initial_state"], tz["conv_state"],
                    o=o, final_state=S)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()
    _sampled_check(dp, o.view(B * T, H, D), S, [(0, 3), (1, 17), (2, 30), (3, 8)], "32K prefill without clamp",
                   lower_bound=float("-inf"))


def test_varlen_262k_sampled(kda):
    from kda_inputs.device_gen import DeviceProblem
    dev = torch.device("cuda:0")
    dp = DeviceProblem(5, VARLEN_LENGTHS, H, D, D, BF16, dev, state_seqs=[1, 3, 5, 7])
    cfg = dp.config(out_dtype=torch.bfloat16)
    tz = dp.tensors
    N = len(VARLEN_LENGTHS)
    o = torch.empty((sum(VARLEN_LENGTHS), H, D), dtype=torch.bfloat16, device=dev)
    S = torch.empty((N, H, D, D), device=dev)
    kda.kda_varlen_prefill(cfg, tz["cu_seqlens"], tz["q"], tz["k"], tz["v"], tz["alpha"], tz["b"],
                           tz["initial_state"], None, o=o, final_state=S)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()
    _sampled_check(dp, o, S, [(0, 3), (1, 10), (4, 17), (7, 31)], "varlen")


def test_decode_256x128_sampled(kda):
    dp = workload_decode()                      # N=256, H=32, d=128, 128 steps
    dev = torch.device("cuda:0")
    cfg, S, cs = decode_to_device(dp, dev, out_dtype=torch.bfloat16)
    items = [(0, 0), (17, 5), (128, 16), (200, 27), (255, 31)]
    # fp64 reference state of the sampled (sequence, head) pairs
    Sref = {it: dp.state[it[0], it[1]].astype(np.float64) for it in items}
    cref = {it: dp.conv_state[it[0]] for it in items}
    params = (dp.w_q, dp.w_k, dp.w_v, dp.A_log, dp.dt_bias)
    o_all, ref_all = [], []
    for step in range(dp.steps):
        toks = dp.tokens(step)
        o = kda.kda_decode_step(cfg, *tokens_to_device(toks, dp.io, dev), S, cs)
        og = o.double().cpu().numpy()
        for (n, h) in items:
            tok1 = tuple(a[n:n + 1] for a in toks)
            oi, Si, ci = oracle.decode_reference(Sref[(n, h)][None, None].repeat(H, axis=1), cref[(n, h)][None],
                                                 tok1, params, H, D, D, dp.io, items=[h])
            Sref[(n, h)] = Si[0, h]
            # the history shifts by one raw input (q | k | v channels of this token)
            newest = np.concatenate([tok1[0][0], tok1[1][0], tok1[2][0]])[None]
            cref[(n, h)] = np.concatenate([cref[(n, h)][1:], newest], 0)
            o_all.append(og[n, h])
            ref_all.append(oi[0, h])
    torch.cuda.synchronize()
    _bf16_check(np.stack(o_all), np.stack(ref_all), "decode 128 steps")
    for (n, h) in items:
        es = rel_fro(S[n, h].double().cpu().numpy(), Sref[(n, h)])
        print(f"decode seq {n} head {h}: state after 128 steps {es:.3e}")
        assert es <= 1e-3
        assert np.array_equal(from_torch_bf16(cs[n]), cref[(n, h)])
