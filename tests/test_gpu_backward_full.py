"""GPU parity of the backward pass at the benchmark's full size and in its
launch configuration: B=4, T=32768, H=32, dk=dv=128, bf16 inputs and dO,
the initial state and conv history of every sequence, a random fp32 gradient
of the final state, the same seeds as the benchmark.  Every gradient of every
(sequence, head) is compared with the fp64 gradient oracle, one sequence at a
time; the parameter gradients (conv taps, dt_bias, A_log) are the oracle's
per-sequence results summed.  Bound as in the reduced-size tests:
|g - g_ref| <= 5e-5 (RMS(g_ref) + |g_ref|) elementwise.
"""
import numpy as np
import pytest
import torch

import oracle
from kda_inputs import BF16
from tests.helpers import max_over_rms

pytestmark = [pytest.mark.gpu, pytest.mark.slow]
H, D, B, T = 32, 128, 4, 32768
EPS = 5e-5
PER_SEQ = ("dq", "dk", "dv", "dalpha", "db")
PARAMS = ("dw_q", "dw_k", "dw_v", "ddt_bias", "dA_log")


@pytest.fixture(scope="module")
def kda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_03_amd as m
    return m


def scaled(got, ref):
    rms = float(np.sqrt(np.mean(ref ** 2)))
    return float(np.max(np.abs(got - ref) / (rms + np.abs(ref))))


def test_backward_32k_every_head(kda):
    from kda_inputs.device_gen import DeviceProblem
    dev = torch.device("cuda:0")
    dp = DeviceProblem(3, [T] * B, H, D, D, BF16, dev, state_seqs=list(range(B)))
    cfg = dp.config(out_dtype=torch.bfloat16)
    tz = dp.tensors
    g = torch.Generator(device=dev)
    g.manual_seed(9_000_001)
    d_o = torch.randn((B * T, H, D), generator=g, device=dev).to(torch.bfloat16)
    dST = torch.randn((B, H, D, D), generator=g, device=dev)
    grads = kda.kda_varlen_backward(cfg, tz["cu_seqlens"], tz["q"], tz["k"], tz["v"], tz["alpha"], tz["b"],
                                    tz["initial_state"], tz["conv_state"], d_o=d_o, d_final_state=dST)
    torch.cuda.synchronize()
    print("[full backward] GPU gradients done", flush=True)
    for name, x in grads.items():
        assert x is not None and torch.isfinite(x).all(), f"{name} missing or not finite"
    cu = dp.cu_seqlens
    param_ref = {}
    for n in range(B):
        t0, t1 = int(cu[n]), int(cu[n + 1])
        sp = dp.seq_problem(n)
        dO_n = d_o[t0:t1].float().double().cpu().numpy()
        ref = oracle.backward(sp, dO_n, dST[n:n + 1].double().cpu().numpy())
        del dO_n
        errs = {}
        for name in PER_SEQ:
            got = grads[name][t0:t1].double().cpu().numpy().reshape(ref[name].shape)
            errs[name] = scaled(got, ref[name])
        for name, sl in (("dS0", slice(n, n + 1)), ("dconv", slice(n, n + 1))):
            got = grads[name][sl].double().cpu().numpy().reshape(ref[name].shape)
            errs[name] = scaled(got, ref[name])
        for name in PARAMS:
            param_ref[name] = param_ref.get(name, 0.0) + ref[name]
        del ref
        print(f"[full backward] seq {n} ({t1 - t0} tokens, all {H} heads): " +
              " ".join(f"{k}={v:.1e}" for k, v in errs.items()), flush=True)
        for name, e in errs.items():
            assert e <= EPS, f"seq {n} {name}: |g - g_ref| / (RMS + |g_ref|) reaches {e:.3e} > {EPS}"
    for name in PARAMS:
        got = grads[name].double().cpu().numpy().reshape(param_ref[name].shape)
        e = scaled(got, param_ref[name])
        print(f"[full backward] {name}: {e:.1e} (max/RMS {max_over_rms(got, param_ref[name]):.1e})", flush=True)
        assert e <= EPS, f"{name}: |g - g_ref| / (RMS + |g_ref|) reaches {e:.3e} > {EPS}"
