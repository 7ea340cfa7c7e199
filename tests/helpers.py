"""Small helpers shared by the tests (no method arithmetic here)."""
from __future__ import annotations

import numpy as np

from kda_inputs import FP32, Problem, make_problem


def rand_head(seed, L, dk, dv, gate_scale=0.3, with_state=True):
    """Random post-preprocess inputs for one head: unit keys/queries, negative
    log-decays, beta in (0, 1)."""
    r = np.random.default_rng(seed)
    q = r.standard_normal((L, dk)); q /= np.linalg.norm(q, axis=1, keepdims=True)
    k = r.standard_normal((L, dk)); k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = r.standard_normal((L, dv))
    g = -gate_scale * r.random((L, dk))
    beta = r.random(L)
    S0 = r.standard_normal((dk, dv)) if with_state else None
    return q, k, v, g, beta, S0


def small_problem(seed, seqlens, H=2, dk=8, dv=8, io=FP32, state=True, conv=True):
    N = len(seqlens)
    return make_problem(1000 + seed, seqlens, H, dk, dv, io,
                        state_seqs=list(range(N)) if state else None, state_std=0.5,
                        conv_state=conv)


def rel_fro(a, b):
    return float(np.linalg.norm((a - b).ravel()) / max(np.linalg.norm(np.asarray(b).ravel()), 1e-300))


def max_over_rms(a, ref):
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    return float(np.max(np.abs(np.asarray(a, dtype=np.float64) - ref))) / max(rms, 1e-300)


def slice_head(p: Problem, n: int, h: int) -> Problem:
    """The sub-problem of sequence n, head h as a one-sequence, one-head
    problem (storage slicing only), so the oracle can check sampled outputs of
    large workloads one (sequence, head) at a time."""
    cu = p.cu_seqlens
    t0, t1 = int(cu[n]), int(cu[n + 1])
    dk, dv, H = p.dk, p.dv, p.H
    cs = None
    if p.conv_state is not None:
        c = p.conv_state[n:n + 1]
        cs = np.concatenate([c[:, :, h * dk:(h + 1) * dk], c[:, :, H * dk + h * dk:H * dk + (h + 1) * dk],
                             c[:, :, 2 * H * dk + h * dv:2 * H * dk + (h + 1) * dv]], axis=2)
    S0 = None if p.initial_state is None else p.initial_state[n:n + 1, h:h + 1]
    return Problem([t1 - t0], 1, dk, dv, p.io,
                   np.ascontiguousarray(p.q[t0:t1, h * dk:(h + 1) * dk]),
                   np.ascontiguousarray(p.k[t0:t1, h * dk:(h + 1) * dk]),
                   np.ascontiguousarray(p.v[t0:t1, h * dv:(h + 1) * dv]),
                   np.ascontiguousarray(p.alpha[t0:t1, h:h + 1]), np.ascontiguousarray(p.b[t0:t1, h:h + 1]),
                   p.w_q[h * dk:(h + 1) * dk], p.w_k[h * dk:(h + 1) * dk], p.w_v[h * dv:(h + 1) * dv],
                   p.A_log[h:h + 1], p.dt_bias[h * dk:(h + 1) * dk], S0, cs)


def bf16_half_ulp(x):
    """Half a bf16 ulp at |x| (normal range)."""
    ax = np.maximum(np.abs(x), 1e-30)
    e = np.floor(np.log2(ax))
    return np.ldexp(1.0, (e - 8).astype(np.int64))


def check_bf16_output(o_bf16_f64, o_ref, bound):
    """|o - o_ref| <= bound * RMS(o_ref) + half a bf16 ulp, elementwise: the
    tolerance applied to a bf16 store of an fp32 result within bound."""
    rms = float(np.sqrt(np.mean(o_ref ** 2)))
    lim = bound * rms + bf16_half_ulp(np.abs(o_ref) + bound * rms)
    excess = np.abs(o_bf16_f64 - o_ref) - lim
    return float(np.max(excess)) <= 0.0, float(np.max(np.abs(o_bf16_f64 - o_ref)) / rms)
