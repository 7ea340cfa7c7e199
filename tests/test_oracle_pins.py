"""Pins for the fp64 oracle (CPU only).

Each check ties the oracle to something other than itself: an independent
restatement (product form, chunked form), a closed form, an invariant of the
delta rule, or a library routine for a sub-step.
"""
import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import bruteforce, chunked
from kda_inputs import BF16, FP32, Problem, as_f64
from tests.helpers import max_over_rms, rand_head, rel_fro, small_problem


# ---------------------------------------------------------------- recurrence
@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("dk,dv", [(5, 3), (4, 6)])
def test_recurrence_matches_unrolled_products(oracle_lib, seed, dk, dv):
    q, k, v, g, beta, S0 = rand_head(seed, 12, dk, dv)
    o, S = oracle.recurrence(q, k, v, g, beta, S0)
    o_bf, S_bf = bruteforce.states_and_outputs(q, k, v, g, beta, S0)
    assert np.allclose(o, o_bf, rtol=1e-12, atol=1e-12)
    assert np.allclose(S, S_bf, rtol=1e-12, atol=1e-12)


def test_one_token_closed_form(oracle_lib):
    # S1 = Diag(e^g) S0 + beta k (v - k^T Diag(e^g) S0)^T ; o = q^T S1
    q, k, v, g, beta, S0 = rand_head(7, 1, 6, 4)
    o, S = oracle.recurrence(q, k, v, g, beta, S0)
    Sd = np.exp(g[0])[:, None] * S0
    S1 = Sd + beta[0] * np.outer(k[0], v[0] - k[0] @ Sd)
    assert np.allclose(S, S1, rtol=1e-14, atol=1e-14)
    assert np.allclose(o[0], q[0] @ S1, rtol=1e-14, atol=1e-14)


def test_beta_zero_only_decays(oracle_lib):
    q, k, v, g, beta, S0 = rand_head(3, 20, 6, 5)
    beta[:] = 0.0
    o, S = oracle.recurrence(q, k, v, g, beta, S0)
    Gam = np.cumsum(g, axis=0)
    assert np.allclose(S, np.exp(Gam[-1])[:, None] * S0, rtol=1e-13, atol=0)
    for t in range(20):
        assert np.allclose(o[t], (q[t] * np.exp(Gam[t])) @ S0, rtol=1e-12, atol=1e-15)


def test_orthonormal_keys_recall(oracle_lib):
    # g = 0, beta = 1, orthonormal keys: every stored value is recalled exactly,
    # and a query equal to the current key reads back the current value.
    dk, dv, L = 8, 5, 8
    r = np.random.default_rng(11)
    Qm, _ = np.linalg.qr(r.standard_normal((dk, dk)))
    k = Qm.T[:L]
    v = r.standard_normal((L, dv))
    g = np.zeros((L, dk))
    beta = np.ones(L)
    S0 = r.standard_normal((dk, dv))
    o, S = oracle.recurrence(k, k, v, g, beta, S0)
    for j in range(L):
        assert np.allclose(k[j] @ S, v[j], atol=1e-13)
        assert np.allclose(o[j], v[j], atol=1e-13)


def test_repeated_key_last_write_wins(oracle_lib):
    dk, dv = 6, 3
    r = np.random.default_rng(5)
    key = r.standard_normal(dk); key /= np.linalg.norm(key)
    k = np.stack([key] * 4)
    v = r.standard_normal((4, dv))
    o, S = oracle.recurrence(k, k, v, np.zeros((4, dk)), np.ones(4), np.zeros((dk, dv)))
    assert np.allclose(key @ S, v[-1], atol=1e-14)
    assert np.allclose(o, v, atol=1e-14)


def test_linear_in_state_and_values(oracle_lib):
    q, k, v, g, beta, S0 = rand_head(9, 15, 5, 4)
    _, _, v2, _, _, S02 = rand_head(10, 15, 5, 4)
    a, b = 0.7, -1.3
    o1, S1 = oracle.recurrence(q, k, v, g, beta, S0)
    o2, S2 = oracle.recurrence(q, k, v2, g, beta, S02)
    o3, S3 = oracle.recurrence(q, k, a * v + b * v2, g, beta, a * S0 + b * S02)
    assert np.allclose(o3, a * o1 + b * o2, rtol=1e-12, atol=1e-12)
    assert np.allclose(S3, a * S1 + b * S2, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("L,chunk", [(100, 16), (64, 64), (130, 64), (7, 64)])
def test_chunked_form_matches_token_loop(oracle_lib, L, chunk):
    q, k, v, g, beta, S0 = rand_head(21 + L, L, 16, 12, gate_scale=2.0)
    g = np.maximum(g * 3.0, -5.0)          # strong decays, reaching the safe-gate bound
    o, S = oracle.recurrence(q, k, v, g, beta, S0)
    oc, Sc = chunked.forward(q, k, v, g, beta, S0, chunk=chunk)
    assert max_over_rms(oc, o) < 1e-12
    assert rel_fro(Sc, S) < 1e-12


# ---------------------------------------------------------------- preprocess
def _torch_conv_silu(x, w):
    """Library reference: nn.Conv1d(C, C, groups=C, kernel_size=4, padding=3,
    bias=False) keeping the first T outputs, then SiLU.  x [T, C], w [C, 4]."""
    xt = torch.from_numpy(np.ascontiguousarray(x.T))[None]
    wt = torch.from_numpy(np.ascontiguousarray(w))[:, None, :]
    y = torch.nn.functional.conv1d(xt, wt, padding=3, groups=x.shape[1])[0, :, : x.shape[0]]
    return torch.nn.functional.silu(y).numpy().T, y.numpy().T


def test_conv_silu_matches_torch_conv1d(oracle_lib):
    p = small_problem(1, [37], H=2, dk=8, dv=6, state=False, conv=False)
    for h in range(2):
        qh, kh, vh, g, beta = oracle.preprocess_head(p, 0, h, flags=oracle.FLAG_SKIP_L2NORM)
        for got, x, w, d in ((qh, p.q, p.w_q, 8), (kh, p.k, p.w_k, 8), (vh, p.v, p.w_v, 6)):
            xs = as_f64(x, p.io)[:, h * d:(h + 1) * d]
            ws = as_f64(w, p.io)[h * d:(h + 1) * d]
            ref, _ = _torch_conv_silu(xs, ws)
            assert np.allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_conv_single_channel_numpy_convolve(oracle_lib):
    p = small_problem(2, [20], H=1, dk=4, dv=4, state=False, conv=False)
    qh, _, _, _, _ = oracle.preprocess_head(p, 0, 0, flags=oracle.FLAG_SKIP_L2NORM)
    x = as_f64(p.q, p.io)[:, 1]
    w = as_f64(p.w_q, p.io)[1]
    # y_t = sum_j w[j] x[t-3+j]  ==  full convolution of x with reversed taps
    y = np.convolve(x, w[::-1])[:20]
    assert np.allclose(qh[:, 1], y * scipy.special.expit(y), rtol=1e-12, atol=1e-13)


def test_conv_identity_taps_and_history(oracle_lib):
    # taps [0,0,0,1]: y = x;  taps [1,0,0,0]: y_t = x_{t-3}, reading the history
    p = small_problem(3, [6], H=1, dk=4, dv=4, state=False, conv=True)
    p.w_q = np.zeros_like(p.w_q); p.w_q[:, 3] = 1.0
    p.w_k = np.zeros_like(p.w_k); p.w_k[:, 0] = 1.0
    qh, kh, _, _, _ = oracle.preprocess_head(p, 0, 0, flags=oracle.FLAG_SKIP_L2NORM)
    x = as_f64(p.q, p.io)
    assert np.allclose(qh, x * scipy.special.expit(x), rtol=1e-14)
    xk = as_f64(p.k, p.io)
    hist = as_f64(p.conv_state, p.io)[0][:, 4:8]          # k channels of head 0
    ext = np.concatenate([hist, xk], axis=0)              # [3 + T, 4]
    yk = ext[:6]
    assert np.allclose(kh, yk * scipy.special.expit(yk), rtol=1e-14)


def test_l2norm_unit_and_direction(oracle_lib):
    p = small_problem(4, [25], H=2, dk=8, dv=8, state=False, conv=False)
    for h in range(2):
        qn, kn, _, _, _ = oracle.preprocess_head(p, 0, h)
        qr, kr, _, _, _ = oracle.preprocess_head(p, 0, h, flags=oracle.FLAG_SKIP_L2NORM)
        for n, r in ((qn, qr), (kn, kr)):
            norms = np.linalg.norm(n, axis=1)
            rn = np.linalg.norm(r, axis=1)
            # |u / sqrt(|u|^2 + eps)| = |u| / sqrt(|u|^2 + eps)
            assert np.allclose(norms, rn / np.sqrt(rn ** 2 + oracle.DEFAULT_EPS), rtol=1e-14)
            assert np.allclose(n * rn[:, None], r * norms[:, None], rtol=1e-12, atol=1e-14)


def test_scale_multiplies_q_only(oracle_lib):
    p = small_problem(5, [10], H=1, dk=8, dv=8, state=False, conv=False)
    q1, k1, v1, _, _ = oracle.preprocess_head(p, 0, 0)
    q2, k2, v2, _, _ = oracle.preprocess_head(p, 0, 0, scale=0.25)
    assert np.allclose(q2, 0.25 * q1, rtol=1e-15) and np.array_equal(k1, k2) and np.array_equal(v1, v2)


def test_gate_special_values(oracle_lib):
    p = small_problem(6, [40], H=2, dk=8, dv=8, state=False, conv=False)
    alpha = as_f64(p.alpha, p.io)
    # softplus via a library routine (logaddexp), and the clamp at -5
    for h in range(2):
        _, _, _, g, _ = oracle.preprocess_head(p, 0, h)
        x = alpha[:, h, :] + p.dt_bias.astype(np.float64)[h * 8:(h + 1) * 8]
        ref = np.maximum(-np.exp(np.float64(p.A_log[h])) * np.logaddexp(0.0, x), -5.0)
        assert np.allclose(g, ref, rtol=1e-14, atol=1e-15)
        assert (g <= 0).all() and (g >= -5.0).all()
    # A_log = -inf: no decay at all
    p2 = small_problem(6, [40], H=2, dk=8, dv=8, state=False, conv=False)
    p2.A_log = np.array([-np.inf, -np.inf], dtype=np.float32)
    _, _, _, g0, _ = oracle.preprocess_head(p2, 0, 1)
    assert np.all(g0 == 0.0)
    # alpha + dt_bias = 0 gives softplus = ln 2
    p3 = small_problem(6, [3], H=1, dk=4, dv=4, state=False, conv=False)
    p3.alpha = np.zeros_like(p3.alpha); p3.dt_bias = np.zeros_like(p3.dt_bias)
    p3.A_log = np.array([0.5], dtype=np.float32)
    _, _, _, g3, _ = oracle.preprocess_head(p3, 0, 0)
    assert np.allclose(g3, -np.exp(np.float64(np.float32(0.5))) * np.log(2.0), rtol=1e-15)
    # large inputs hit the bound exactly
    p3.alpha = np.full_like(p3.alpha, 50.0)
    _, _, _, g4, _ = oracle.preprocess_head(p3, 0, 0)
    assert np.all(g4 == -5.0)
    _, _, _, g5, _ = oracle.preprocess_head(p3, 0, 0, lower_bound=-np.inf)
    assert np.allclose(g5, -np.exp(np.float64(np.float32(0.5))) * 50.0, rtol=1e-14)


def test_gate_clamp_is_hit_on_workload_distribution(oracle_lib):
    from kda_inputs import make_problem
    p = make_problem(77, [256], 8, 32, 32, BF16)
    hits = 0
    for h in range(8):
        _, _, _, g, _ = oracle.preprocess_head(p, 0, h)
        hits += int(np.sum(g == -5.0))
        assert (g >= -5.0).all()
    assert hits > 0


def test_beta_is_sigmoid(oracle_lib):
    p = small_problem(8, [30], H=3, dk=4, dv=4, state=False, conv=False)
    b = as_f64(p.b, p.io)
    for h in range(3):
        _, _, _, _, beta = oracle.preprocess_head(p, 0, h)
        assert np.allclose(beta, scipy.special.expit(b[:, h]), rtol=1e-15)
        _, _, _, _, beta2 = oracle.preprocess_head(p, 0, h, flags=oracle.FLAG_BETA_X2)
        assert np.allclose(beta2, 2 * beta, rtol=1e-15)
    p.b = np.zeros_like(p.b)
    _, _, _, _, beta0 = oracle.preprocess_head(p, 0, 0)
    assert np.all(beta0 == 0.5)


# ---------------------------------------------------------------- test hooks
# The flags that feed the recurrence post-activation inputs.  Each hook must
# hand its input through untouched: no conv, no SiLU, no clamp, no sigmoid.

def test_skip_conv_passes_raw_inputs(oracle_lib):
    p = small_problem(14, [23], H=2, dk=8, dv=6, state=False, conv=True)
    for h in range(2):
        qh, kh, vh, _, _ = oracle.preprocess_head(p, 0, h,
                                                  flags=oracle.FLAG_SKIP_CONV | oracle.FLAG_SKIP_L2NORM)
        for got, x, d in ((qh, p.q, 8), (kh, p.k, 8), (vh, p.v, 6)):
            assert np.array_equal(got, as_f64(x, p.io)[:, h * d:(h + 1) * d])
    # with the L2 norm on, SKIP_CONV fed SiLU(conv(x)) (computed by torch's
    # conv1d, stored as fp32) reproduces the default path from raw x up to
    # that fp32 rounding of the activations
    p2 = small_problem(15, [31], H=2, dk=8, dv=6, state=False, conv=False)
    acts = []
    for x, w in ((p2.q, p2.w_q), (p2.k, p2.w_k), (p2.v, p2.w_v)):
        u, _ = _torch_conv_silu(as_f64(x, p2.io), as_f64(w, p2.io))
        acts.append(np.ascontiguousarray(u, dtype=np.float32))
    pre = Problem(p2.seqlens, p2.H, p2.dk, p2.dv, FP32, acts[0], acts[1], acts[2], p2.alpha, p2.b,
                  p2.w_q, p2.w_k, p2.w_v, p2.A_log, p2.dt_bias)
    for h in range(2):
        ref = oracle.preprocess_head(p2, 0, h)
        got = oracle.preprocess_head(pre, 0, h, flags=oracle.FLAG_SKIP_CONV)
        for a, b in zip(got, ref):
            assert np.allclose(a, b, rtol=2e-6, atol=1e-7)


def test_raw_gate_is_alpha_unclamped(oracle_lib):
    p = small_problem(16, [12], H=2, dk=8, dv=8, state=False, conv=False)
    r = np.random.default_rng(16)
    p.alpha = r.uniform(-30.0, 0.5, size=p.alpha.shape).astype(np.float32)   # far below the -5 bound
    p.alpha[0, 0, :3] = [-5.0, -5.0000001, 0.0]
    for h in range(2):
        _, _, _, g, _ = oracle.preprocess_head(p, 0, h, flags=oracle.FLAG_RAW_GATE)
        assert np.array_equal(g, p.alpha[:, h, :].astype(np.float64))
        _, _, _, g2, _ = oracle.preprocess_head(p, 0, h, flags=oracle.FLAG_RAW_GATE, lower_bound=-1.0)
        assert np.array_equal(g2, g)
    assert (p.alpha < -5.0).any()


def test_raw_beta_is_b(oracle_lib):
    p = small_problem(17, [15], H=3, dk=4, dv=4, state=False, conv=False)
    r = np.random.default_rng(17)
    p.b = r.uniform(-0.5, 1.5, size=p.b.shape).astype(np.float32)
    for h in range(3):
        _, _, _, _, beta = oracle.preprocess_head(p, 0, h, flags=oracle.FLAG_RAW_BETA)
        assert np.array_equal(beta, p.b[:, h].astype(np.float64))
        _, _, _, _, beta2 = oracle.preprocess_head(p, 0, h, flags=oracle.FLAG_RAW_BETA | oracle.FLAG_BETA_X2)
        assert np.array_equal(beta2, 2.0 * p.b[:, h].astype(np.float64))


# ---------------------------------------------------------------- whole forward
def test_forward_equals_preprocess_then_recurrence(oracle_lib):
    p = small_problem(9, [33, 17], H=2, dk=8, dv=6)
    o, S, cout, _ = oracle.forward(p)
    cu = p.cu_seqlens
    for n in range(2):
        for h in range(2):
            qh, kh, vh, g, beta = oracle.preprocess_head(p, n, h)
            on, Sn = bruteforce.states_and_outputs(qh, kh, vh, g, beta, p.initial_state[n, h]) \
                if cu[n + 1] - cu[n] <= 20 else oracle.recurrence(qh, kh, vh, g, beta, p.initial_state[n, h])
            assert np.allclose(o[cu[n]:cu[n + 1], h], on, rtol=1e-13, atol=1e-13)
            assert np.allclose(S[n, h], Sn, rtol=1e-13, atol=1e-13)


def test_varlen_sequences_are_independent(oracle_lib):
    p = small_problem(10, [5, 64, 1, 70], H=2, dk=8, dv=8)
    o, S, cout, _ = oracle.forward(p)
    cu = p.cu_seqlens
    for n in range(4):
        sl = slice(cu[n], cu[n + 1])
        sub = Problem([p.seqlens[n]], p.H, p.dk, p.dv, p.io, p.q[sl], p.k[sl], p.v[sl], p.alpha[sl],
                      p.b[sl], p.w_q, p.w_k, p.w_v, p.A_log, p.dt_bias,
                      p.initial_state[n:n + 1], p.conv_state[n:n + 1])
        o1, S1, c1, _ = oracle.forward(sub)
        assert np.array_equal(o1, o[sl]) and np.array_equal(S1[0], S[n]) and np.array_equal(c1[0], cout[n])


@pytest.mark.parametrize("T1,T2", [(20, 1), (20, 2), (20, 5), (2, 4), (0, 3)])
def test_prefill_then_decode_equals_long_prefill(oracle_lib, T1, T2):
    p = small_problem(11, [T1 + T2], H=2, dk=8, dv=8)
    o_full, S_full, c_full, _ = oracle.forward(p)
    # prefill of the first T1 tokens
    pre = Problem([T1], p.H, p.dk, p.dv, p.io, p.q[:T1], p.k[:T1], p.v[:T1], p.alpha[:T1], p.b[:T1],
                  p.w_q, p.w_k, p.w_v, p.A_log, p.dt_bias, p.initial_state, p.conv_state)
    o1, S, cs, _ = oracle.forward(pre)
    outs = [o1]
    for t in range(T1, T1 + T2):
        tok = tuple(a[t:t + 1] for a in (p.q, p.k, p.v, p.alpha, p.b))
        ot, S, cs = oracle.decode_reference(S, cs, tok, (p.w_q, p.w_k, p.w_v, p.A_log, p.dt_bias),
                                            p.H, p.dk, p.dv, p.io)
        outs.append(ot)
    o_cat = np.concatenate(outs, axis=0)
    assert np.allclose(o_cat, o_full, rtol=1e-12, atol=1e-13)
    assert np.allclose(S, S_full, rtol=1e-12, atol=1e-13)
    assert np.array_equal(cs, c_full)


def test_conv_state_out_short_sequences(oracle_lib):
    # a sequence shorter than the kernel history keeps the older history entries
    p = small_problem(12, [1, 2, 3, 4], H=1, dk=4, dv=4)
    _, _, cout, _ = oracle.forward(p)
    cin = as_f64(p.conv_state, p.io)
    raw = np.concatenate([as_f64(p.q, p.io), as_f64(p.k, p.io), as_f64(p.v, p.io)], axis=1)
    cu = p.cu_seqlens
    for n, L in enumerate(p.seqlens):
        ext = np.concatenate([cin[n], raw[cu[n]:cu[n + 1]]], axis=0)
        assert np.array_equal(cout[n], ext[-3:])


def test_items_subset_matches_full(oracle_lib):
    p = small_problem(13, [9, 12], H=3, dk=4, dv=4)
    o, S, _, _ = oracle.forward(p)
    o2, S2, _, _ = oracle.forward(p, items=[1, 5])
    assert np.array_equal(o2[:9, 1], o[:9, 1]) and np.array_equal(S2[1, 2], S[1, 2])
    assert np.isnan(o2[:9, 0]).all()


# ---- the output epilogue: o_norm (RMS over a head's dv outputs) x sigmoid gate
# (AliceAI page, sections 二 and 三).  Properties that fix every part of it:
# the mean over the row (not a sum, not over other heads), eps inside the
# square root, a per-channel weight, and the logistic function of the gate.

def _og_rows(seed, rows, dv):
    r = np.random.default_rng(seed)
    o = r.standard_normal((rows, dv)) * r.uniform(0.1, 10.0, size=(rows, 1))
    g = r.standard_normal((rows, dv)) * 3
    return o, g


def test_output_gate_unit_rms_and_scale_invariance(oracle_lib):
    o, _ = _og_rows(11, 12, 16)
    big = np.full_like(o, 60.0)           # sigmoid(60) = 1 - 9e-27: the gate fully open
    y = oracle.output_gate(o, big, np.ones(16), eps=0.0)
    np.testing.assert_allclose(np.mean(y * y, axis=1), 1.0, rtol=1e-13)
    for c in (1e-3, 7.5):
        np.testing.assert_allclose(oracle.output_gate(c * o, big, np.ones(16), eps=0.0), y, rtol=1e-13)
    np.testing.assert_allclose(oracle.output_gate(-o, big, np.ones(16), eps=0.0), -y, rtol=1e-13)


def test_output_gate_eps_inside_the_root(oracle_lib):
    # rows of +-sqrt(m): mean square exactly m; with eps = m every |y| is 1/sqrt(2)
    dv = 8
    signs = np.array([1, -1, 1, 1, -1, -1, 1, -1], dtype=np.float64)
    for m in (0.25, 4.0, 9.0):
        o = (np.sqrt(m) * signs)[None, :]
        y = oracle.output_gate(o, np.full_like(o, 60.0), np.ones(dv), eps=m)
        np.testing.assert_allclose(y[0], signs / np.sqrt(2.0), rtol=1e-13)


def test_output_gate_logistic_gate_and_channel_weights(oracle_lib):
    o, g = _og_rows(12, 6, 16)
    w = np.linspace(-2.0, 3.0, 16)
    full = oracle.output_gate(o, np.full_like(g, 60.0), w)
    # sigmoid(g) + sigmoid(-g) = 1: the two gated outputs add up to the open one
    np.testing.assert_allclose(oracle.output_gate(o, g, w) + oracle.output_gate(o, -g, w), full,
                               rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(oracle.output_gate(o, np.zeros_like(g), w), 0.5 * full, rtol=1e-13)
    np.testing.assert_allclose(oracle.output_gate(o, np.full_like(g, np.log(3.0)), w), 0.75 * full,
                               rtol=1e-13)
    # a one-hot weight passes exactly one channel of every row
    for j in (0, 5, 15):
        e = np.zeros(16)
        e[j] = 1.0
        y = oracle.output_gate(o, g, e)
        assert np.all(np.delete(y, j, axis=1) == 0.0)
        assert np.all(y[:, j] != 0.0)


def test_output_gate_rows_are_independent(oracle_lib):
    o, g = _og_rows(13, 10, 32)
    w = np.random.default_rng(14).uniform(0.5, 1.5, 32)
    y = oracle.output_gate(o, g, w)
    o2, g2 = o.copy(), g.copy()
    o2[3] = np.random.default_rng(15).standard_normal(32) * 100
    g2[7] = -g2[7]
    y2 = oracle.output_gate(o2, g2, w)
    same = [r for r in range(10) if r not in (3, 7)]
    assert np.array_equal(y[same], y2[same])
    assert not np.allclose(y[3], y2[3]) and not np.allclose(y[7], y2[7])
    # [T, H, dv] layout: each (token, head) row is normalised on its own
    y3 = oracle.output_gate(o.reshape(5, 2, 32), g.reshape(5, 2, 32), w)
    assert np.array_equal(y3.reshape(10, 32), y)


def test_decode_multi_reference_composes_the_token_loop(oracle_lib):
    """K tokens through slots equal K one-token decode steps on the gathered
    states; committing m < K tokens leaves the state of the m-th step, and 0
    leaves the pools untouched."""
    from kda_inputs import BF16, make_tokens, workload_decode
    K, P = 3, 5
    dp = workload_decode(N=P, H=2, d=16, steps=1, workload_id=77)   # a pool of 5 states and histories
    pool = dp.state.astype(np.float64) * 5
    cpool = dp.conv_state
    params = (dp.w_q, dp.w_k, dp.w_v, dp.A_log, dp.dt_bias)
    toks = make_tokens(79, 3 * K, 2, 16, 16, BF16)
    slots = np.array([4, -1, 1])
    o, Sp, Cp = oracle.decode_multi_reference(pool, cpool, slots, toks, params, 2, 16, 16, BF16, K)
    assert np.all(np.isnan(o[1])) and np.array_equal(Sp[[0, 2, 3]], pool[[0, 2, 3]])
    from kda_inputs import as_f64
    for n in (0, 2):
        S, C = pool[slots[n]][None], cpool[slots[n]][None]
        for t in range(K):
            one = tuple(a[n * K + t:n * K + t + 1] for a in toks)
            o1, S, C = oracle.decode_reference(S, C, one, params, 2, 16, 16, BF16)
            assert np.allclose(o1[0], o[n, t], rtol=1e-12, atol=1e-14)
        assert np.allclose(S[0], Sp[slots[n]], rtol=1e-12, atol=1e-14)
        assert np.array_equal(C[0], Cp[slots[n]])
    # commit counts: 0 keeps the pools, m keeps the m-th state
    o2, Sp2, Cp2 = oracle.decode_multi_reference(pool, cpool, slots, toks, params, 2, 16, 16, BF16, K,
                                                 n_commit=[0, 3, 1])
    assert np.array_equal(o2[[0, 2]], o[[0, 2]])
    assert np.array_equal(Sp2[4], pool[4]) and np.array_equal(Cp2[4], as_f64(cpool[4], BF16))
    one = tuple(a[2 * K:2 * K + 1] for a in toks)
    _, S1, C1 = oracle.decode_reference(pool[1][None], cpool[1][None], one, params, 2, 16, 16, BF16)
    assert np.allclose(S1[0], Sp2[1], rtol=1e-12, atol=1e-14) and np.array_equal(C1[0], Cp2[1])
