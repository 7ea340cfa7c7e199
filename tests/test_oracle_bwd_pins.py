"""Pins for the fp64 gradient oracle (CPU only).

The gradient oracle (oracle/kda_oracle_bwd.c) is tied to things other than
itself:
- central finite differences of the forward oracle (itself pinned in
  test_oracle_pins.py) along a random direction of every input tensor and
  parameter, for the loss  sum(o * R_o) + sum(S_T * R_S);
- the beta = 0 closed form, where the state only decays:
  o_t = (q_t * e^{G_t})^T S_0 and S_T = Diag(e^{G_T}) S_0, whose gradients are
  written out by hand below;
- agreement of the whole-batch gradient with the recurrence-alone gradient
  chained by hand through the test hooks.
Sequences of 2, 70 and 9 tokens cover the conv history (shorter than the
kernel), the 64-token checkpoint segments of the oracle and dk != dv.
"""
import numpy as np
import pytest

import oracle
from kda_inputs import FP64, Problem

FLAGS = {
    "default": 0,
    "beta_x2": oracle.FLAG_BETA_X2,
    "hooks": oracle.FLAG_SKIP_CONV | oracle.FLAG_SKIP_L2NORM | oracle.FLAG_RAW_GATE | oracle.FLAG_RAW_BETA,
}
TENSORS = ("q", "k", "v", "alpha", "b", "initial_state", "conv_state", "w_q", "w_k", "w_v", "dt_bias", "A_log")
GRAD_OF = {"q": "dq", "k": "dk", "v": "dv", "alpha": "dalpha", "b": "db", "initial_state": "dS0",
           "conv_state": "dconv", "w_q": "dw_q", "w_k": "dw_k", "w_v": "dw_v", "dt_bias": "ddt_bias",
           "A_log": "dA_log"}


def fd_problem(seed, lens=(2, 70, 9), H=2, dk=5, dv=4, hooks=False, lb=-5.0):
    """A float64 problem whose gates are clamped in places but never within
    1e-3 of the bound (so finite differences do not straddle the kink)."""
    r = np.random.default_rng(seed)
    T = sum(lens)
    N = len(lens)
    for _ in range(50):
        p = Problem(list(lens), H, dk, dv, FP64, r.standard_normal((T, H * dk)), r.standard_normal((T, H * dk)),
                    r.standard_normal((T, H * dv)), r.standard_normal((T, H, dk)), r.standard_normal((T, H)),
                    r.standard_normal((H * dk, 4)) * 0.5, r.standard_normal((H * dk, 4)) * 0.5,
                    r.standard_normal((H * dv, 4)) * 0.5, r.uniform(0.5, 1.4, size=H),
                    r.standard_normal(H * dk) * 0.3, r.standard_normal((N, H, dk, dv)) * 0.5,
                    r.standard_normal((N, 3, H * (2 * dk + dv))))
        if hooks:
            # post-activation inputs: unit-scale q, k; log-decays in (-2, 0); beta in (0, 1)
            p.alpha = -r.uniform(0.05, 2.0, size=(T, H, dk))
            p.b = r.uniform(0.1, 0.9, size=(T, H))
            p.q *= 0.4
            p.k *= 0.4
            return p
        z = p.alpha + p.dt_bias.reshape(H, dk)[None]
        graw = -np.exp(p.A_log)[None, :, None] * np.logaddexp(0.0, z)
        if (graw < lb).any() and np.min(np.abs(graw - lb)) > 1e-3:
            return p
    raise AssertionError("no problem with a clean clamp margin")


def loss(p, R_o, R_S, **kw):
    o, S, _, _ = oracle.forward(p, with_conv_out=False, **kw)
    return float(np.sum(o * R_o) + np.sum(S * R_S))


def check_fd(p, flags, lb=-5.0, seed=0, h=1e-5, rtol=2e-6, scale=1.0):
    r = np.random.default_rng(seed + 99)
    N, H, dk, dv = len(p.seqlens), p.H, p.dk, p.dv
    R_o = r.standard_normal((p.total_T, H, dv))
    R_S = r.standard_normal((N, H, dk, dv))
    g = oracle.backward(p, R_o, R_S, flags=flags, lower_bound=lb, scale=scale)
    kw = dict(flags=flags, lower_bound=lb, scale=scale)
    for name in TENSORS:
        x0 = np.array(getattr(p, name), dtype=np.float64)
        E = r.standard_normal(x0.shape)
        setattr(p, name, x0 + h * E)
        lp = loss(p, R_o, R_S, **kw)
        setattr(p, name, x0 - h * E)
        lm = loss(p, R_o, R_S, **kw)
        setattr(p, name, x0)
        fd = (lp - lm) / (2 * h)
        an = float(np.sum(g[GRAD_OF[name]] * E))
        mag = max(abs(fd), abs(an), 1e-3 * float(np.linalg.norm(g[GRAD_OF[name]].ravel())), 1e-12)
        assert abs(fd - an) <= rtol * mag + 1e-9, f"{name}: finite difference {fd:.10g} vs gradient {an:.10g}"


@pytest.mark.parametrize("variant", sorted(FLAGS))
def test_gradient_matches_finite_differences(oracle_lib, variant):
    p = fd_problem(11, hooks=variant == "hooks")
    check_fd(p, FLAGS[variant], scale=0.8)   # q's scale differs from 1, so it cannot leak onto k


def test_gradient_without_clamp_and_with_scale(oracle_lib):
    p = fd_problem(12)
    r = np.random.default_rng(5)
    R_o = r.standard_normal((p.total_T, p.H, p.dv))
    R_S = r.standard_normal((len(p.seqlens), p.H, p.dk, p.dv))
    g = oracle.backward(p, R_o, R_S, lower_bound=-np.inf, scale=0.7)
    x0 = p.alpha.copy()
    E = r.standard_normal(x0.shape)
    h = 1e-5
    p.alpha = x0 + h * E
    lp = loss(p, R_o, R_S, lower_bound=-np.inf, scale=0.7)
    p.alpha = x0 - h * E
    lm = loss(p, R_o, R_S, lower_bound=-np.inf, scale=0.7)
    p.alpha = x0
    fd = (lp - lm) / (2 * h)
    assert abs(fd - np.sum(g["dalpha"] * E)) <= 2e-6 * abs(fd)
    # with the clamp on, the clamped channels take no gradient at all
    gc = oracle.backward(p, R_o, R_S)
    z = p.alpha + p.dt_bias.reshape(p.H, p.dk)[None]
    clamped = -np.exp(p.A_log)[None, :, None] * np.logaddexp(0.0, z) < -5.0
    assert clamped.any() and np.all(gc["dalpha"][clamped] == 0.0)
    assert np.all(g["dalpha"][clamped] != 0.0)


def test_beta_zero_closed_form(oracle_lib):
    """beta = 0 (raw beta, test hooks on): S_t = Diag(e^{G_t}) S_0 and
    o_t = (q_t * e^{G_t})^T S_0, so dq_t = e^{G_t} * (S_0 do_t),
    dS_0 = sum_t (q_t e^{G_t}) do_t^T + Diag(e^{G_T}) dS_T,
    dg_t = sum_{u >= t} e^{G_u} q_u (S_0 do_u) + e^{G_T} rowsum(dS_T * S_0),
    and dv = dk = 0."""
    p = fd_problem(13, lens=(37,), H=1, dk=6, dv=3, hooks=True)
    p.b = np.zeros_like(p.b)
    r = np.random.default_rng(6)
    dO = r.standard_normal((37, 1, 3))
    dST = r.standard_normal((1, 1, 6, 3))
    g = oracle.backward(p, dO, dST, flags=FLAGS["hooks"])
    q, G, S0 = p.q, np.cumsum(p.alpha[:, 0, :], axis=0), p.initial_state[0, 0]
    Sdo = dO[:, 0, :] @ S0.T                       # (S_0 do_t) for every t, [T, dk]
    np.testing.assert_allclose(g["dq"], np.exp(G) * Sdo, rtol=1e-12, atol=1e-14)
    dS0 = (q * np.exp(G)).T @ dO[:, 0, :] + np.exp(G[-1])[:, None] * dST[0, 0]
    np.testing.assert_allclose(g["dS0"][0, 0], dS0, rtol=1e-12, atol=1e-14)
    per_t = np.exp(G) * q * Sdo
    dg = np.cumsum(per_t[::-1], axis=0)[::-1] + (np.exp(G[-1]) * np.sum(dST[0, 0] * S0, axis=1))[None]
    np.testing.assert_allclose(g["dalpha"][:, 0, :], dg, rtol=1e-12, atol=1e-14)
    assert np.all(g["dv"] == 0.0) and np.all(g["dk"] == 0.0)


def test_batch_gradient_chains_the_recurrence_gradient(oracle_lib):
    """With every hook on, the raw inputs are the recurrence's own inputs:
    the whole-batch gradient must equal the recurrence-alone gradient of each
    (sequence, head), and d(raw beta) must be the gradient of beta itself."""
    p = fd_problem(14, lens=(70, 3), H=2, dk=4, dv=6, hooks=True)
    r = np.random.default_rng(7)
    dO = r.standard_normal((73, 2, 6))
    g = oracle.backward(p, dO, None, flags=FLAGS["hooks"])
    cu = p.cu_seqlens
    for n in range(2):
        for h in range(2):
            sl = slice(cu[n], cu[n + 1])
            dq, dk, dv, dg, dbeta, dS0 = oracle.recurrence_backward(
                p.q[sl, h * 4:(h + 1) * 4], p.k[sl, h * 4:(h + 1) * 4], p.v[sl, h * 6:(h + 1) * 6],
                p.alpha[sl, h], p.b[sl, h], p.initial_state[n, h], dO[sl, h])
            np.testing.assert_array_equal(g["dq"][sl, h * 4:(h + 1) * 4], dq)
            np.testing.assert_array_equal(g["dk"][sl, h * 4:(h + 1) * 4], dk)
            np.testing.assert_array_equal(g["dv"][sl, h * 6:(h + 1) * 6], dv)
            np.testing.assert_array_equal(g["dalpha"][sl, h], dg)
            np.testing.assert_array_equal(g["db"][sl, h], dbeta)
            np.testing.assert_array_equal(g["dS0"][n, h], dS0)
