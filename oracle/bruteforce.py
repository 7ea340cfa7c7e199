"""Brute-force product form of the KDA recurrence -- TEST INFRASTRUCTURE.

An independent restatement used to pin the C oracle on tiny inputs.  The
per-token update on the AliceAI-Foundation-80B-A3B page (section 二: decay,
predict with k, correct by beta*(v - prediction), write k*delta^T) is linear
in the state, so one token is the affine map

    S_t = M_t S_{t-1} + beta_t k_t v_t^T,   M_t = (I - beta_t k_t k_t^T) Diag(exp(g_t)).

Unrolling gives the closed sum

    S_t = (M_t ... M_1) S_0 + sum_{s<=t} (M_t ... M_{s+1}) beta_s k_s v_s^T,

and o_t = q_t^T S_t.  This module evaluates that sum with explicit dk x dk
transition matrices and matrix products (O(T^2) products), never running the
token recurrence itself.
"""
from __future__ import annotations

import numpy as np


def transition(k, g, beta):
    """M = (I - beta k k^T) Diag(exp(g)) for one token."""
    k = np.asarray(k, dtype=np.float64)
    dk = k.shape[0]
    return (np.eye(dk) - beta * np.outer(k, k)) @ np.diag(np.exp(g))


def states_and_outputs(q, k, v, g, beta, S0=None):
    """Return (o [L, dv], S_L [dk, dv]) from the unrolled product sum."""
    q, k, v, g = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g))
    beta = np.asarray(beta, dtype=np.float64)
    L, dk = k.shape
    dv = v.shape[1]
    S0 = np.zeros((dk, dv)) if S0 is None else np.asarray(S0, dtype=np.float64)
    Ms = [transition(k[t], g[t], beta[t]) for t in range(L)]
    o = np.zeros((L, dv))
    S_t = S0
    for t in range(L):
        prod = np.eye(dk)
        for s in range(t + 1):          # left-multiply in time order: M_s ... M_1
            prod = Ms[s] @ prod
        S_t = prod @ S0
        for s in range(t + 1):
            tail = np.eye(dk)
            for r in range(s + 1, t + 1):   # M_t ... M_{s+1}
                tail = Ms[r] @ tail
            S_t = S_t + tail @ (beta[s] * np.outer(k[s], v[s]))
        o[t] = q[t] @ S_t
    return o, S_t
