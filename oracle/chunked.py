"""Chunked (WY) form of the KDA recurrence in float64 -- TEST INFRASTRUCTURE.

The pages give only the per-token loop (AliceAI-Foundation-80B-A3B page,
section 二).  The GPU path evaluates the same map chunk by chunk; this module
is the plain fp64 statement of that chunked algebra, derived by unrolling the
token loop inside one chunk.  It pins the derivation against the token loop
(they agree to rounding), so the GPU path's algebra is checked independently
of any GPU code.

Within a chunk of tokens r = 0..C-1 with start state S_0, let
G_r = sum_{i<=r} g_i (per key channel).  Writing delta_r for the correction
vector of token r, the loop gives

    delta_r = beta_r (v_r - (k_r * e^{G_r})^T S_0) - sum_{i<r} A[r,i] delta_i
    A[r,i]  = beta_r sum_c k_r[c] k_i[c] e^{G_r[c] - G_i[c]}       (i < r)

so (I + A) Delta = Diag(beta) (V - K+ S_0) with K+ = K * e^{G}.  Then

    O   = Q+ S_0 + Aqk Delta,  Q+ = Q * e^{G},
    Aqk[r,i] = sum_c q_r[c] k_i[c] e^{G_r[c] - G_i[c]}   (i <= r)
    S_C = Diag(e^{G_{C-1}}) S_0 + (K * e^{G_{C-1} - G})^T Delta.
"""
from __future__ import annotations

import numpy as np


def forward(q, k, v, g, beta, S0=None, chunk: int = 64):
    q, k, v, g = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g))
    beta = np.asarray(beta, dtype=np.float64)
    L, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.zeros((L, dv))
    for c0 in range(0, L, chunk):
        c1 = min(L, c0 + chunk)
        Q, K, V, Gg, B = q[c0:c1], k[c0:c1], v[c0:c1], g[c0:c1], beta[c0:c1]
        n = c1 - c0
        G = np.cumsum(Gg, axis=0)                       # [n, dk]
        # pairwise decays e^{G_r - G_i}, per channel
        D = np.exp(G[:, None, :] - G[None, :, :])       # [n, n, dk]
        A = np.einsum("rc,ic,ric->ri", K, K, D) * B[:, None]
        A = np.tril(A, -1)
        Aqk = np.tril(np.einsum("rc,ic,ric->ri", Q, K, D))
        Kp = K * np.exp(G)
        rhs = B[:, None] * (V - Kp @ S)
        Delta = np.linalg.solve(np.eye(n) + A, rhs)
        o[c0:c1] = (Q * np.exp(G)) @ S + Aqk @ Delta
        Kt = K * np.exp(G[-1][None, :] - G)
        S = np.exp(G[-1])[:, None] * S + Kt.T @ Delta
    return o, S
