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
