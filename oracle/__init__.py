"""fp64 CPU oracle for the KDA core -- TEST INFRASTRUCTURE.

Only ``tests/``, the smoke check in ``__graft_entry__`` and the CPU-baseline
leg of ``bench.py`` may import this package.  It shares no code with the HIP
library: its arithmetic lives in ``kda_oracle.c`` (plain C, double precision,
token by token) and in the numpy modules ``bruteforce`` and ``chunked``, which
pin the C code from independent derivations.

Every function here accepts the *stored* input tensors (bf16 bit patterns or
float32, as produced by ``kda_inputs``) and widens them exactly to float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

from kda_inputs import BF16, FP32, Problem, as_f64

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_SRC_BWD = os.path.join(_HERE, "kda_oracle_bwd.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")

FLAG_SKIP_CONV = 1
FLAG_SKIP_L2NORM = 2
FLAG_RAW_GATE = 4
FLAG_RAW_BETA = 8
FLAG_BETA_X2 = 16

DEFAULT_LOWER_BOUND = -5.0   # safe gate (Ling-3.0-flash-VL page, section "KDA 层的安全门")
DEFAULT_EPS = 1e-6           # L2-norm epsilon (not stated on the pages; a reading)
DEFAULT_ONORM_EPS = 1e-6     # o_norm epsilon (not stated on the pages; a reading)


def build(force: bool = False) -> str:
    """Compile the C oracle (forward and gradient) with gcc into
    ``oracle/libkda_oracle.so``."""
    newest = max(os.path.getmtime(_SRC), os.path.getmtime(_SRC_BWD))
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < newest:
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-std=c11", "-Wall",
                               "-o", tmp, _SRC, _SRC_BWD, "-lm", "-lpthread"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        dp = ctypes.POINTER(ctypes.c_double)
        lib.kda_oracle_forward.restype = ctypes.c_int
        lib.kda_oracle_forward.argtypes = [
            ctypes.c_int, ctypes.POINTER(ctypes.c_int64), ctypes.c_int, ctypes.c_int, ctypes.c_int,
            dp, dp, dp, dp, dp, dp, dp, dp, dp, dp,
            ctypes.c_double, ctypes.c_double, ctypes.c_double, ctypes.c_uint,
            dp, dp, dp, dp, dp, ctypes.POINTER(ctypes.c_int32), ctypes.c_int, ctypes.c_int]
        lib.kda_oracle_preprocess_head.restype = None
        lib.kda_oracle_preprocess_head.argtypes = [
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            dp, dp, dp, dp, dp, dp, dp, dp, dp, dp, dp,
            ctypes.c_double, ctypes.c_double, ctypes.c_double, ctypes.c_uint,
            dp, dp, dp, dp, dp]
        lib.kda_oracle_output_gate.restype = None
        lib.kda_oracle_output_gate.argtypes = [ctypes.c_long, ctypes.c_int, dp, dp, dp, ctypes.c_double, dp]
        lib.kda_oracle_backward.restype = ctypes.c_int
        lib.kda_oracle_backward.argtypes = [
            ctypes.c_int, ctypes.POINTER(ctypes.c_int64), ctypes.c_int, ctypes.c_int, ctypes.c_int,
            dp, dp, dp, dp, dp, dp, dp, dp, dp, dp,
            ctypes.c_double, ctypes.c_double, ctypes.c_double, ctypes.c_uint,
            dp, dp, dp, dp,
            dp, dp, dp, dp, dp, dp, dp, dp, dp, dp, dp, dp, ctypes.c_int]
        lib.kda_oracle_recurrence_bwd.restype = None
        lib.kda_oracle_recurrence_bwd.argtypes = [
            ctypes.c_int, ctypes.c_int, ctypes.c_int, dp, dp, dp, dp, dp, dp, dp, ctypes.c_long, dp,
            dp, dp, dp, dp, dp, dp]
        lib.kda_oracle_recurrence.restype = None
        lib.kda_oracle_recurrence.argtypes = [
            ctypes.c_int, ctypes.c_int, ctypes.c_int, dp, dp, dp, dp, dp, dp, dp, ctypes.c_long]
        _lib = lib
    return _lib


def _p(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.dtype == np.float64 and a.flags.c_contiguous
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _f64(a, io):
    return None if a is None else np.ascontiguousarray(as_f64(a, io))


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def forward(p: Problem, *, scale: float = 1.0, lower_bound: float = DEFAULT_LOWER_BOUND,
            eps: float = DEFAULT_EPS, flags: int = 0, initial_state=None, conv_state=None,
            items: Optional[Sequence[int]] = None, nthreads: Optional[int] = None,
            with_conv_out: bool = True):
    """Run the oracle over a packed problem.

    Returns (o [total_T, H, dv], S [N, H, dk, dv], conv_out [N, 3, Ctot] or None,
    threads_used), all float64.  ``initial_state``/``conv_state`` default to the
    problem's own; pass arrays to override (used by continuation tests).
    ``items`` restricts the work to the listed (seq*H + head) pairs; rows of
    the other pairs are left as NaN.
    """
    lib = _load()
    io = p.io
    H, dk, dv = p.H, p.dk, p.dv
    N = len(p.seqlens)
    cu = np.ascontiguousarray(p.cu_seqlens, dtype=np.int64)
    q, k, v = _f64(p.q, io), _f64(p.k, io), _f64(p.v, io)
    alpha, b = _f64(p.alpha, io), _f64(p.b, io)
    w_q, w_k, w_v = _f64(p.w_q, io), _f64(p.w_k, io), _f64(p.w_v, io)
    A_log = np.ascontiguousarray(p.A_log, dtype=np.float64)
    dt_bias = np.ascontiguousarray(p.dt_bias, dtype=np.float64)
    S0 = initial_state if initial_state is not None else p.initial_state
    S0 = None if S0 is None else np.ascontiguousarray(np.asarray(S0, dtype=np.float64))
    cs = conv_state if conv_state is not None else p.conv_state
    if cs is not None and cs.dtype == np.uint16:
        cs = as_f64(cs, BF16)
    cs = None if cs is None else np.ascontiguousarray(np.asarray(cs, dtype=np.float64))
    # the C code trusts these shapes
    assert S0 is None or S0.shape == (N, H, dk, dv)
    assert cs is None or cs.shape == (N, 3, p.ctot)
    total = p.total_T
    o = np.full((total, H, dv), np.nan)
    S = np.full((N, H, dk, dv), np.nan)
    cout = np.zeros((N, 3, p.ctot)) if with_conv_out else None
    it = None
    n_it = 0
    if items is not None:
        it = np.ascontiguousarray(np.asarray(items, dtype=np.int32))
        n_it = int(it.size)
    nt = nthreads if nthreads is not None else default_threads()
    used = lib.kda_oracle_forward(
        N, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), H, dk, dv,
        _p(q), _p(k), _p(v), _p(alpha), _p(b), _p(w_q), _p(w_k), _p(w_v), _p(A_log), _p(dt_bias),
        float(scale), float(lower_bound), float(eps), int(flags),
        _p(S0), _p(cs), _p(o), _p(S), _p(cout),
        None if it is None else it.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), n_it, int(nt))
    return o, S, cout, used


def preprocess_head(p: Problem, seq: int, h: int, *, scale: float = 1.0,
                    lower_bound: float = DEFAULT_LOWER_BOUND, eps: float = DEFAULT_EPS,
                    flags: int = 0, conv_state=None):
    """Post-preprocess tensors of one (sequence, head): q, k [L, dk], v [L, dv],
    g [L, dk], beta [L] (float64)."""
    lib = _load()
    io = p.io
    H, dk, dv = p.H, p.dk, p.dv
    cu = p.cu_seqlens
    t0, t1 = int(cu[seq]), int(cu[seq + 1])
    L = t1 - t0
    q = np.ascontiguousarray(_f64(p.q, io)[t0:t1])
    k = np.ascontiguousarray(_f64(p.k, io)[t0:t1])
    v = np.ascontiguousarray(_f64(p.v, io)[t0:t1])
    alpha = np.ascontiguousarray(_f64(p.alpha, io)[t0:t1])
    b = np.ascontiguousarray(_f64(p.b, io)[t0:t1])
    w_q, w_k, w_v = _f64(p.w_q, io), _f64(p.w_k, io), _f64(p.w_v, io)
    A_log = np.ascontiguousarray(p.A_log, dtype=np.float64)
    dt_bias = np.ascontiguousarray(p.dt_bias, dtype=np.float64)
    cs = conv_state if conv_state is not None else p.conv_state
    if cs is not None:
        cs = as_f64(cs, BF16) if cs.dtype == np.uint16 else np.asarray(cs, dtype=np.float64)
        cs = np.ascontiguousarray(cs[seq])
    qh = np.zeros((L, dk)); kh = np.zeros((L, dk)); vh = np.zeros((L, dv))
    g = np.zeros((L, dk)); beta = np.zeros((L,))
    lib.kda_oracle_preprocess_head(L, H, dk, dv, h, _p(q), _p(k), _p(v), _p(alpha), _p(b),
                                   _p(w_q), _p(w_k), _p(w_v), _p(A_log), _p(dt_bias), _p(cs),
                                   float(scale), float(lower_bound), float(eps), int(flags),
                                   _p(qh), _p(kh), _p(vh), _p(g), _p(beta))
    return qh, kh, vh, g, beta


def recurrence(q, k, v, g, beta, S0=None):
    """The token recurrence alone on post-preprocess inputs of one head.
    q, k, g [L, dk]; v [L, dv]; beta [L]; S0 [dk, dv] or None.
    Returns (o [L, dv], S [dk, dv])."""
    lib = _load()
    q, k, v, g = (np.ascontiguousarray(np.asarray(a, dtype=np.float64)) for a in (q, k, v, g))
    beta = np.ascontiguousarray(np.asarray(beta, dtype=np.float64))
    L, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64, copy=True, order="C")
    o = np.zeros((L, dv))
    lib.kda_oracle_recurrence(L, dk, dv, _p(q), _p(k), _p(v), _p(g), _p(beta), _p(S), _p(o), dv)
    return o, S


def backward(p: Problem, dO, dST=None, *, scale: float = 1.0, lower_bound: float = DEFAULT_LOWER_BOUND,
             eps: float = DEFAULT_EPS, flags: int = 0, initial_state=None, conv_state=None,
             nthreads: Optional[int] = None):
    """Gradient of a packed problem's outputs (o and the final state) with
    respect to every input: the vector-Jacobian product for the loss
    gradients dO [total_T, H, dv] and dST [N, H, dk, dv] (None: the final
    state does not enter the loss).

    Returns a dict of float64 arrays: dq, dk [total_T, H*dk]; dv [total_T,
    H*dv]; dalpha [total_T, H, dk]; db [total_T, H]; dS0 [N, H, dk, dv];
    dconv [N, 3, Ctot] (gradient w.r.t. the incoming conv history);
    dw_q, dw_k [H*dk, 4]; dw_v [H*dv, 4]; ddt_bias [H*dk]; dA_log [H]."""
    lib = _load()
    io = p.io
    H, dk, dv = p.H, p.dk, p.dv
    N = len(p.seqlens)
    cu = np.ascontiguousarray(p.cu_seqlens, dtype=np.int64)
    q, k, v = _f64(p.q, io), _f64(p.k, io), _f64(p.v, io)
    alpha, b = _f64(p.alpha, io), _f64(p.b, io)
    w_q, w_k, w_v = _f64(p.w_q, io), _f64(p.w_k, io), _f64(p.w_v, io)
    A_log = np.ascontiguousarray(p.A_log, dtype=np.float64)
    dt_bias = np.ascontiguousarray(p.dt_bias, dtype=np.float64)
    S0 = initial_state if initial_state is not None else p.initial_state
    S0 = None if S0 is None else np.ascontiguousarray(np.asarray(S0, dtype=np.float64))
    cs = conv_state if conv_state is not None else p.conv_state
    if cs is not None and cs.dtype == np.uint16:
        cs = as_f64(cs, BF16)
    cs = None if cs is None else np.ascontiguousarray(np.asarray(cs, dtype=np.float64))
    dO = np.ascontiguousarray(np.asarray(dO, dtype=np.float64))
    dST = None if dST is None else np.ascontiguousarray(np.asarray(dST, dtype=np.float64))
    T = p.total_T
    assert dO.shape == (T, H, dv) and (dST is None or dST.shape == (N, H, dk, dv))
    assert S0 is None or S0.shape == (N, H, dk, dv)
    assert cs is None or cs.shape == (N, 3, p.ctot)
    out = {"dq": np.zeros((T, H * dk)), "dk": np.zeros((T, H * dk)), "dv": np.zeros((T, H * dv)),
           "dalpha": np.zeros((T, H, dk)), "db": np.zeros((T, H)), "dS0": np.zeros((N, H, dk, dv)),
           "dconv": np.zeros((N, 3, p.ctot)), "dw_q": np.zeros((H * dk, 4)), "dw_k": np.zeros((H * dk, 4)),
           "dw_v": np.zeros((H * dv, 4)), "ddt_bias": np.zeros(H * dk), "dA_log": np.zeros(H)}
    nt = nthreads if nthreads is not None else default_threads()
    lib.kda_oracle_backward(
        N, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), H, dk, dv,
        _p(q), _p(k), _p(v), _p(alpha), _p(b), _p(w_q), _p(w_k), _p(w_v), _p(A_log), _p(dt_bias),
        float(scale), float(lower_bound), float(eps), int(flags), _p(S0), _p(cs), _p(dO), _p(dST),
        _p(out["dq"]), _p(out["dk"]), _p(out["dv"]), _p(out["dalpha"]), _p(out["db"]), _p(out["dS0"]),
        _p(out["dconv"]), _p(out["dw_q"]), _p(out["dw_k"]), _p(out["dw_v"]), _p(out["ddt_bias"]),
        _p(out["dA_log"]), int(nt))
    return out


def recurrence_backward(q, k, v, g, beta, S0, dO, dST=None):
    """Gradient of the token recurrence alone (one head, post-preprocess
    inputs): returns (dq, dk, dv, dg, dbeta, dS0), float64."""
    lib = _load()
    q, k, v, g = (np.ascontiguousarray(np.asarray(a, dtype=np.float64)) for a in (q, k, v, g))
    beta = np.ascontiguousarray(np.asarray(beta, dtype=np.float64))
    L, dk = q.shape
    dv = v.shape[1]
    S0 = None if S0 is None else np.ascontiguousarray(np.asarray(S0, dtype=np.float64))
    dO = np.ascontiguousarray(np.asarray(dO, dtype=np.float64))
    dST = None if dST is None else np.ascontiguousarray(np.asarray(dST, dtype=np.float64))
    dq, dkk, dg = np.zeros((L, dk)), np.zeros((L, dk)), np.zeros((L, dk))
    dvv, dbeta, dS0 = np.zeros((L, dv)), np.zeros(L), np.zeros((dk, dv))
    lib.kda_oracle_recurrence_bwd(L, dk, dv, _p(q), _p(k), _p(v), _p(g), _p(beta), _p(S0), _p(dO), dv, _p(dST),
                                  _p(dq), _p(dkk), _p(dvv), _p(dg), _p(dbeta), _p(dS0))
    return dq, dkk, dvv, dg, dbeta, dS0


def decode_reference(S, conv_state, tokens, params, H, dk, dv, io, *, scale=1.0,
                     lower_bound=DEFAULT_LOWER_BOUND, eps=DEFAULT_EPS, flags=0,
                     items: Optional[Sequence[int]] = None, nthreads: Optional[int] = None):
    """One decode step for N sequences (one token each): a length-1 forward per
    sequence with the given state and conv history.

    S [N, H, dk, dv] fp32/fp64; conv_state [N, 3, Ctot] stored dtype;
    tokens = (q, k, v, alpha, b) for N tokens; params = (w_q, w_k, w_v, A_log, dt_bias).
    Returns (o [N, H, dv], S_new, conv_new) in float64."""
    q, k, v, alpha, b = tokens
    w_q, w_k, w_v, A_log, dt_bias = params
    N = q.shape[0]
    prob = Problem([1] * N, H, dk, dv, io, q, k, v, alpha, b, w_q, w_k, w_v, A_log, dt_bias,
                   np.asarray(S, dtype=np.float64), conv_state)
    o, S_new, cout, _ = forward(prob, scale=scale, lower_bound=lower_bound, eps=eps, flags=flags,
                               items=items, nthreads=nthreads)
    return o, S_new, cout


def output_gate(o, gate, weight, eps: float = DEFAULT_ONORM_EPS):
    """The output epilogue: y = o / sqrt(mean(o^2) + eps) * weight * sigmoid(gate)
    per (token, head) row, the mean over the row's dv channels (AliceAI page,
    sections 二 and 三: ``o_norm`` and the sigmoid output gate).
    o, gate [..., dv] (float64 or stored arrays widened by the caller);
    weight [dv].  Returns y with o's shape, float64."""
    lib = _load()
    o = np.ascontiguousarray(np.asarray(o, dtype=np.float64))
    gate = np.ascontiguousarray(np.asarray(gate, dtype=np.float64))
    w = np.ascontiguousarray(np.asarray(weight, dtype=np.float64))
    assert o.shape == gate.shape and o.shape[-1] == w.size
    dv = o.shape[-1]
    y = np.empty_like(o)
    lib.kda_oracle_output_gate(int(o.size // dv) if dv else 0, dv, _p(o), _p(gate), _p(w), float(eps), _p(y))
    return y


def decode_multi_reference(state_pool, conv_pool, slots, tokens, params, H, dk, dv, io, K, n_commit=None, *,
                           scale=1.0, lower_bound=DEFAULT_LOWER_BOUND, eps=DEFAULT_EPS, flags=0,
                           nthreads: Optional[int] = None):
    """K tokens for each of N sequences whose state and conv history live in
    pools, found through ``slots`` (a negative slot: the sequence is skipped).

    state_pool [P, H, dk, dv]; conv_pool [P, 3, Ctot] (stored dtype); slots [N];
    tokens = (q, k, v, alpha, b) packed sequence-major, N*K tokens; params as
    in ``decode_reference``; n_commit [N] (tokens whose updates are kept,
    0..K) or None for K.  The outputs of all K tokens follow the token loop
    from the slot's state; the pools receive the state and conv history after
    the first n_commit[n] tokens -- the same loop over fewer tokens (sequences
    of length 0 pass both through).  Returns (o [N, K, H, dv] with NaN rows for
    skipped sequences, state_pool', conv_pool') in float64."""
    q, k, v, alpha, b = tokens
    w_q, w_k, w_v, A_log, dt_bias = params
    slots = np.asarray(slots)
    N = slots.size
    assert state_pool.shape[1:] == (H, dk, dv) and conv_pool.shape[1:] == (3, H * (2 * dk + dv))
    assert slots.max(initial=-1) < state_pool.shape[0] == conv_pool.shape[0]
    assert all(a.shape[0] == N * K for a in tokens)
    commit = np.full(N, K) if n_commit is None else np.clip(np.asarray(n_commit), 0, K)
    S_pool = np.array(state_pool, dtype=np.float64, copy=True)
    cs_pool = np.array(as_f64(conv_pool, BF16) if conv_pool.dtype == np.uint16 else conv_pool, dtype=np.float64,
                       copy=True)
    o = np.full((N, K, H, dv), np.nan)
    act = [n for n in range(N) if slots[n] >= 0]
    if not act:
        return o, S_pool, cs_pool
    tok = np.concatenate([np.arange(n * K, (n + 1) * K) for n in act])
    sel = lambda a: np.ascontiguousarray(a[tok])
    S0 = np.stack([S_pool[slots[n]] for n in act])
    C0 = np.stack([cs_pool[slots[n]] for n in act])
    full = Problem([K] * len(act), H, dk, dv, io, sel(q), sel(k), sel(v), sel(alpha), sel(b),
                   w_q, w_k, w_v, A_log, dt_bias, S0, C0)
    kw = dict(scale=scale, lower_bound=lower_bound, eps=eps, flags=flags, nthreads=nthreads)
    o_all, _, _, _ = forward(full, **kw)
    for i, n in enumerate(act):
        o[n] = o_all[i * K:(i + 1) * K]
    # the committed prefix of every sequence: the same loop over its first n_commit tokens
    tok_c = np.concatenate([np.arange(n * K, n * K + int(commit[n])) for n in act]).astype(np.int64)
    selc = lambda a: np.ascontiguousarray(a[tok_c])
    part = Problem([int(commit[n]) for n in act], H, dk, dv, io, selc(q), selc(k), selc(v), selc(alpha), selc(b),
                   w_q, w_k, w_v, A_log, dt_bias, S0, C0)
    _, S_c, c_c, _ = forward(part, **kw)
    for i, n in enumerate(act):
        S_pool[slots[n]] = S_c[i]
        cs_pool[slots[n]] = c_c[i]
    return o, S_pool, cs_pool
