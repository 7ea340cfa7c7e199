"""Seeded synthetic inputs for the KDA core.

This module is shared by the fp64 oracle tests and by the HIP path's tests and
benchmark.  It draws random numbers and converts storage formats; it contains
none of the method's arithmetic (no conv, gate, normalisation or recurrence).

Every tensor comes from its own numpy PCG64 stream keyed by
``SeedSequence([workload_id, tensor_id, step])`` so that any tensor can be
regenerated independently.  Floating draws are made in float32 and, for bf16
workloads, rounded to bf16 with round-to-nearest-even.  bf16 tensors are held
as numpy ``uint16`` bit patterns.

Distributions (second parameter of N(.,.) is the standard deviation):
  raw q, k, v       ~ N(0, 1)              [T, H*dk], [T, H*dk], [T, H*dv]
  alpha             ~ N(0, 1)              [T, H, dk]
  b (pre-sigmoid)   ~ N(0, 1)              [T, H]
  conv weights      ~ N(0, 0.25)           [H*dk, 4], [H*dk, 4], [H*dv, 4]
  A_log             ~ U(-1, 1)   fp32      [H]
  dt_bias           ~ N(0, 0.1)  fp32      [H*dk]
  initial state     ~ N(0, 0.02) fp32      [N, H, dk, dv]   (where requested)
  conv state        ~ N(0, 1)              [N, 3, H*(2dk+dv)] (where requested)
  output epilogue:  gate ~ N(0, 2) [T, H, dv]; o_norm weight ~ U(0.5, 1.5) fp32
                    [dv]; a stand-alone o ~ N(0, s_row^2) [T, H, dv] with
                    log10 s_row ~ U(-2, 1) per (token, head) row
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np

BF16 = "bf16"
FP32 = "fp32"
FP64 = "fp64"   # float64 storage: only for oracle-side tests (finite differences)

# tensor ids inside the seed sequence
T_Q, T_K, T_V, T_ALPHA, T_B = 0, 1, 2, 3, 4
T_WQ, T_WK, T_WV, T_ALOG, T_DTB = 5, 6, 7, 8, 9
T_S0, T_CONV = 10, 11
T_GATE, T_ONW, T_O, T_OSCALE = 12, 13, 14, 15


def rng(workload_id: int, tensor_id: int, step: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([workload_id, tensor_id, step])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round to nearest, ties to even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    out = np.empty(u.shape, dtype=np.uint16)
    # process in slabs to bound temporary memory on very large tensors
    flat_u = u.reshape(-1)
    flat_o = out.reshape(-1)
    step = 1 << 24
    for s in range(0, flat_u.size, step):
        blk = flat_u[s:s + step]
        nan = (blk & 0x7FFFFFFF) > 0x7F800000
        r = blk + (((blk >> 16) & 1) + 0x7FFF).astype(np.uint32)
        o = (r >> 16).astype(np.uint16)
        if nan.any():
            o[nan] = ((blk[nan] >> 16) | 0x0040).astype(np.uint16)
        flat_o[s:s + step] = o
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def as_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of a stored tensor (bf16 bits, float32 or float64)."""
    if dtype == BF16:
        return bf16_bits_to_f32(x).astype(np.float64)
    if dtype == FP64:
        return np.asarray(x, dtype=np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def _normal(workload_id, tensor_id, shape, std=1.0, step=0, dtype=FP32):
    x = rng(workload_id, tensor_id, step).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if dtype == BF16:
        return f32_to_bf16_bits(x)
    return x


@dataclass
class Problem:
    """One packed batch of sequences plus the per-layer parameters.

    Tensors use the library's layouts with a leading packed-token dimension:
    q/k [total_T, H*dk], v [total_T, H*dv], alpha [total_T, H, dk],
    b [total_T, H]; conv weights [C, 4] (tap 3 multiplies the current token);
    initial_state [N, H, dk, dv] fp32 or None; conv_state [N, 3, Ctot] or None.
    """
    seqlens: List[int]
    H: int
    dk: int
    dv: int
    io: str
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    alpha: np.ndarray
    b: np.ndarray
    w_q: np.ndarray
    w_k: np.ndarray
    w_v: np.ndarray
    A_log: np.ndarray
    dt_bias: np.ndarray
    initial_state: Optional[np.ndarray] = None
    conv_state: Optional[np.ndarray] = None
    meta: Dict = field(default_factory=dict)

    @property
    def total_T(self) -> int:
        return int(sum(self.seqlens))

    @property
    def cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.seqlens)]).astype(np.int64)

    @property
    def ctot(self) -> int:
        return self.H * (2 * self.dk + self.dv)


def make_params(workload_id: int, H: int, dk: int, dv: int, io: str):
    """Per-layer parameters: conv weights, A_log, dt_bias."""
    w_q = _normal(workload_id, T_WQ, (H * dk, 4), 0.25, dtype=io)
    w_k = _normal(workload_id, T_WK, (H * dk, 4), 0.25, dtype=io)
    w_v = _normal(workload_id, T_WV, (H * dv, 4), 0.25, dtype=io)
    A_log = rng(workload_id, T_ALOG).uniform(-1.0, 1.0, size=(H,)).astype(np.float32)
    dt_bias = _normal(workload_id, T_DTB, (H * dk,), 0.1, dtype=FP32)
    return w_q, w_k, w_v, A_log, dt_bias


def make_tokens(workload_id: int, total_T: int, H: int, dk: int, dv: int, io: str, step: int = 0):
    """Per-token raw inputs q, k, v, alpha, b for ``total_T`` packed tokens."""
    q = _normal(workload_id, T_Q, (total_T, H * dk), step=step, dtype=io)
    k = _normal(workload_id, T_K, (total_T, H * dk), step=step, dtype=io)
    v = _normal(workload_id, T_V, (total_T, H * dv), step=step, dtype=io)
    alpha = _normal(workload_id, T_ALPHA, (total_T, H, dk), step=step, dtype=io)
    b = _normal(workload_id, T_B, (total_T, H), step=step, dtype=io)
    return q, k, v, alpha, b


def make_problem(workload_id: int, seqlens: Sequence[int], H: int, dk: int, dv: int, io: str,
                 state_seqs: Optional[Sequence[int]] = None, state_std: float = 0.02,
                 conv_state: bool = False, step: int = 0) -> Problem:
    """Build a seeded problem.  ``state_seqs`` lists the sequences that start
    from a random initial state (the others start from zeros); None means no
    initial state at all."""
    seqlens = [int(s) for s in seqlens]
    total = int(sum(seqlens))
    q, k, v, alpha, b = make_tokens(workload_id, total, H, dk, dv, io, step)
    w_q, w_k, w_v, A_log, dt_bias = make_params(workload_id, H, dk, dv, io)
    N = len(seqlens)
    S0 = None
    if state_seqs is not None:
        S0 = np.zeros((N, H, dk, dv), dtype=np.float32)
        full = _normal(workload_id, T_S0, (N, H, dk, dv), state_std, dtype=FP32)
        for n in state_seqs:
            S0[n] = full[n]
    cs = None
    if conv_state:
        cs = _normal(workload_id, T_CONV, (N, 3, H * (2 * dk + dv)), 1.0, dtype=io)
    return Problem(seqlens, H, dk, dv, io, q, k, v, alpha, b, w_q, w_k, w_v, A_log, dt_bias, S0, cs)


def make_output_gate_inputs(workload_id: int, n_tokens: int, H: int, dv: int, io: str, step: int = 0):
    """Inputs of the output epilogue: gate [n_tokens, H, dv] (io dtype) and the
    o_norm weight [dv] (fp32)."""
    gate = _normal(workload_id, T_GATE, (n_tokens, H, dv), 2.0, step=step, dtype=io)
    w = rng(workload_id, T_ONW).uniform(0.5, 1.5, size=(dv,)).astype(np.float32)
    return gate, w


def make_epilogue_o(workload_id: int, n_tokens: int, H: int, dv: int, dtype: str, step: int = 0):
    """A stand-alone attention output [n_tokens, H, dv] whose rows have scales
    spread over three decades (the epilogue normalises each row)."""
    scale = 10.0 ** rng(workload_id, T_OSCALE, step).uniform(-2.0, 1.0, size=(n_tokens, H, 1))
    x = rng(workload_id, T_O, step).standard_normal((n_tokens, H, dv), dtype=np.float32) * scale.astype(np.float32)
    x = x.astype(np.float32)
    return f32_to_bf16_bits(x) if dtype == BF16 else x


# --------------------------------------------------------------------------
# The five workloads of the KDA core (sizes as stated by the workload list
# this library is measured on).  ``reduced`` variants keep the structure with
# fewer tokens so a CPU oracle finishes in seconds.
# --------------------------------------------------------------------------
VARLEN_LENGTHS = [1024, 2048, 4096, 8192, 16384, 32768, 65536, 132096]


def workload_tiny_fp32() -> Problem:
    """B=1, T=64, H=2, dk=dv=16, fp32, zero initial state."""
    return make_problem(1, [64], 2, 16, 16, FP32)


def workload_prefill_4k(io: str = BF16) -> Problem:
    """B=1, T=4096, H=32, dk=dv=128, bf16 inputs, zero initial state."""
    return make_problem(2, [4096], 32, 128, 128, io)


def workload_prefill_32k() -> Problem:
    """B=4, T=32768, H=32, dk=dv=128, bf16, initial state ~N(0,0.02)."""
    return make_problem(3, [32768] * 4, 32, 128, 128, BF16, state_seqs=[0, 1, 2, 3])


def workload_varlen() -> Problem:
    """8 packed sequences (262144 tokens), H=32, d=128, bf16; the odd-indexed
    half (2048, 8192, 32768, 132096 tokens) start from a random state."""
    return make_problem(5, VARLEN_LENGTHS, 32, 128, 128, BF16, state_seqs=[1, 3, 5, 7])


@dataclass
class DecodeProblem:
    N: int
    H: int
    dk: int
    dv: int
    io: str
    steps: int
    state: np.ndarray          # [N, H, dk, dv] fp32
    conv_state: np.ndarray     # [N, 3, Ctot]
    w_q: np.ndarray
    w_k: np.ndarray
    w_v: np.ndarray
    A_log: np.ndarray
    dt_bias: np.ndarray
    workload_id: int = 4

    def tokens(self, step: int):
        """Fresh q, k, v, alpha, b for decode step ``step`` (one token per sequence)."""
        return make_tokens(self.workload_id, self.N, self.H, self.dk, self.dv, self.io, step=step + 1)


def workload_decode(N: int = 256, H: int = 32, d: int = 128, steps: int = 128, io: str = BF16,
                    workload_id: int = 4) -> DecodeProblem:
    """N sequences x 1 token per step, fp32 state ~N(0,0.02), conv state of
    3 prior inputs ~N(0,1); fresh inputs every step."""
    w_q, w_k, w_v, A_log, dt_bias = make_params(workload_id, H, d, d, io)
    S = _normal(workload_id, T_S0, (N, H, d, d), 0.02, dtype=FP32)
    cs = _normal(workload_id, T_CONV, (N, 3, H * 3 * d), 1.0, dtype=io)
    return DecodeProblem(N, H, d, d, io, steps, S, cs, w_q, w_k, w_v, A_log, dt_bias, workload_id)
