"""Seeded synthetic inputs generated directly on the GPU (for full-size runs).

Per-token tensors of the large workloads (hundreds of millions of values) are
drawn on the device with torch's counter-based Philox generator, seeded from
``SeedSequence([workload_id, tensor_id, step])``, in float32 and rounded to
bf16 (round to nearest even) where the workload is bf16.  Small per-layer
parameters and initial states come from the numpy streams of ``kda_inputs``.
The oracle later reads back exactly the stored bytes of the heads it checks,
so both sides see identical inputs.  No method arithmetic here.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np
import torch

from . import (BF16, FP32, T_ALPHA, T_B, T_CONV, T_K, T_Q, T_S0, T_V, Problem, make_params, _normal)


def _seed(workload_id: int, tensor_id: int, step: int) -> int:
    return int(np.random.SeedSequence([workload_id, tensor_id, step, 0xD]).generate_state(1, np.uint64)[0] >> 1)


def device_normal(shape, workload_id: int, tensor_id: int, device, io: str, std: float = 1.0, step: int = 0):
    g = torch.Generator(device=device)
    g.manual_seed(_seed(workload_id, tensor_id, step))
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(torch.bfloat16) if io == BF16 else x


def device_tokens(workload_id, total_T, H, dk, dv, io, device, step=0):
    q = device_normal((total_T, H * dk), workload_id, T_Q, device, io, step=step)
    k = device_normal((total_T, H * dk), workload_id, T_K, device, io, step=step)
    v = device_normal((total_T, H * dv), workload_id, T_V, device, io, step=step)
    alpha = device_normal((total_T, H, dk), workload_id, T_ALPHA, device, io, step=step)
    b = device_normal((total_T, H), workload_id, T_B, device, io, step=step)
    return q, k, v, alpha, b


class DeviceProblem:
    """A packed problem whose per-token tensors live on the device.

    Attributes: seqlens, H, dk, dv, io, tensors (dict: q, k, v, alpha, b,
    cu_seqlens, initial_state, conv_state on the device) and the host
    parameters w_q, w_k, w_v, A_log, dt_bias, initial_state, conv_state.
    """

    def __init__(self, workload_id: int, seqlens: Sequence[int], H: int, dk: int, dv: int, io: str, device,
                 state_seqs: Optional[Sequence[int]] = None, state_std: float = 0.02, conv_state: bool = False):
        self.workload_id, self.seqlens, self.H, self.dk, self.dv, self.io = workload_id, list(seqlens), H, dk, dv, io
        self.device = device
        total = int(sum(seqlens))
        self.w_q, self.w_k, self.w_v, self.A_log, self.dt_bias = make_params(workload_id, H, dk, dv, io)
        N = len(seqlens)
        self.initial_state = None
        if state_seqs is not None:
            S0 = np.zeros((N, H, dk, dv), dtype=np.float32)
            full = _normal(workload_id, T_S0, (N, H, dk, dv), state_std, dtype=FP32)
            for n in state_seqs:
                S0[n] = full[n]
            self.initial_state = S0
        self.conv_state = _normal(workload_id, T_CONV, (N, 3, H * (2 * dk + dv)), 1.0, dtype=io) if conv_state else None
        q, k, v, alpha, b = device_tokens(workload_id, total, H, dk, dv, io, device)
        from .torch_io import to_torch
        self.tensors = {"q": q, "k": k, "v": v, "alpha": alpha, "b": b,
                        "cu_seqlens": torch.tensor(np.concatenate([[0], np.cumsum(seqlens)]), dtype=torch.int32,
                                                   device=device),
                        "initial_state": None if self.initial_state is None else
                        torch.from_numpy(self.initial_state).to(device),
                        "conv_state": None if self.conv_state is None else to_torch(self.conv_state, io, device)}

    @property
    def cu_seqlens(self):
        return np.concatenate([[0], np.cumsum(self.seqlens)]).astype(np.int64)

    @property
    def ctot(self):
        return self.H * (2 * self.dk + self.dv)

    def config(self, out_dtype=None, **kw):
        from .torch_io import make_config
        return make_config(self, self.device, out_dtype, **kw)

    def seq_problem(self, n: int) -> Problem:
        """Host copy of the stored inputs of sequence n, all heads, as a
        one-sequence problem."""
        cu = self.cu_seqlens
        t0, t1 = int(cu[n]), int(cu[n + 1])
        T = self.tensors

        def host(x):
            x = x.contiguous()
            if x.dtype == torch.bfloat16:
                return x.view(torch.int16).cpu().numpy().view(np.uint16)
            return x.cpu().numpy()

        cs = None if self.conv_state is None else self.conv_state[n:n + 1]
        S0 = None if self.initial_state is None else self.initial_state[n:n + 1]
        return Problem([t1 - t0], self.H, self.dk, self.dv, self.io,
                       host(T["q"][t0:t1]), host(T["k"][t0:t1]), host(T["v"][t0:t1]), host(T["alpha"][t0:t1]),
                       host(T["b"][t0:t1]), self.w_q, self.w_k, self.w_v, self.A_log, self.dt_bias, S0, cs)

    def head_problem(self, n: int, h: int, t_end: Optional[int] = None) -> Problem:
        """Host copy of the stored inputs of sequence n, head h (optionally only
        its first t_end tokens) as a one-sequence, one-head problem."""
        cu = self.cu_seqlens
        t0, t1 = int(cu[n]), int(cu[n + 1])
        if t_end is not None:
            t1 = t0 + min(t_end, t1 - t0)
        dk, dv, H = self.dk, self.dv, self.H
        T = self.tensors

        def host(x):
            x = x.contiguous()
            if x.dtype == torch.bfloat16:
                return x.view(torch.int16).cpu().numpy().view(np.uint16)
            return x.cpu().numpy()

        cs = None
        if self.conv_state is not None:
            c = self.conv_state[n:n + 1]
            cs = np.concatenate([c[:, :, h * dk:(h + 1) * dk], c[:, :, H * dk + h * dk:H * dk + (h + 1) * dk],
                                 c[:, :, 2 * H * dk + h * dv:2 * H * dk + (h + 1) * dv]], axis=2)
        S0 = None if self.initial_state is None else self.initial_state[n:n + 1, h:h + 1]
        return Problem([t1 - t0], 1, dk, dv, self.io,
                       host(T["q"][t0:t1, h * dk:(h + 1) * dk]), host(T["k"][t0:t1, h * dk:(h + 1) * dk]),
                       host(T["v"][t0:t1, h * dv:(h + 1) * dv]), host(T["alpha"][t0:t1, h:h + 1]),
                       host(T["b"][t0:t1, h:h + 1]),
                       self.w_q[h * dk:(h + 1) * dk], self.w_k[h * dk:(h + 1) * dk], self.w_v[h * dv:(h + 1) * dv],
                       self.A_log[h:h + 1], self.dt_bias[h * dk:(h + 1) * dk], S0, cs)
