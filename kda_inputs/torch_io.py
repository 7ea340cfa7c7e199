"""Stage seeded problems on a torch device for the HIP library.

Storage conversion only: bf16 bit patterns become torch.bfloat16 tensors with
the same bits, float32 stays float32.  Imports the binding lazily so that the
oracle side never loads the HIP library.
"""
from __future__ import annotations

import numpy as np
import torch

from . import BF16, DecodeProblem, Problem


def to_torch(a: np.ndarray, io: str, device) -> torch.Tensor:
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def from_torch_bf16(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> uint16 bit patterns (host)."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def make_config(p, device, out_dtype=None, **kw):
    import gated_delta_rule_03_amd as kda
    io_t = torch.bfloat16 if p.io == BF16 else torch.float32
    return kda.Config(
        A_log=torch.from_numpy(np.ascontiguousarray(p.A_log, dtype=np.float32)).to(device),
        dt_bias=torch.from_numpy(np.ascontiguousarray(p.dt_bias, dtype=np.float32)).to(device),
        conv_w_q=to_torch(p.w_q, p.io, device), conv_w_k=to_torch(p.w_k, p.io, device),
        conv_w_v=to_torch(p.w_v, p.io, device), num_heads=p.H, head_k_dim=p.dk, head_v_dim=p.dv,
        io_dtype=io_t, out_dtype=out_dtype if out_dtype is not None else io_t, **kw)


def problem_to_device(p: Problem, device, out_dtype=None, **kw):
    """Returns (Config, dict of device tensors) for a packed problem.  The dict
    holds q, k, v, alpha, b (leading packed-token dim), cu_seqlens (int32),
    initial_state (fp32 or None) and conv_state (or None)."""
    cfg = make_config(p, device, out_dtype, **kw)
    t = {name: to_torch(getattr(p, name), p.io, device) for name in ("q", "k", "v", "alpha", "b")}
    t["cu_seqlens"] = torch.from_numpy(p.cu_seqlens.astype(np.int32)).to(device)
    t["initial_state"] = None if p.initial_state is None else \
        torch.from_numpy(np.ascontiguousarray(p.initial_state, dtype=np.float32)).to(device)
    t["conv_state"] = None if p.conv_state is None else to_torch(p.conv_state, p.io, device)
    return cfg, t


def decode_to_device(dp: DecodeProblem, device, out_dtype=None, **kw):
    """Returns (Config, state [N,H,dk,dv] fp32, conv_state) on the device."""
    cfg = make_config(dp, device, out_dtype, **kw)
    S = torch.from_numpy(np.ascontiguousarray(dp.state, dtype=np.float32)).to(device)
    cs = to_torch(dp.conv_state, dp.io, device)
    return cfg, S, cs


def tokens_to_device(tokens, io: str, device):
    return tuple(to_torch(a, io, device) for a in tokens)
