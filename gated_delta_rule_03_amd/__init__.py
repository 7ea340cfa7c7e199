"""Python binding of the MI355X KDA library (``libkda.so``, C ABI in include/kda.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  PyTorch provides device memory and the stream.
The library must have been built (``python gated_delta_rule_03_amd/build.py``);
importing the binding without it raises ImportError -- there is no fallback.

Entry points (same names as the C ABI):
  kda_prefill(cfg, q, k, v, alpha, b, ...)          B equal-length sequences
  kda_varlen_prefill(cfg, cu_seqlens, q, ...)       packed sequences
  kda_decode_step(cfg, q, k, v, alpha, b, state, conv_state, o=None)
  kda_decode_multi(cfg, q, ..., state_pool, conv_pool, slots=, n_commit=)
  kda_decode_step_gated / kda_decode_multi_gated   the same, output epilogue fused
  kda_output_gate(cfg, o, gate, o_norm_weight)     the output epilogue alone
  kda_prefill_workspace_bytes / kda_varlen_workspace_bytes / kda_prefill_slab_workspace_bytes
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass, field
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkda.so")

KDA_OK = 0
KDA_ERR_INVALID_ARGUMENT = 1
KDA_ERR_UNSUPPORTED = 2
KDA_ERR_WORKSPACE_TOO_SMALL = 3
KDA_ERR_HIP = 4

KDA_BF16 = 0
KDA_FP32 = 1

FLAG_SKIP_CONV = 1 << 0
FLAG_SKIP_L2NORM = 1 << 1
FLAG_RAW_GATE = 1 << 2
FLAG_RAW_BETA = 1 << 3
FLAG_BETA_X2 = 1 << 4

STAGES = ("chunk_table", "chunk_prep", "chunk_scan", "conv_state", "decode", "output_gate", "backward")
NUM_STAGES = len(STAGES)

EXPORTED = ("kda_version", "kda_status_string", "kda_prefill_workspace_bytes", "kda_prefill",
            "kda_varlen_workspace_bytes", "kda_varlen_prefill", "kda_decode_step", "kda_decode_multi",
            "kda_decode_step_gated", "kda_decode_multi_gated", "kda_output_gate", "kda_varlen_prefill_noalloc",
            "kda_varlen_backward_workspace_bytes", "kda_varlen_backward", "kda_prefill_slab_workspace_bytes")

# the fixed scratch behind kda_varlen_prefill_noalloc (KDA_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 256 << 20


class KdaError(RuntimeError):
    def __init__(self, status: int, name: str):
        super().__init__(f"{name} returned {status_string(status)} ({status})")
        self.status = status


class KdaConfigC(ctypes.Structure):
    _fields_ = [
        ("num_heads", ctypes.c_int32),
        ("head_k_dim", ctypes.c_int32),
        ("head_v_dim", ctypes.c_int32),
        ("io_dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("gate_lower_bound", ctypes.c_float),
        ("l2norm_eps", ctypes.c_float),
        ("chunk_size", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
        ("A_log", ctypes.c_void_p),
        ("dt_bias", ctypes.c_void_p),
        ("conv_w_q", ctypes.c_void_p),
        ("conv_w_k", ctypes.c_void_p),
        ("conv_w_v", ctypes.c_void_p),
        ("stage_events", ctypes.c_void_p),
    ]


def _load_library():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"KDA HIP library not built: {LIB_PATH} is missing "
                          "(run `python gated_delta_rule_03_amd/build.py`)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    cfgp = ctypes.POINTER(KdaConfigC)
    lib.kda_version.restype = i32
    lib.kda_version.argtypes = []
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_status_string.argtypes = [ctypes.c_int]
    lib.kda_prefill_workspace_bytes.restype = sz
    lib.kda_prefill_workspace_bytes.argtypes = [cfgp, i32, i32]
    lib.kda_varlen_workspace_bytes.restype = sz
    lib.kda_varlen_workspace_bytes.argtypes = [cfgp, i32, i32]
    lib.kda_prefill_slab_workspace_bytes.restype = sz
    lib.kda_prefill_slab_workspace_bytes.argtypes = [cfgp, i32, i32]
    lib.kda_prefill.restype = ctypes.c_int
    lib.kda_prefill.argtypes = [cfgp, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.kda_varlen_prefill.restype = ctypes.c_int
    lib.kda_varlen_prefill.argtypes = [cfgp, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.kda_varlen_prefill_noalloc.restype = ctypes.c_int
    lib.kda_varlen_prefill_noalloc.argtypes = [cfgp, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.kda_varlen_backward_workspace_bytes.restype = sz
    lib.kda_varlen_backward_workspace_bytes.argtypes = [cfgp, i32, i32]
    lib.kda_varlen_backward.restype = ctypes.c_int
    lib.kda_varlen_backward.argtypes = [cfgp, i32, i32] + [vp] * 23 + [sz, vp]
    lib.kda_decode_step.restype = ctypes.c_int
    lib.kda_decode_step.argtypes = [cfgp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.kda_decode_multi.restype = ctypes.c_int
    lib.kda_decode_multi.argtypes = [cfgp, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.kda_decode_step_gated.restype = ctypes.c_int
    lib.kda_decode_step_gated.argtypes = [cfgp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp]
    lib.kda_decode_multi_gated.restype = ctypes.c_int
    lib.kda_decode_multi_gated.argtypes = [cfgp, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                           ctypes.c_float, vp, vp, vp]
    lib.kda_output_gate.restype = ctypes.c_int
    lib.kda_output_gate.argtypes = [cfgp, ctypes.c_int64, vp, vp, vp, ctypes.c_float, vp, vp]
    return lib


_lib = _load_library()


def library():
    """The loaded ctypes library handle."""
    return _lib


def status_string(status: int) -> str:
    return _lib.kda_status_string(int(status)).decode()


def version() -> int:
    return int(_lib.kda_version())


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return KDA_BF16
    if dt == torch.float32:
        return KDA_FP32
    raise ValueError(f"unsupported dtype {dt}")


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


@dataclass
class Config:
    """Per-layer parameters and numerics of the KDA core (device tensors)."""
    A_log: torch.Tensor          # [H] fp32
    dt_bias: torch.Tensor        # [H*dk] fp32
    conv_w_q: torch.Tensor       # [H*dk, 4] io dtype
    conv_w_k: torch.Tensor       # [H*dk, 4]
    conv_w_v: torch.Tensor       # [H*dv, 4]
    num_heads: int
    head_k_dim: int
    head_v_dim: int
    io_dtype: torch.dtype = torch.bfloat16
    out_dtype: torch.dtype = torch.bfloat16
    scale: float = 1.0
    gate_lower_bound: float = -5.0
    l2norm_eps: float = 1e-6
    chunk_size: int = 64
    flags: int = 0
    stage_events: Optional[object] = None   # ctypes array of 2*NUM_STAGES hipEvent_t, or None
    _c: Optional[KdaConfigC] = field(default=None, repr=False)

    def c_struct(self) -> KdaConfigC:
        c = KdaConfigC()
        c.num_heads = self.num_heads
        c.head_k_dim = self.head_k_dim
        c.head_v_dim = self.head_v_dim
        c.io_dtype = _dtype_code(self.io_dtype)
        c.out_dtype = _dtype_code(self.out_dtype)
        c.scale = self.scale
        c.gate_lower_bound = self.gate_lower_bound
        c.l2norm_eps = self.l2norm_eps
        c.chunk_size = self.chunk_size
        c.flags = self.flags
        for name in ("A_log", "dt_bias", "conv_w_q", "conv_w_k", "conv_w_v"):
            t = getattr(self, name)
            setattr(c, name, None if t is None else t.data_ptr())
        c.stage_events = None if self.stage_events is None else ctypes.cast(self.stage_events, ctypes.c_void_p)
        self._c = c   # keep alive
        return c

    @property
    def ctot(self) -> int:
        return self.num_heads * (2 * self.head_k_dim + self.head_v_dim)


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(status: int, name: str):
    if status != KDA_OK:
        raise KdaError(status, name)


def kda_prefill_workspace_bytes(cfg: Config, B: int, T: int) -> int:
    return int(_lib.kda_prefill_workspace_bytes(ctypes.byref(cfg.c_struct()), B, T))


def kda_varlen_workspace_bytes(cfg: Config, N: int, total_T: int) -> int:
    return int(_lib.kda_varlen_workspace_bytes(ctypes.byref(cfg.c_struct()), N, total_T))


def kda_prefill_slab_workspace_bytes(cfg: Config, N: int, slab_tokens: int) -> int:
    """Workspace for the chunked prefill of N sequences run in slabs of
    slab_tokens positions; passing a workspace of this size (smaller than
    the one-pass size) to kda_prefill / kda_varlen_prefill runs them in slabs."""
    return int(_lib.kda_prefill_slab_workspace_bytes(ctypes.byref(cfg.c_struct()), N, slab_tokens))


def _workspace(nbytes: int, device, workspace: Optional[torch.Tensor]) -> torch.Tensor:
    if workspace is not None:
        return workspace
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def kda_prefill(cfg: Config, q, k, v, alpha, b, initial_state=None, conv_state_in=None, *,
                o=None, final_state=None, conv_state_out=None, workspace=None, stream=None):
    """q, k [B, T, H*dk]; v [B, T, H*dv]; alpha [B, T, H, dk]; b [B, T, H].
    Returns (o [B, T, H, dv], final_state or None, conv_state_out or None)."""
    B, T = q.shape[0], q.shape[1]
    H, dv = cfg.num_heads, cfg.head_v_dim
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=cfg.out_dtype, device=q.device)
    nbytes = kda_prefill_workspace_bytes(cfg, B, T)
    ws = _workspace(nbytes, q.device, workspace)
    st = _lib.kda_prefill(ctypes.byref(cfg.c_struct()), B, T, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(b),
                          _ptr(initial_state), _ptr(conv_state_in), _ptr(o), _ptr(final_state),
                          _ptr(conv_state_out), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "kda_prefill")
    return o, final_state, conv_state_out


def kda_varlen_prefill(cfg: Config, cu_seqlens, q, k, v, alpha, b, initial_state=None, conv_state_in=None, *,
                       o=None, final_state=None, conv_state_out=None, workspace=None, stream=None):
    """cu_seqlens int32 [N+1] on the device; q, k [total_T, H*dk]; v [total_T, H*dv];
    alpha [total_T, H, dk]; b [total_T, H].  Returns (o, final_state, conv_state_out)."""
    N = cu_seqlens.numel() - 1
    total = q.shape[0]
    H, dv = cfg.num_heads, cfg.head_v_dim
    if cu_seqlens.dtype != torch.int32:
        raise ValueError("cu_seqlens must be int32")
    if o is None:
        o = torch.empty((total, H, dv), dtype=cfg.out_dtype, device=q.device)
    nbytes = kda_varlen_workspace_bytes(cfg, N, total)
    ws = _workspace(nbytes, q.device, workspace)
    st = _lib.kda_varlen_prefill(ctypes.byref(cfg.c_struct()), N, total, _ptr(cu_seqlens), _ptr(q), _ptr(k),
                                 _ptr(v), _ptr(alpha), _ptr(b), _ptr(initial_state), _ptr(conv_state_in),
                                 _ptr(o), _ptr(final_state), _ptr(conv_state_out), _ptr(ws),
                                 ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "kda_varlen_prefill")
    return o, final_state, conv_state_out


def kda_varlen_prefill_noalloc(cfg: Config, cu_seqlens, q, k, v, alpha, b, initial_state=None, conv_state_in=None,
                               *, o, final_state=None, conv_state_out=None, stream=None):
    """kda_varlen_prefill on the library's fixed per-GPU scratch: no workspace
    argument and no allocation (o must be passed in).  Batches whose
    workspace exceeds NOALLOC_SCRATCH_BYTES raise KdaError
    (KDA_ERR_WORKSPACE_TOO_SMALL).  Returns (o, final_state, conv_state_out)."""
    N = cu_seqlens.numel() - 1
    if cu_seqlens.dtype != torch.int32:
        raise ValueError("cu_seqlens must be int32")
    st = _lib.kda_varlen_prefill_noalloc(ctypes.byref(cfg.c_struct()), N, q.shape[0], _ptr(cu_seqlens), _ptr(q),
                                         _ptr(k), _ptr(v), _ptr(alpha), _ptr(b), _ptr(initial_state),
                                         _ptr(conv_state_in), _ptr(o), _ptr(final_state), _ptr(conv_state_out),
                                         _stream(stream))
    _check(st, "kda_varlen_prefill_noalloc")
    return o, final_state, conv_state_out


def kda_varlen_backward_workspace_bytes(cfg: Config, N: int, total_T: int) -> int:
    return int(_lib.kda_varlen_backward_workspace_bytes(ctypes.byref(cfg.c_struct()), N, total_T))


def kda_varlen_backward(cfg: Config, cu_seqlens, q, k, v, alpha, b, initial_state=None, conv_state_in=None, *,
                        d_o, d_final_state=None, want_initial_state=True, want_conv_state=True, workspace=None,
                        stream=None):
    """Gradient of a loss through o and the final state of kda_varlen_prefill
    with respect to every input and parameter.  d_o [total_T, H, dv] (out
    dtype), d_final_state [N, H, dk, dv] fp32 or None.  Returns a dict of
    fp32 tensors: dq, dk [total_T, H*dk], dv [total_T, H*dv], dalpha
    [total_T, H, dk], db [total_T, H], dS0 [N, H, dk, dv] (or None), dconv
    [N, 3, Ctot] (or None), dw_q, dw_k [H*dk, 4], dw_v [H*dv, 4], ddt_bias
    [H*dk], dA_log [H]."""
    N = cu_seqlens.numel() - 1
    total = q.shape[0]
    H, dk, dv = cfg.num_heads, cfg.head_k_dim, cfg.head_v_dim
    if cu_seqlens.dtype != torch.int32:
        raise ValueError("cu_seqlens must be int32")
    dev = q.device
    f = lambda *shape: torch.empty(shape, dtype=torch.float32, device=dev)
    g = {"dq": f(total, H * dk), "dk": f(total, H * dk), "dv": f(total, H * dv), "dalpha": f(total, H, dk),
         "db": f(total, H), "dS0": f(N, H, dk, dv) if want_initial_state else None,
         "dconv": f(N, 3, cfg.ctot) if want_conv_state else None, "dw_q": f(H * dk, 4), "dw_k": f(H * dk, 4),
         "dw_v": f(H * dv, 4), "ddt_bias": f(H * dk), "dA_log": f(H)}
    nbytes = kda_varlen_backward_workspace_bytes(cfg, N, total)
    ws = _workspace(nbytes, dev, workspace)
    st = _lib.kda_varlen_backward(ctypes.byref(cfg.c_struct()), N, total, _ptr(cu_seqlens), _ptr(q), _ptr(k),
                                  _ptr(v), _ptr(alpha), _ptr(b), _ptr(initial_state), _ptr(conv_state_in),
                                  _ptr(d_o), _ptr(d_final_state), _ptr(g["dq"]), _ptr(g["dk"]), _ptr(g["dv"]),
                                  _ptr(g["dalpha"]), _ptr(g["db"]), _ptr(g["dS0"]), _ptr(g["dconv"]),
                                  _ptr(g["dw_q"]), _ptr(g["dw_k"]), _ptr(g["dw_v"]), _ptr(g["ddt_bias"]),
                                  _ptr(g["dA_log"]), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "kda_varlen_backward")
    return g


def kda_decode_step(cfg: Config, q, k, v, alpha, b, state, conv_state, *, o=None, stream=None):
    """One token for each of N sequences: q, k [N, H*dk]; v [N, H*dv];
    alpha [N, H, dk]; b [N, H]; state [N, H, dk, dv] fp32 and conv_state
    [N, 3, Ctot] are updated in place.  Returns o [N, H, dv]."""
    N = q.shape[0]
    if o is None:
        o = torch.empty((N, cfg.num_heads, cfg.head_v_dim), dtype=cfg.out_dtype, device=q.device)
    st = _lib.kda_decode_step(ctypes.byref(cfg.c_struct()), N, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(b),
                              _ptr(state), _ptr(conv_state), _ptr(o), _stream(stream))
    _check(st, "kda_decode_step")
    return o


def kda_decode_multi(cfg: Config, q, k, v, alpha, b, state_pool, conv_pool, *, slots=None, n_commit=None, o=None,
                     stream=None):
    """K tokens for each of N sequences through state / conv-history pools:
    q, k [N, K, H*dk]; v [N, K, H*dv]; alpha [N, K, H, dk]; b [N, K, H];
    state_pool [P, H, dk, dv] fp32 and conv_pool [P, 3, Ctot] are updated in
    place (rows slots[n], after the first n_commit[n] tokens).  slots and
    n_commit are int32 device tensors [N] or None.  Returns o [N, K, H, dv]."""
    N, K = q.shape[0], q.shape[1]
    for t in (slots, n_commit):
        if t is not None and (t.dtype != torch.int32 or t.numel() != N):
            raise ValueError("slots and n_commit must be int32 tensors of N entries")
    if o is None:
        o = torch.empty((N, K, cfg.num_heads, cfg.head_v_dim), dtype=cfg.out_dtype, device=q.device)
    st = _lib.kda_decode_multi(ctypes.byref(cfg.c_struct()), N, K, _ptr(slots), _ptr(q), _ptr(k), _ptr(v),
                               _ptr(alpha), _ptr(b), _ptr(state_pool), _ptr(conv_pool), _ptr(o), _ptr(n_commit),
                               _stream(stream))
    _check(st, "kda_decode_multi")
    return o


def kda_decode_step_gated(cfg: Config, q, k, v, alpha, b, state, conv_state, gate, o_norm_weight,
                          eps: float = 1e-6, *, y=None, stream=None):
    """kda_decode_step with the output epilogue fused: gate [N, H, dv] (io
    dtype), o_norm_weight [dv] fp32.  Returns y [N, H, dv] (out dtype) =
    o / sqrt(mean(o^2) + eps) * o_norm_weight * sigmoid(gate) per row."""
    N = q.shape[0]
    if y is None:
        y = torch.empty((N, cfg.num_heads, cfg.head_v_dim), dtype=cfg.out_dtype, device=q.device)
    st = _lib.kda_decode_step_gated(ctypes.byref(cfg.c_struct()), N, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                    _ptr(b), _ptr(state), _ptr(conv_state), _ptr(gate), _ptr(o_norm_weight),
                                    float(eps), _ptr(y), _stream(stream))
    _check(st, "kda_decode_step_gated")
    return y


def kda_decode_multi_gated(cfg: Config, q, k, v, alpha, b, state_pool, conv_pool, gate, o_norm_weight,
                           eps: float = 1e-6, *, slots=None, n_commit=None, y=None, stream=None):
    """kda_decode_multi with the output epilogue fused: gate [N, K, H, dv]
    (io dtype), o_norm_weight [dv] fp32.  Returns y [N, K, H, dv]."""
    N, K = q.shape[0], q.shape[1]
    for t in (slots, n_commit):
        if t is not None and (t.dtype != torch.int32 or t.numel() != N):
            raise ValueError("slots and n_commit must be int32 tensors of N entries")
    if y is None:
        y = torch.empty((N, K, cfg.num_heads, cfg.head_v_dim), dtype=cfg.out_dtype, device=q.device)
    st = _lib.kda_decode_multi_gated(ctypes.byref(cfg.c_struct()), N, K, _ptr(slots), _ptr(q), _ptr(k), _ptr(v),
                                     _ptr(alpha), _ptr(b), _ptr(state_pool), _ptr(conv_pool), _ptr(gate),
                                     _ptr(o_norm_weight), float(eps), _ptr(y), _ptr(n_commit), _stream(stream))
    _check(st, "kda_decode_multi_gated")
    return y


def kda_output_gate(cfg: Config, o, gate, o_norm_weight, eps: float = 1e-6, *, y=None, stream=None):
    """The output epilogue: y = o / sqrt(mean(o^2) + eps) * o_norm_weight * sigmoid(gate)
    per (token, head) row.  o [..., H, dv] out_dtype; gate the same shape in
    io_dtype; o_norm_weight [dv] fp32.  y defaults to a new tensor; pass
    y=o to work in place.  Returns y."""
    if o.shape != gate.shape or o.shape[-1] != cfg.head_v_dim or o.shape[-2] != cfg.num_heads:
        raise ValueError("o and gate must both be [..., num_heads, head_v_dim]")
    n_tokens = o.numel() // (cfg.num_heads * cfg.head_v_dim) if o.numel() else 0
    if y is None:
        y = torch.empty_like(o)
    st = _lib.kda_output_gate(ctypes.byref(cfg.c_struct()), n_tokens, _ptr(o), _ptr(gate), _ptr(o_norm_weight),
                              float(eps), _ptr(y), _stream(stream))
    _check(st, "kda_output_gate")
    return y
