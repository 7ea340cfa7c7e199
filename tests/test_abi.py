"""The C ABI: header, exported symbols and host-side validation (CPU only).

Every call here fails validation (or is a no-op) before any launch, so no GPU
is needed; outputs passed in are host canaries that must stay untouched.
"""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


@pytest.fixture(scope="module")
def kda():
    lib_path = os.path.join(ROOT, "gated_delta_rule_03_amd", "libkda.so")
    if not os.path.exists(lib_path):
        pytest.fail("libkda.so is not built (run __graft_entry__.build())")
    import gated_delta_rule_03_amd as m
    return m


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_0-9]+)\s*\(", src)))


def test_header_compiles_as_c_and_cpp(tmp_path):
    for lang, std in (("c", "-std=c99"), ("c++", "-std=c++17")):
        subprocess.check_call(["gcc", "-fsyntax-only", "-Wall", "-Werror", std, "-x", lang, HEADER])


def test_every_declared_symbol_is_exported(kda):
    names = declared_functions()
    assert set(names) == set(kda.EXPORTED)
    for n in names:
        assert hasattr(kda.library(), n), n
    nm = subprocess.run(["nm", "-D", "--defined-only", kda.LIB_PATH], capture_output=True, text=True).stdout
    for n in names:
        assert re.search(rf"\bT {n}$", nm, flags=re.M), f"{n} not exported as a text symbol"


def test_version_and_status_strings(kda):
    assert kda.version() == 105
    for code, name in ((0, "KDA_OK"), (1, "KDA_ERR_INVALID_ARGUMENT"), (2, "KDA_ERR_UNSUPPORTED"),
                       (3, "KDA_ERR_WORKSPACE_TOO_SMALL"), (4, "KDA_ERR_HIP")):
        assert kda.status_string(code) == name


def test_struct_layout_matches_header(kda):
    # kda_config_t: 10 four-byte fields, then 6 pointers
    assert ctypes.sizeof(kda.KdaConfigC) == 10 * 4 + 6 * 8
    assert kda.KdaConfigC.A_log.offset == 40


class Canary:
    def __init__(self, n=64):
        self.a = np.full(n, 12345.0, dtype=np.float32)

    @property
    def ptr(self):
        return ctypes.c_void_p(self.a.ctypes.data)

    def untouched(self):
        return bool(np.all(self.a == 12345.0))


def make_cfg(kda, H=2, dk=16, dv=16, **kw):
    keep = [Canary() for _ in range(5)]
    c = kda.KdaConfigC()
    c.num_heads, c.head_k_dim, c.head_v_dim = H, dk, dv
    c.io_dtype, c.out_dtype = kda.KDA_BF16, kda.KDA_FP32
    c.scale, c.gate_lower_bound, c.l2norm_eps, c.chunk_size, c.flags = 1.0, -5.0, 1e-6, 64, 0
    c.A_log, c.dt_bias, c.conv_w_q, c.conv_w_k, c.conv_w_v = (k.a.ctypes.data for k in keep)
    for name, val in kw.items():
        setattr(c, name, val)
    return c, keep


def call_prefill(kda, cfg, B=1, T=8, null=(), ws_bytes=None):
    bufs = {n: Canary(1 << 12) for n in ("q", "k", "v", "alpha", "b", "S0", "cin", "o", "Sout", "cout", "ws")}
    ptr = {n: (None if n in null else b.ptr) for n, b in bufs.items()}
    need = kda.library().kda_prefill_workspace_bytes(ctypes.byref(cfg), B, T)
    st = kda.library().kda_prefill(ctypes.byref(cfg), B, T, ptr["q"], ptr["k"], ptr["v"], ptr["alpha"], ptr["b"],
                                   ptr["S0"], ptr["cin"], ptr["o"], ptr["Sout"], ptr["cout"], ptr["ws"],
                                   need if ws_bytes is None else ws_bytes, None)
    return st, bufs


@pytest.mark.parametrize("missing", ["q", "k", "v", "alpha", "b", "o", "ws"])
def test_null_required_pointer(kda, missing):
    cfg, _ = make_cfg(kda)
    st, bufs = call_prefill(kda, cfg, null=(missing,))
    assert st == kda.KDA_ERR_INVALID_ARGUMENT
    assert all(b.untouched() for b in bufs.values())


@pytest.mark.parametrize("field,val", [("head_k_dim", 48), ("head_v_dim", 32), ("io_dtype", 7),
                                       ("out_dtype", 3), ("chunk_size", 32), ("flags", 1 << 9),
                                       ("num_heads", 70000)])
def test_unsupported_configuration(kda, field, val):
    cfg, _ = make_cfg(kda, **{field: val})
    st, bufs = call_prefill(kda, cfg)
    assert st == kda.KDA_ERR_UNSUPPORTED
    assert all(b.untouched() for b in bufs.values())
    assert kda.library().kda_prefill_workspace_bytes(ctypes.byref(cfg), 1, 8) == 0


def test_invalid_sizes_and_parameters(kda):
    cfg, _ = make_cfg(kda)
    assert call_prefill(kda, cfg, B=-1)[0] == kda.KDA_ERR_INVALID_ARGUMENT
    assert call_prefill(kda, cfg, T=-5)[0] == kda.KDA_ERR_INVALID_ARGUMENT
    cfg2, _ = make_cfg(kda, A_log=None)
    assert call_prefill(kda, cfg2)[0] == kda.KDA_ERR_INVALID_ARGUMENT
    cfg3, _ = make_cfg(kda, conv_w_v=None)
    assert call_prefill(kda, cfg3)[0] == kda.KDA_ERR_INVALID_ARGUMENT
    cfg4, _ = make_cfg(kda, conv_w_v=None, flags=kda.FLAG_SKIP_CONV)
    assert call_prefill(kda, cfg4, null=("ws",))[0] == kda.KDA_ERR_INVALID_ARGUMENT   # only ws missing now
    cfg5, _ = make_cfg(kda, gate_lower_bound=float("nan"))
    assert call_prefill(kda, cfg5)[0] == kda.KDA_ERR_INVALID_ARGUMENT
    assert kda.library().kda_prefill(None, 1, 8, *([None] * 11), 0, None) == kda.KDA_ERR_INVALID_ARGUMENT


def test_workspace_too_small(kda):
    cfg, _ = make_cfg(kda)
    st, bufs = call_prefill(kda, cfg, ws_bytes=100)
    assert st == kda.KDA_ERR_WORKSPACE_TOO_SMALL
    assert all(b.untouched() for b in bufs.values())


def test_workspace_query_grows_with_size(kda):
    cfg, _ = make_cfg(kda, H=32, dk=128, dv=128)
    lib = kda.library()
    a = lib.kda_prefill_workspace_bytes(ctypes.byref(cfg), 1, 64)
    b = lib.kda_prefill_workspace_bytes(ctypes.byref(cfg), 1, 128)
    c = lib.kda_varlen_workspace_bytes(ctypes.byref(cfg), 2, 128)
    assert 0 < a < b <= c
    assert a % 256 == 0


def test_slab_workspace_query(kda):
    """The workspace of the chunked prefill in slabs: one slab's chunk table
    and records plus the carried state, independent of the batch's length;
    a workspace below one 64-token slab is refused before any launch."""
    cfg, _ = make_cfg(kda, H=32, dk=128, dv=128)
    lib = kda.library()
    q = lambda N, S: lib.kda_prefill_slab_workspace_bytes(ctypes.byref(cfg), N, S)
    assert q(1, 1) == q(1, 64) > 0 and q(1, 65) == q(1, 128) > q(1, 64)
    assert q(4, 8192) > q(2, 8192) > q(1, 8192) and q(4, 8192) % 256 == 0
    # the carried state [N][H][dk][dv] fp32 and N x S / 64 chunk records
    assert q(4, 8192) > 4 * 32 * 128 * 128 * 4 + 4 * 128 * 32 * 140 * 1024
    assert q(4, 8192) < lib.kda_prefill_workspace_bytes(ctypes.byref(cfg), 4, 32768) / 3
    assert q(0, 64) == 0 and q(1, 0) == 0
    cfg_rec, _ = make_cfg(kda, H=32, dk=128, dv=128, gate_lower_bound=float("-inf"))
    assert lib.kda_prefill_slab_workspace_bytes(ctypes.byref(cfg_rec), 1, 64) == 0   # no slabs for the recurrent form
    # below one slab: refused, nothing touched
    small, _ = make_cfg(kda)
    one = lib.kda_prefill_slab_workspace_bytes(ctypes.byref(small), 1, 64)
    assert 0 < one < lib.kda_prefill_workspace_bytes(ctypes.byref(small), 1, 4096)
    st, bufs = call_prefill(kda, small, B=1, T=4096, ws_bytes=one - 1)
    assert st == kda.KDA_ERR_WORKSPACE_TOO_SMALL and all(b.untouched() for b in bufs.values())


def test_workspace_of_the_recurrent_form(kda):
    """A gate lower bound below the chunked form's floor (-5.4) selects the
    recurrent form, whose workspace holds one fp32 record of 4 dk + 4 floats
    per (head, token) besides the chunk table."""
    lib = kda.library()
    H, D, B, T = 4, 64, 2, 300
    rec = H * B * T * (4 * D + 4) * 4
    for lb in (float("-inf"), -5.41, -30.0):
        cfg, _ = make_cfg(kda, H=H, dk=D, dv=D, gate_lower_bound=lb)
        a = lib.kda_prefill_workspace_bytes(ctypes.byref(cfg), B, T)
        v = lib.kda_varlen_workspace_bytes(ctypes.byref(cfg), B, B * T)
        assert rec < a < rec + 64 * 1024 and a % 256 == 0
        assert rec < v < rec + 64 * 1024
        st, bufs = call_prefill(kda, cfg, ws_bytes=100)   # validated as usual before any launch
        assert st == kda.KDA_ERR_WORKSPACE_TOO_SMALL and all(b.untouched() for b in bufs.values())
    # at the floor itself the chunked form's per-(chunk, head) records are sized
    cfg, _ = make_cfg(kda, H=H, dk=D, dv=D, gate_lower_bound=-5.4)
    chunked = lib.kda_prefill_workspace_bytes(ctypes.byref(cfg), B, T)
    assert chunked > 0 and chunked != lib.kda_prefill_workspace_bytes(
        ctypes.byref(make_cfg(kda, H=H, dk=D, dv=D, gate_lower_bound=-6.0)[0]), B, T)


def test_empty_batches_are_noops(kda):
    cfg, _ = make_cfg(kda)
    lib = kda.library()
    st, bufs = call_prefill(kda, cfg, B=0, null=("q", "k", "v", "alpha", "b", "o", "ws"))
    assert st == kda.KDA_OK and all(b.untouched() for b in bufs.values())
    assert lib.kda_varlen_prefill(ctypes.byref(cfg), 0, 0, None, *([None] * 10), None, 0, None) == kda.KDA_OK
    assert lib.kda_decode_step(ctypes.byref(cfg), 0, *([None] * 8), None) == kda.KDA_OK


def test_varlen_and_decode_validation(kda):
    cfg, _ = make_cfg(kda)
    lib = kda.library()
    c = Canary()
    p = c.ptr
    # varlen: missing cu_seqlens
    assert lib.kda_varlen_prefill(ctypes.byref(cfg), 2, 16, None, p, p, p, p, p, None, None, p, None, None,
                                  p, 1 << 30, None) == kda.KDA_ERR_INVALID_ARGUMENT
    assert lib.kda_varlen_prefill(ctypes.byref(cfg), -1, 16, p, p, p, p, p, p, None, None, p, None, None,
                                  p, 1 << 30, None) == kda.KDA_ERR_INVALID_ARGUMENT
    assert lib.kda_varlen_prefill(ctypes.byref(cfg), 2, 16, p, p, p, p, p, p, None, None, p, None, None,
                                  p, 10, None) == kda.KDA_ERR_WORKSPACE_TOO_SMALL
    # decode: state and conv history are required
    assert lib.kda_decode_step(ctypes.byref(cfg), 4, p, p, p, p, p, None, p, p, None) == kda.KDA_ERR_INVALID_ARGUMENT
    assert lib.kda_decode_step(ctypes.byref(cfg), 4, p, p, p, p, p, p, None, p, None) == kda.KDA_ERR_INVALID_ARGUMENT
    assert lib.kda_decode_step(ctypes.byref(cfg), -2, p, p, p, p, p, p, p, p, None) == kda.KDA_ERR_INVALID_ARGUMENT
    assert c.untouched()


def test_output_gate_validation(kda):
    lib = kda.library()
    c = Canary(1 << 12)
    p = c.ptr
    cfg, _ = make_cfg(kda, H=4, dk=64, dv=64)
    og = lambda cfg_, n, o, g, w, eps, y: lib.kda_output_gate(
        None if cfg_ is None else ctypes.byref(cfg_), n, o, g, w, eps, y, None)
    assert og(None, 4, p, p, p, 1e-6, p) == kda.KDA_ERR_INVALID_ARGUMENT
    assert og(cfg, -1, p, p, p, 1e-6, p) == kda.KDA_ERR_INVALID_ARGUMENT
    assert og(cfg, 4, p, p, p, float("nan"), p) == kda.KDA_ERR_INVALID_ARGUMENT
    assert og(cfg, 4, p, p, p, -1e-3, p) == kda.KDA_ERR_INVALID_ARGUMENT
    for missing in range(4):
        args = [p, p, p, p]
        args[missing] = None
        assert og(cfg, 4, args[0], args[1], args[2], 1e-6, args[3]) == kda.KDA_ERR_INVALID_ARGUMENT
    assert og(make_cfg(kda, H=4, dk=64, dv=48)[0], 4, p, p, p, 1e-6, p) == kda.KDA_ERR_UNSUPPORTED
    assert og(make_cfg(kda, H=4, dk=64, dv=64, out_dtype=5)[0], 4, p, p, p, 1e-6, p) == kda.KDA_ERR_UNSUPPORTED
    # the epilogue does not need the prefill's parameters, and 0 tokens is a no-op
    assert og(make_cfg(kda, H=4, dk=64, dv=64, A_log=None, conv_w_q=None)[0], 0, None, None, None, 1e-6,
              None) == kda.KDA_OK
    assert c.untouched()


def test_decode_multi_validation(kda):
    lib = kda.library()
    c = Canary(1 << 12)
    p = c.ptr
    cfg, _ = make_cfg(kda)
    dm = lambda cfg_, N, K, ptrs: lib.kda_decode_multi(ctypes.byref(cfg_), N, K, None, *ptrs, None, None)
    full = [p] * 8
    assert dm(cfg, 2, 0, full) == kda.KDA_ERR_INVALID_ARGUMENT
    assert dm(cfg, -1, 2, full) == kda.KDA_ERR_INVALID_ARGUMENT
    assert dm(cfg, 2, 65, full) == kda.KDA_ERR_UNSUPPORTED
    for missing in range(8):
        ptrs = list(full)
        ptrs[missing] = None
        assert dm(cfg, 2, 3, ptrs) == kda.KDA_ERR_INVALID_ARGUMENT
    assert dm(cfg, 0, 3, [None] * 8) == kda.KDA_OK
    assert dm(make_cfg(kda, dv=32)[0], 2, 3, full) == kda.KDA_ERR_UNSUPPORTED
    assert c.untouched()


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU; asked for more it exits with a message
    before touching any device."""
    r = subprocess.run([os.sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_gated_decode_validation(kda):
    """The fused-epilogue decode calls validate the epilogue's arguments (gate,
    weight, eps) as well as the decode's, before any launch."""
    lib = kda.library()
    c = Canary(1 << 12)
    p = c.ptr
    cfg, _ = make_cfg(kda)
    ds = lambda N, gate, w, eps, ptrs=(p,) * 7: lib.kda_decode_step_gated(
        ctypes.byref(cfg), N, *ptrs, gate, w, eps, p, None)
    assert ds(2, None, p, 1e-6) == kda.KDA_ERR_INVALID_ARGUMENT
    assert ds(2, p, None, 1e-6) == kda.KDA_ERR_INVALID_ARGUMENT
    assert ds(2, p, p, float("nan")) == kda.KDA_ERR_INVALID_ARGUMENT
    assert ds(2, p, p, -1.0) == kda.KDA_ERR_INVALID_ARGUMENT
    assert ds(2, p, p, 1e-6, (p, p, p, p, p, None, p)) == kda.KDA_ERR_INVALID_ARGUMENT   # no state
    assert ds(0, None, None, 1e-6) == kda.KDA_OK
    dm = lambda N, K, gate, w, eps: lib.kda_decode_multi_gated(ctypes.byref(cfg), N, K, None, p, p, p, p, p, p, p,
                                                              gate, w, eps, p, None, None)
    assert dm(2, 3, None, p, 1e-6) == kda.KDA_ERR_INVALID_ARGUMENT
    assert dm(2, 3, p, None, 1e-6) == kda.KDA_ERR_INVALID_ARGUMENT
    assert dm(2, 3, p, p, -0.5) == kda.KDA_ERR_INVALID_ARGUMENT
    assert dm(2, 65, p, p, 1e-6) == kda.KDA_ERR_UNSUPPORTED
    assert dm(0, 3, None, None, 1e-6) == kda.KDA_OK
    assert c.untouched()


def test_backward_validation(kda):
    """The backward refuses what it does not handle (the recurrent form's
    gates, test hooks other than beta x2) and checks its pointers and
    workspace before any launch."""
    lib = kda.library()
    c = Canary(1 << 12)
    p = c.ptr
    bw = lambda cfg_, N, T, ptrs, ws_bytes=1 << 30: lib.kda_varlen_backward(
        ctypes.byref(cfg_), N, T, *ptrs, p, ws_bytes, None)
    full = [p] * 22                            # cu_seqlens .. dA_log; the workspace is added by bw
    cfg, _ = make_cfg(kda)
    assert bw(make_cfg(kda, gate_lower_bound=float("-inf"))[0], 2, 16, full) == kda.KDA_ERR_UNSUPPORTED
    assert bw(make_cfg(kda, flags=kda.FLAG_RAW_GATE)[0], 2, 16, full) == kda.KDA_ERR_UNSUPPORTED
    assert bw(make_cfg(kda, flags=kda.FLAG_SKIP_CONV)[0], 2, 16, full) == kda.KDA_ERR_UNSUPPORTED
    assert bw(cfg, -1, 16, full) == kda.KDA_ERR_INVALID_ARGUMENT
    for missing in (0, 1, 8, 10, 17, 21):      # cu_seqlens, q, d_o, dq, dw_q, dA_log
        ptrs = list(full)
        ptrs[missing] = None
        assert bw(cfg, 2, 16, ptrs) == kda.KDA_ERR_INVALID_ARGUMENT, missing
    assert bw(cfg, 2, 16, full, ws_bytes=100) == kda.KDA_ERR_WORKSPACE_TOO_SMALL
    assert bw(cfg, 0, 0, [None] * 22) == kda.KDA_OK
    assert lib.kda_varlen_backward_workspace_bytes(ctypes.byref(cfg), 2, 16) > 0
    assert lib.kda_varlen_backward_workspace_bytes(
        ctypes.byref(make_cfg(kda, flags=kda.FLAG_RAW_BETA)[0]), 2, 16) == 0
    assert c.untouched()
