#!/usr/bin/env python3
"""Benchmark of the MI355X KDA core.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Headline: chunked prefill of B=4 sequences x T=32768 tokens, H=32 heads,
dk=dv=128, bf16 inputs, fp32 state with a random initial state (the
long-context prefill workload).  A step is one kda_prefill call over the whole
batch; inputs are resident in HBM before the timed region.  The same run also
times the single-token decode step (256 sequences, 128 steps) and the varlen
packed prefill (8 sequences, 262144 tokens), reported as sub-objects.

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

H, D = 32, 128
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
FP32_VALU_PEAK_TFLOPS = 157.3  # MI355X fp32 vector
BF16_MFMA_PEAK_TFLOPS = 2500.0 # MI355X dense bf16 matrix
CHUNK = 64

# Algorithmic work of the chunked prefill per token-head (d = 128):
#   minimum HBM bytes: raw bf16 q, k, v (3 x 2d) and alpha (2d) and b (2) in,
#   bf16 o (2d) out = 1282 B; per (sequence, head) the fp32 state in and out
#   and per sequence the conv history (3 raw inputs per channel) in and out.
#   FLOPs of the chunked form: 2C(3dk + 2dv) + 6 dk dv + 2C^2/3 = 182,955, all
#   matrix products except the C^2 solve.  The matrix cores issue every
#   product three times (two bf16 pieces per operand: hi*hi, hi*lo, lo*hi).
BYTES_PER_TOKEN_HEAD = 4 * 2 * D + 2 + 2 * D
FLOPS_PER_TOKEN_HEAD = 2 * CHUNK * (3 * D + 2 * D) + 6 * D * D + 2 * CHUNK * CHUNK / 3.0
MFMA_PASSES = 3


def prefill_alg_bytes(B, T, conv_in=False):
    """Minimum HBM bytes of one prefill call of B sequences x T tokens."""
    ctot = H * 3 * D
    return (B * T * H * BYTES_PER_TOKEN_HEAD + 2 * B * H * D * D * 4
            + (2 if conv_in else 1) * B * 3 * ctot * 2)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """hipEvent_t handles through the HIP runtime already loaded by torch."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        e = ctypes.c_void_p()
        assert self.lib.hipEventCreate(ctypes.byref(e)) == 0
        return e

    def record(self, e, stream_ptr):
        assert self.lib.hipEventRecord(e, ctypes.c_void_p(stream_ptr)) == 0

    def ms(self, a, b):
        out = ctypes.c_float()
        rc = self.lib.hipEventElapsedTime(ctypes.byref(out), a, b)
        return float(out.value) if rc == 0 else float("nan")

    def stage_array(self, stages):
        """A (2*NUM_STAGES) array of events with entries only for `stages`."""
        import gated_delta_rule_03_amd as kda
        arr = (ctypes.c_void_p * (2 * kda.NUM_STAGES))()
        for s in stages:
            arr[2 * s] = self.create()
            arr[2 * s + 1] = self.create()
        return arr


def stage_means(ev, arrays, stages):
    out = {}
    for s in stages:
        vals = [ev.ms(a[2 * s], a[2 * s + 1]) for a in arrays]
        out[s] = sum(vals) / len(vals)
    return out


def bench_prefill(kda, torch, ev, steps, warmup):
    from kda_inputs import BF16
    from kda_inputs.device_gen import DeviceProblem
    dev = torch.device("cuda:0")
    B, T = 4, 32768
    t0 = time.time()
    dp = DeviceProblem(3, [T] * B, H, D, D, BF16, dev, state_seqs=list(range(B)))
    log(f"[bench] prefill inputs generated on device in {time.time() - t0:.1f}s")
    cfg = dp.config(out_dtype=torch.bfloat16)
    tz = dp.tensors
    q, k, v = (tz[n].view(B, T, -1) for n in ("q", "k", "v"))
    alpha, b = tz["alpha"].view(B, T, H, D), tz["b"].view(B, T, H)
    o = torch.empty((B, T, H, D), dtype=torch.bfloat16, device=dev)
    S_out = torch.empty((B, H, D, D), dtype=torch.float32, device=dev)
    cs_out = torch.empty((B, 3, dp.ctot), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(kda.kda_prefill_workspace_bytes(cfg, B, T), dtype=torch.uint8, device=dev)
    log(f"[bench] prefill workspace {ws.numel() / 2**30:.2f} GiB")
    stream = torch.cuda.current_stream()

    def step():
        kda.kda_prefill(cfg, q, k, v, alpha, b, tz["initial_state"], tz["conv_state"], o=o, final_state=S_out,
                        conv_state_out=cs_out, workspace=ws, stream=stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stages = [kda.STAGES.index(n) for n in ("chunk_table", "chunk_prep", "chunk_scan", "conv_state")]
    arrays = [ev.stage_array(stages) for _ in range(steps)]
    e0, e1 = ev.create(), ev.create()
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev.record(e0, stream.cuda_stream)
    for i in range(steps):
        cfg.stage_events = arrays[i]
        step()
    ev.record(e1, stream.cuda_stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    cfg.stage_events = None
    gpu_ms = ev.ms(e0, e1)
    per_stage = stage_means(ev, arrays, stages)
    log(f"[bench] prefill: {steps} steps, wall {wall * 1e3:.1f} ms, events {gpu_ms:.1f} ms; stage ms " +
        ", ".join(f"{kda.STAGES[s]}={per_stage[s]:.3f}" for s in stages))
    return dp, wall, gpu_ms, per_stage


def roofline_for(kda, per_stage, ms_step, B, T):
    """Roofline object of the prefill: the path's algorithmic bytes (1282 B
    per token-head plus state and conv history) over the mean duration of the
    stage that takes longest, against 8 TB/s.  Beside it: the matrix-core
    fraction of the whole step (algorithmic FLOPs, and as issued with the
    three compensated passes) against the dense bf16 peak, and the HBM bytes
    the counters measured for that kernel and for the whole path."""
    name_of = {i: n for i, n in enumerate(kda.STAGES)}
    s_dom = max(per_stage, key=per_stage.get)
    name = name_of[s_dom]
    ms = per_stage[s_dom]
    nbytes = prefill_alg_bytes(B, T)
    flops = FLOPS_PER_TOKEN_HEAD * B * T * H
    gbs = nbytes / (ms * 1e-3) / 1e9
    traffic = measured_traffic(name)
    path_traffic = [measured_traffic(n) for n in ("chunk_prep", "chunk_scan")]
    path_traffic = None if None in path_traffic else sum(path_traffic)
    tf_step = flops / (ms_step * 1e-3) / 1e12
    return {"kernel": name, "bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
            "avg_ms": round(ms, 4), "bytes_per_launch": nbytes,
            "bytes_basis": "algorithmic: 1282 B per token-head (bf16 q, k, v, alpha, b in; bf16 o out) "
                           "+ fp32 state in/out + conv history out",
            "traffic_over_algorithmic": None if traffic is None else round(traffic / nbytes, 3),
            "path_traffic": path_traffic,
            "path_traffic_over_algorithmic": None if path_traffic is None else round(path_traffic / nbytes, 3),
            "flops_per_step": flops,
            "mfma_frac": round(tf_step / BF16_MFMA_PEAK_TFLOPS, 4),
            "mfma_frac_issued": round(MFMA_PASSES * tf_step / BF16_MFMA_PEAK_TFLOPS, 4),
            "mfma_basis": "182,955 FLOP per token-head over the step time vs 2.5 PFLOP/s dense bf16; "
                          "'issued' counts the 3 compensated bf16 passes"}


def measured_traffic(stage):
    """HBM bytes per launch of a stage's kernel from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE counters (scaled by a plain copy's readings), or
    None when there are none or the kernel's source has changed since."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)["kernels"][stage]
        with open(os.path.join(ROOT, "gated_delta_rule_03_amd", "csrc", rec["source"]), "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()[:16]
    except (OSError, KeyError, ValueError):
        return None
    return rec["traffic_bytes"] if sha == rec["source_sha256_16"] else None


def bench_decode(kda, torch, ev, n_steps=128, warmup=3):
    from kda_inputs import BF16, make_params
    from kda_inputs.device_gen import device_tokens
    from kda_inputs.torch_io import make_config
    dev = torch.device("cuda:0")
    N, wid = 256, 4

    class P:  # parameter holder for make_config
        pass
    p = P()
    p.H, p.dk, p.dv, p.io = H, D, D, BF16
    p.w_q, p.w_k, p.w_v, p.A_log, p.dt_bias = make_params(wid, H, D, D, BF16)
    cfg = make_config(p, dev, torch.bfloat16)
    g = torch.Generator(device=dev)
    g.manual_seed(4_000_017)
    S = (torch.randn((N, H, D, D), generator=g, device=dev) * 0.02).contiguous()
    cs = torch.randn((N, 3, H * 3 * D), generator=g, device=dev).to(torch.bfloat16)
    toks = [device_tokens(wid, N, H, D, D, BF16, dev, step=s + 1) for s in range(n_steps)]
    o = torch.empty((N, H, D), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        kda.kda_decode_step(cfg, *toks[i], S, cs, o=o, stream=stream)
    torch.cuda.synchronize()
    st = kda.STAGES.index("decode")
    arrays = [ev.stage_array([st]) for _ in range(n_steps)]
    w0 = time.perf_counter()
    for i in range(n_steps):
        cfg.stage_events = arrays[i]
        kda.kda_decode_step(cfg, *toks[i], S, cs, o=o, stream=stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    cfg.stage_events = None
    us = [1e3 * ev.ms(a[2 * st], a[2 * st + 1]) for a in arrays]
    mean_us = sum(us) / len(us)
    ctot = H * 3 * D
    bytes_step = (2 * N * H * D * D * 4          # state in + out (fp32)
                  + 2 * N * 3 * ctot * 2         # conv history in + out (bf16)
                  + N * (ctot + H * D + H) * 2   # q, k, v, alpha, b (bf16)
                  + N * H * D * 2)               # o (bf16)
    gbs = bytes_step / (mean_us * 1e-6) / 1e9
    log(f"[bench] decode: mean {mean_us:.1f} us/step, p50 {statistics.median(us):.1f} us, {gbs:.0f} GB/s")
    return {"workload": "kda decode step, 256 sequences x 1 token, H=32, dk=dv=128, bf16 in, fp32 state, 128 steps",
            "us_per_step": round(mean_us, 2), "us_per_step_p50": round(statistics.median(us), 2),
            "wall_us_per_step": round(wall / n_steps * 1e6, 2),
            "roofline": {"kernel": "decode", "bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic("decode"),
                         "bytes_per_launch": bytes_step}}


def bench_decode_multi(kda, torch, ev, n_calls=64, warmup=3, K=2):
    """Serving decode with one MTP draft: 256 sequences x K = 2 tokens through
    slots into a pool of 320 rows, the draft of every other sequence
    rejected (commit 1 or 2)."""
    from kda_inputs import BF16, make_params
    from kda_inputs.device_gen import device_tokens
    from kda_inputs.torch_io import make_config
    dev = torch.device("cuda:0")
    N, P, wid = 256, 320, 6

    class Prm:
        pass
    p = Prm()
    p.H, p.dk, p.dv, p.io = H, D, D, BF16
    p.w_q, p.w_k, p.w_v, p.A_log, p.dt_bias = make_params(wid, H, D, D, BF16)
    cfg = make_config(p, dev, torch.bfloat16)
    g = torch.Generator(device=dev)
    g.manual_seed(6_000_029)
    S = (torch.randn((P, H, D, D), generator=g, device=dev) * 0.02).contiguous()
    cs = torch.randn((P, 3, H * 3 * D), generator=g, device=dev).to(torch.bfloat16)
    slots = torch.randperm(P, generator=g, device=dev)[:N].to(torch.int32)
    commit = (1 + torch.arange(N, device=dev) % 2).to(torch.int32)
    calls = []
    for c in range(n_calls):
        t = device_tokens(wid, N * K, H, D, D, BF16, dev, step=c + 1)
        calls.append((t[0].view(N, K, -1), t[1].view(N, K, -1), t[2].view(N, K, -1), t[3].view(N, K, H, D),
                      t[4].view(N, K, H)))
    o = torch.empty((N, K, H, D), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        kda.kda_decode_multi(cfg, *calls[i], S, cs, slots=slots, n_commit=commit, o=o, stream=stream)
    st = kda.STAGES.index("decode")
    arrays = [ev.stage_array([st]) for _ in range(n_calls)]
    torch.cuda.synchronize()
    for i in range(n_calls):
        cfg.stage_events = arrays[i]
        kda.kda_decode_multi(cfg, *calls[i], S, cs, slots=slots, n_commit=commit, o=o, stream=stream)
    torch.cuda.synchronize()
    cfg.stage_events = None
    us = [1e3 * ev.ms(a[2 * st], a[2 * st + 1]) for a in arrays]
    mean_us = sum(us) / len(us)
    ctot = H * 3 * D
    nbytes = (2 * N * H * D * D * 4 + 2 * N * 3 * ctot * 2 + N * K * (ctot + H * D + H) * 2 + N * K * H * D * 2)
    gbs = nbytes / (mean_us * 1e-6) / 1e9
    log(f"[bench] decode multi (K={K}): mean {mean_us:.1f} us/call, {gbs:.0f} GB/s")
    return {"workload": f"kda serving decode, 256 sequences x {K} tokens (one MTP draft) through slots of a 320-row "
                        "pool, commit 1 or 2, H=32, dk=dv=128, bf16 in, fp32 state",
            "us_per_call": round(mean_us, 2), "us_per_token_step": round(mean_us / K, 2),
            "roofline": {"kernel": "decode_multi", "bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic("decode_multi"),
                         "bytes_per_launch": nbytes}}


def bench_varlen(kda, torch, ev, steps=3, warmup=1):
    from kda_inputs import BF16, VARLEN_LENGTHS
    from kda_inputs.device_gen import DeviceProblem
    dev = torch.device("cuda:0")
    dp = DeviceProblem(5, VARLEN_LENGTHS, H, D, D, BF16, dev, state_seqs=[1, 3, 5, 7])
    cfg = dp.config(out_dtype=torch.bfloat16)
    tz = dp.tensors
    total = sum(VARLEN_LENGTHS)
    N = len(VARLEN_LENGTHS)
    o = torch.empty((total, H, D), dtype=torch.bfloat16, device=dev)
    S_out = torch.empty((N, H, D, D), dtype=torch.float32, device=dev)
    ws = torch.empty(kda.kda_varlen_workspace_bytes(cfg, N, total), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        kda.kda_varlen_prefill(cfg, tz["cu_seqlens"], tz["q"], tz["k"], tz["v"], tz["alpha"], tz["b"],
                               tz["initial_state"], None, o=o, final_state=S_out, workspace=ws, stream=stream)

    for _ in range(warmup):
        step()
    e0, e1 = ev.create(), ev.create()
    torch.cuda.synchronize()
    ev.record(e0, stream.cuda_stream)
    for _ in range(steps):
        step()
    ev.record(e1, stream.cuda_stream)
    torch.cuda.synchronize()
    ms = ev.ms(e0, e1) / steps
    log(f"[bench] varlen: {ms:.2f} ms/step, {total / ms * 1e3 / 1e6:.2f} M tokens/s")
    del ws
    return {"workload": "kda varlen prefill, 8 packed sequences (1024..132096, 262144 tokens), H=32, dk=dv=128, bf16",
            "ms_per_step": round(ms, 3), "tokens_per_s": round(total / ms * 1e3, 1)}


def bench_prefill_4k(kda, torch, ev, steps=20, warmup=3):
    """The short prefill (B=1, T=4096, zero initial state).  Its 0.17 GB of
    inputs fit in the 256 MB Infinity Cache, so it is timed twice: back to back
    (warm) and with a 1 GiB buffer written before every call (scrubbed)."""
    from kda_inputs import BF16
    from kda_inputs.device_gen import DeviceProblem
    dev = torch.device("cuda:0")
    T = 4096
    dp = DeviceProblem(2, [T], H, D, D, BF16, dev)
    cfg = dp.config(out_dtype=torch.bfloat16)
    tz = dp.tensors
    q, k, v = (tz[n].view(1, T, -1) for n in ("q", "k", "v"))
    alpha, b = tz["alpha"].view(1, T, H, D), tz["b"].view(1, T, H)
    o = torch.empty((1, T, H, D), dtype=torch.bfloat16, device=dev)
    S_out = torch.empty((1, H, D, D), dtype=torch.float32, device=dev)
    cs_out = torch.empty((1, 3, dp.ctot), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(kda.kda_prefill_workspace_bytes(cfg, 1, T), dtype=torch.uint8, device=dev)
    scrub = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        kda.kda_prefill(cfg, q, k, v, alpha, b, None, None, o=o, final_state=S_out, conv_state_out=cs_out,
                        workspace=ws, stream=stream)

    out = {}
    for mode in ("warm", "scrubbed"):
        for _ in range(warmup):
            step()
        pairs = [(ev.create(), ev.create()) for _ in range(steps)]
        torch.cuda.synchronize()
        for e0, e1 in pairs:
            if mode == "scrubbed":
                scrub.fill_(1.0)
            ev.record(e0, stream.cuda_stream)
            step()
            ev.record(e1, stream.cuda_stream)
        torch.cuda.synchronize()
        vals = [ev.ms(a, b_) for a, b_ in pairs]
        out[mode] = statistics.median(vals)
    nbytes = prefill_alg_bytes(1, T)
    log(f"[bench] 4K prefill: warm {out['warm'] * 1e3:.1f} us, scrubbed {out['scrubbed'] * 1e3:.1f} us")
    del ws, scrub
    return {"workload": "kda chunked prefill B=1 T=4096 H=32 dk=dv=128, bf16, zero initial state, bf16 o",
            "us_warm_p50": round(out["warm"] * 1e3, 2), "us_scrubbed_p50": round(out["scrubbed"] * 1e3, 2),
            "tokens_per_s_warm": round(T / out["warm"] * 1e3, 1),
            "tokens_per_s_scrubbed": round(T / out["scrubbed"] * 1e3, 1),
            "path_hbm_frac_scrubbed": round(nbytes / (out["scrubbed"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "bytes_per_call": nbytes}


# Peak of fp32 VALU lane operations (non-packed, as this library is built):
# 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz.
VALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12


def bench_prefill_no_clamp(kda, torch, ev, dp, steps=5, warmup=2):
    """The same 32K prefill with the gate's clamp off (lower bound -inf): the
    recurrent form (token pre-pass + register-resident recurrent scan)."""
    dev = torch.device("cuda:0")
    B, T = 4, 32768
    cfg = dp.config(out_dtype=torch.bfloat16, gate_lower_bound=float("-inf"))
    tz = dp.tensors
    q, k, v = (tz[n].view(B, T, -1) for n in ("q", "k", "v"))
    alpha, b = tz["alpha"].view(B, T, H, D), tz["b"].view(B, T, H)
    o = torch.empty((B, T, H, D), dtype=torch.bfloat16, device=dev)
    S_out = torch.empty((B, H, D, D), dtype=torch.float32, device=dev)
    ws = torch.empty(kda.kda_prefill_workspace_bytes(cfg, B, T), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        kda.kda_prefill(cfg, q, k, v, alpha, b, tz["initial_state"], tz["conv_state"], o=o, final_state=S_out,
                        workspace=ws, stream=stream)

    for _ in range(warmup):
        step()
    stages = [kda.STAGES.index(n) for n in ("chunk_prep", "chunk_scan")]
    arrays = [ev.stage_array(stages) for _ in range(steps)]
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for i in range(steps):
        cfg.stage_events = arrays[i]
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    cfg.stage_events = None
    per = stage_means(ev, arrays, stages)
    prep_ms, scan_ms = per[stages[0]], per[stages[1]]
    ms = wall / steps * 1e3
    lane_ops = 4 * D * D * B * T * H            # decay multiply, two dot-product FMAs, rank-1 update
    tops = lane_ops / (scan_ms * 1e-3) / 1e12
    log(f"[bench] prefill without clamp: {ms:.2f} ms/step (pre-pass {prep_ms:.3f}, scan {scan_ms:.3f})")
    del ws
    return {"workload": "kda prefill B=4 T=32768 H=32 dk=dv=128, bf16, gate lower bound -inf (recurrent form)",
            "ms_per_step": round(ms, 3), "tokens_per_s": round(B * T / ms * 1e3, 1),
            "stage_ms": {"token_prep": round(prep_ms, 4), "recurrent_scan": round(scan_ms, 4)},
            "roofline": {"kernel": "recurrent_scan", "bound": "alu", "achieved": round(tops, 3),
                         "peak": round(VALU_PEAK_TOPS, 2), "unit": "T fp32 VALU lane-ops/s",
                         "frac": round(tops / VALU_PEAK_TOPS, 4), "traffic": measured_traffic("recurrent_scan"),
                         "lane_ops_per_launch": lane_ops}}


def bench_prefill_slabs(kda, torch, ev, dp, slabs=(8192, 2048), steps=10, warmup=2):
    """The 32K prefill with a workspace for slabs of S positions per sequence
    instead of one pass (the chunked form run window after window, the state
    carried between them; results bit-identical to one pass)."""
    dev = torch.device("cuda:0")
    B, T = 4, 32768
    cfg = dp.config(out_dtype=torch.bfloat16)
    tz = dp.tensors
    q, k, v = (tz[n].view(B, T, -1) for n in ("q", "k", "v"))
    alpha, b = tz["alpha"].view(B, T, H, D), tz["b"].view(B, T, H)
    o = torch.empty((B, T, H, D), dtype=torch.bfloat16, device=dev)
    S_out = torch.empty((B, H, D, D), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    out = {"workload": "kda chunked prefill B=4 T=32768 H=32 dk=dv=128, bf16, workspace for slabs of S positions",
           "one_pass_workspace_gib": round(kda.kda_prefill_workspace_bytes(cfg, B, T) / 2**30, 2), "slabs": {}}
    for slab in slabs:
        ws = torch.empty(kda.kda_prefill_slab_workspace_bytes(cfg, B, slab), dtype=torch.uint8, device=dev)

        def step():
            kda.kda_prefill(cfg, q, k, v, alpha, b, tz["initial_state"], tz["conv_state"], o=o, final_state=S_out,
                            workspace=ws, stream=stream)

        for _ in range(warmup):
            step()
        e0, e1 = ev.create(), ev.create()
        torch.cuda.synchronize()
        ev.record(e0, stream.cuda_stream)
        for _ in range(steps):
            step()
        ev.record(e1, stream.cuda_stream)
        torch.cuda.synchronize()
        ms = ev.ms(e0, e1) / steps
        gib = ws.numel() / 2**30
        log(f"[bench] prefill in slabs of {slab}: {ms:.3f} ms/step, workspace {gib:.2f} GiB")
        out["slabs"][str(slab)] = {"ms_per_step": round(ms, 3), "tokens_per_s": round(B * T / ms * 1e3, 1),
                                   "workspace_gib": round(gib, 3)}
        del ws
    return out


def bench_output_gate(kda, torch, ev, steps=20, warmup=3):
    """The o_norm x sigmoid-gate epilogue on the 32K prefill's output shape
    (4 x 32768 tokens x 32 heads x 128, bf16 o and gate), in place."""
    dev = torch.device("cuda:0")
    n = 4 * 32768
    g = torch.Generator(device=dev)
    g.manual_seed(5_000_011)
    o = torch.randn((n, H, D), generator=g, device=dev).to(torch.bfloat16)
    gate = (torch.randn((n, H, D), generator=g, device=dev) * 2).to(torch.bfloat16)
    w = torch.rand((D,), generator=g, device=dev) + 0.5
    cfg = kda.Config(A_log=None, dt_bias=None, conv_w_q=None, conv_w_k=None, conv_w_v=None, num_heads=H,
                     head_k_dim=D, head_v_dim=D, io_dtype=torch.bfloat16, out_dtype=torch.bfloat16)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        kda.kda_output_gate(cfg, o, gate, w, y=o, stream=stream)
    st = kda.STAGES.index("output_gate")
    arrays = [ev.stage_array([st]) for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        cfg.stage_events = arrays[i]
        kda.kda_output_gate(cfg, o, gate, w, y=o, stream=stream)
    torch.cuda.synchronize()
    cfg.stage_events = None
    us = 1e3 * stage_means(ev, arrays, [st])[st]
    nbytes = n * H * D * 2 * 3 + D * 4           # o and gate in, y out (bf16), weight
    gbs = nbytes / (us * 1e-6) / 1e9
    log(f"[bench] output gate: {us:.1f} us/launch, {gbs:.0f} GB/s")
    return {"workload": "kda o_norm x sigmoid output gate, 131072 tokens x 32 heads x 128, bf16, in place",
            "us_per_launch": round(us, 2),
            "roofline": {"kernel": "output_gate", "bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic("output_gate"),
                         "bytes_per_launch": nbytes}}


def bench_backward(kda, torch, ev, dp, steps=5, warmup=1):
    """The backward pass of the headline prefill (B=4, T=32768, H=32, d=128,
    bf16 inputs): gradients of every input and parameter for a random bf16 dO
    and fp32 d(final state), through kda_varlen_backward."""
    dev = torch.device("cuda:0")
    B, T = 4, 32768
    cfg = dp.config(out_dtype=torch.bfloat16)
    tz = dp.tensors
    g = torch.Generator(device=dev)
    g.manual_seed(9_000_001)
    d_o = torch.randn((B * T, H, D), generator=g, device=dev).to(torch.bfloat16)
    dST = torch.randn((B, H, D, D), generator=g, device=dev)
    ws = torch.empty(kda.kda_varlen_backward_workspace_bytes(cfg, B, B * T), dtype=torch.uint8, device=dev)
    log(f"[bench] backward workspace {ws.numel() / 2**30:.2f} GiB")
    stream = torch.cuda.current_stream()

    def step():
        return kda.kda_varlen_backward(cfg, tz["cu_seqlens"], tz["q"], tz["k"], tz["v"], tz["alpha"], tz["b"],
                                       tz["initial_state"], tz["conv_state"], d_o=d_o, d_final_state=dST,
                                       workspace=ws, stream=stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = ev.create(), ev.create()
    ev.record(e0, stream.cuda_stream)
    for _ in range(steps):
        step()
    ev.record(e1, stream.cuda_stream)
    torch.cuda.synchronize()
    ms = ev.ms(e0, e1) / steps
    log(f"[bench] backward: {ms:.2f} ms per call, {B * T / ms * 1e3 / 1e6:.2f} M tokens/s")
    del ws
    return {"workload": "kda backward of the chunked prefill B=4 T=32768 H=32 dk=dv=128, bf16 inputs and dO, "
                        "fp32 gradients of every input and parameter",
            "ms_per_call": round(ms, 3), "tokens_per_s": round(B * T / ms * 1e3, 1)}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(dp, seqs=4, single_items=6):
    """The fp64 oracle on the first `seqs` sequences of the prefill workload
    (all heads, full length) on all host cores the process may use, and on
    one thread over `single_items` (sequence, head) pairs of full length."""
    import numpy as np
    import torch
    import oracle
    from kda_inputs import Problem
    T = dp.seqlens[0]
    n_tok = T * seqs

    def host(x):
        x = x[:n_tok].contiguous()
        return x.view(torch.int16).cpu().numpy().view(np.uint16) if x.dtype == torch.bfloat16 else x.cpu().numpy()
    tz = dp.tensors
    p = Problem([T] * seqs, dp.H, dp.dk, dp.dv, dp.io, host(tz["q"]), host(tz["k"]), host(tz["v"]), host(tz["alpha"]),
                host(tz["b"]), dp.w_q, dp.w_k, dp.w_v, dp.A_log, dp.dt_bias, dp.initial_state[:seqs], None)
    oracle.build()
    t0 = time.perf_counter()
    _, _, _, threads = oracle.forward(p, with_conv_out=False)
    dt = time.perf_counter() - t0
    items = [(i * 37) % (seqs * dp.H) for i in range(single_items)]
    t1 = time.perf_counter()
    oracle.forward(p, with_conv_out=False, items=items, nthreads=1)
    dt1 = time.perf_counter() - t1
    tok_1 = single_items * T / dp.H / dt1          # tokens/s of all heads, from token-heads/s
    log(f"[bench] cpu oracle: {n_tok} tokens x {dp.H} heads in {dt:.1f}s on {threads} threads; "
        f"1 thread: {single_items} x {T} token-heads in {dt1:.1f}s")
    return {"value": round(n_tok / dt, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"fp64 token-by-token oracle on {seqs} of the 4 sequences (all {dp.H} heads, all {T} tokens "
                      f"each, {n_tok} tokens), wall {dt:.1f}s",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "one_thread": {"value": round(tok_1, 1), "unit": "tokens/s",
                           "sample": f"{single_items} (sequence, head) pairs x {T} tokens on 1 thread, "
                                     f"wall {dt1:.1f}s, scaled to tokens/s of all {dp.H} heads"}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the 4K prefill, decode, varlen, no-clamp prefill and output-gate measurements")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device-to-device copy and a 1 GiB elementwise multiply "
                         "(to scale HBM traffic counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the KDA core has no cross-GPU path here (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_delta_rule_03_amd as kda
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    ev = HipEvents()
    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda")   # 1 GiB
        dst = torch.empty_like(src)
        src.fill_(1.0)
        for _ in range(3):
            dst.copy_(src)
        for _ in range(3):             # and a plain elementwise kernel: 1 GiB read, 1 GiB written
            torch.mul(src, 2.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
    B, T = 4, 32768
    dp, wall, gpu_ms, per_stage = bench_prefill(kda, torch, ev, args.steps, args.warmup)
    ms_step = wall / args.steps * 1e3
    value = B * T / (wall / args.steps)
    roof = roofline_for(kda, per_stage, ms_step, B, T)
    path_gbs = prefill_alg_bytes(B, T) / (ms_step * 1e-3) / 1e9
    result = {
        "metric": "KDA prefill tokens/s (H=32,d=128,T=32K) + decode step us; % of roofline",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16x3/fp32", "data": "synthetic",
        "config": {"workload": "kda chunked prefill B=4 T=32768 H=32 dk=dv=128, bf16 q/k/v/alpha/b, fp32 state "
                               "(initial state ~N(0,0.02)), bf16 o, chunk 64",
                   "global_batch": B, "seq_len": T, "parallelism": "none (1 GPU)"},
        "stage_ms": {kda.STAGES[s]: round(v, 4) for s, v in per_stage.items()},
        "gpu_event_ms_per_step": round(gpu_ms / args.steps, 3),
        "roofline": roof,
        "path_hbm_frac": round(path_gbs / HBM_PEAK_GBS, 4),
    }
    if not args.no_extras:
        result["prefill_4k"] = bench_prefill_4k(kda, torch, ev)
        result["decode"] = bench_decode(kda, torch, ev)
        result["decode_multi"] = bench_decode_multi(kda, torch, ev)
        result["varlen"] = bench_varlen(kda, torch, ev)
        result["prefill_no_clamp"] = bench_prefill_no_clamp(kda, torch, ev, dp)
        result["prefill_slabs"] = bench_prefill_slabs(kda, torch, ev, dp)
        result["output_gate"] = bench_output_gate(kda, torch, ev)
        result["backward"] = bench_backward(kda, torch, ev, dp)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(dp)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
