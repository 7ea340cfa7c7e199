"""GPU parity of kda_decode_multi (K tokens per sequence through state and
conv-history pools, with commit counts) against the fp64 oracle.

Bounds as for the decode step: o max|o - o_ref| <= 2e-3 RMS(o_ref) and state
relative Frobenius error <= 1e-3 for bf16 inputs (1e-5 / 1e-5 all-fp32).  Pool
rows that a call must not touch (unused slots, skipped sequences, commit 0)
are compared bit for bit, and so are conv histories (copies of raw inputs).
"""
import numpy as np
import pytest
import torch

import oracle
from kda_inputs import BF16, FP32, as_f64, make_tokens, workload_decode
from kda_inputs.torch_io import decode_to_device, from_torch_bf16, to_torch, tokens_to_device
from tests.helpers import max_over_rms, rel_fro
from tests.test_gpu_parity import kda  # noqa: F401  (fixture)

pytestmark = pytest.mark.gpu

BOUNDS = {BF16: (2e-3, 1e-3), FP32: (1e-5, 1e-5)}


def setup(seed, N, K, P, H, d, io):
    pool = workload_decode(N=P, H=H, d=d, steps=1, io=io, workload_id=seed)
    dev = torch.device("cuda:0")
    cfg, S, cs = decode_to_device(pool, dev, out_dtype=torch.float32)
    toks = make_tokens(seed + 1, N * K, H, d, d, io)
    q, k, v, alpha, b = tokens_to_device(toks, io, dev)
    dtoks = (q.view(N, K, -1), k.view(N, K, -1), v.view(N, K, -1), alpha.view(N, K, H, d), b.view(N, K, H))
    params = (pool.w_q, pool.w_k, pool.w_v, pool.A_log, pool.dt_bias)
    return pool, cfg, S, cs, toks, dtoks, params


def conv_host(cs, io):
    return as_f64(from_torch_bf16(cs), BF16) if io == BF16 else cs.double().cpu().numpy()


def i32(x):
    return torch.tensor(x, dtype=torch.int32, device="cuda:0")


def check(pool, io, o, S, cs, o_ref, S_ref, c_ref, active, touched):
    bo, bs = BOUNDS[io]
    og = o.double().cpu().numpy()
    assert max_over_rms(og[active], o_ref[active]) <= bo
    Sg = S.double().cpu().numpy()
    if touched:
        assert rel_fro(Sg[touched], S_ref[touched]) <= bs
    untouched = [r for r in range(pool.N) if r not in touched]
    assert np.array_equal(S.cpu().numpy()[untouched], pool.state[untouched]), "a pool row changed"
    assert np.array_equal(conv_host(cs, io), c_ref), "conv history mismatch"


@pytest.mark.parametrize("K", [1, 2, 4])
@pytest.mark.parametrize("d", [64, 128])
def test_multi_through_slots(kda, K, d):
    N, P, H = 5, 8, 4
    pool, cfg, S, cs, toks, dtoks, params = setup(1500 + 10 * K + d, N, K, P, H, d, BF16)
    slots = [6, -1, 0, 3, 7]
    o = kda.kda_decode_multi(cfg, *dtoks, S, cs, slots=i32(slots))
    torch.cuda.synchronize()
    o_ref, S_ref, c_ref = oracle.decode_multi_reference(pool.state, pool.conv_state, slots, toks, params, H, d, d,
                                                        BF16, K)
    check(pool, BF16, o, S, cs, o_ref, S_ref, c_ref, [0, 2, 3, 4], [6, 0, 3, 7])


def test_verify_then_commit(kda):
    N, K, P, H, d = 5, 4, 5, 4, 128
    pool, cfg, S, cs, toks, dtoks, params = setup(1600, N, K, P, H, d, BF16)
    slots = [4, 2, 0, 1, 3]
    # verify: every output, pools untouched
    o1 = kda.kda_decode_multi(cfg, *dtoks, S, cs, slots=i32(slots), n_commit=i32([0] * N))
    torch.cuda.synchronize()
    assert np.array_equal(S.cpu().numpy(), pool.state) and np.array_equal(from_torch_bf16(cs), pool.conv_state)
    o_ref, _, _ = oracle.decode_multi_reference(pool.state, pool.conv_state, slots, toks, params, H, d, d, BF16, K)
    assert max_over_rms(o1.double().cpu().numpy(), o_ref) <= 2e-3
    # commit a different number of accepted tokens per sequence
    commit = [0, 1, 2, 4, 3]
    o2 = kda.kda_decode_multi(cfg, *dtoks, S, cs, slots=i32(slots), n_commit=i32(commit))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2), "outputs depend only on the pools' contents before the call"
    _, S_ref, c_ref = oracle.decode_multi_reference(pool.state, pool.conv_state, slots, toks, params, H, d, d,
                                                    BF16, K, n_commit=commit)
    check(pool, BF16, o2, S, cs, o_ref, S_ref, c_ref, list(range(N)), [2, 0, 1, 3])


def test_multi_equals_single_steps(kda):
    N, K, H, d = 4, 3, 4, 128
    pool, cfg, S, cs, toks, dtoks, params = setup(1700, N, K, N, H, d, BF16)
    S2, cs2 = S.clone(), cs.clone()
    o = kda.kda_decode_multi(cfg, *dtoks, S, cs)               # slots = n, every token committed
    steps = [kda.kda_decode_step(cfg, *(t[:, i].contiguous() for t in dtoks), S2, cs2) for i in range(K)]
    torch.cuda.synchronize()
    o_ref, S_ref, c_ref = oracle.decode_multi_reference(pool.state, pool.conv_state, list(range(N)), toks, params,
                                                        H, d, d, BF16, K)
    check(pool, BF16, o, S, cs, o_ref, S_ref, c_ref, list(range(N)), list(range(N)))
    assert torch.equal(cs, cs2)
    assert max_over_rms(torch.stack(steps, 1).double().cpu().numpy(), o_ref) <= 2e-3
    assert rel_fro(S2.double().cpu().numpy(), S_ref) <= 1e-3


@pytest.mark.parametrize("d", [16, 32])
def test_multi_fp32(kda, d):
    N, K, P, H = 3, 3, 4, 3
    pool, cfg, S, cs, toks, dtoks, params = setup(1800 + d, N, K, P, H, d, FP32)
    slots, commit = [1, 3, -1], [2, 3, 1]
    o = kda.kda_decode_multi(cfg, *dtoks, S, cs, slots=i32(slots), n_commit=i32(commit))
    torch.cuda.synchronize()
    o_ref, S_ref, c_ref = oracle.decode_multi_reference(pool.state, pool.conv_state, slots, toks, params, H, d, d,
                                                        FP32, K, n_commit=commit)
    check(pool, FP32, o, S, cs, o_ref, S_ref, c_ref, [0, 1], [1, 3])


def test_multi_serving_shape(kda):
    """256 sequences x 32 heads x 128, one MTP draft (K = 2), slots spread
    over a pool of 300 rows, half of the drafts rejected."""
    N, K, P, H, d = 256, 2, 300, 32, 128
    pool, cfg, S, cs, toks, dtoks, params = setup(1900, N, K, P, H, d, BF16)
    slots = np.random.default_rng(3).permutation(P)[:N].tolist()
    commit = [1 + (n % 2) for n in range(N)]
    o = kda.kda_decode_multi(cfg, *dtoks, S, cs, slots=i32(slots), n_commit=i32(commit))
    torch.cuda.synchronize()
    o_ref, S_ref, c_ref = oracle.decode_multi_reference(pool.state, pool.conv_state, slots, toks, params, H, d, d,
                                                        BF16, K, n_commit=commit)
    check(pool, BF16, o, S, cs, o_ref, S_ref, c_ref, list(range(N)), slots)


def test_multi_across_staging_groups(kda):
    """K = 19 tokens: the inputs are staged eight tokens at a time (groups of
    8, 8 and 3), and the commit counts fall inside and on group edges."""
    N, K, P, H, d = 6, 19, 7, 4, 128
    pool, cfg, S, cs, toks, dtoks, params = setup(2000, N, K, P, H, d, BF16)
    slots, commit = [5, 0, 6, 2, 1, 3], [0, 7, 8, 9, 16, 19]
    o = kda.kda_decode_multi(cfg, *dtoks, S, cs, slots=i32(slots), n_commit=i32(commit))
    torch.cuda.synchronize()
    o_ref, S_ref, c_ref = oracle.decode_multi_reference(pool.state, pool.conv_state, slots, toks, params, H, d, d,
                                                        BF16, K, n_commit=commit)
    check(pool, BF16, o, S, cs, o_ref, S_ref, c_ref, list(range(N)), [0, 6, 2, 1, 3])
