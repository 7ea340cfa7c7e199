"""GPU parity of kda_varlen_prefill_noalloc (the packed prefill on the
library's fixed per-GPU scratch, for callers that cannot allocate) against
kda_varlen_prefill with a caller workspace.  Both run the same kernels on the
same inputs, so o, the final state and the conv history must agree bit for
bit.  Two calls in a row, the second on a smaller batch (the scratch keeps the
first call's bytes); a batch whose one-pass workspace exceeds the scratch,
which runs in slabs; and one where not even a slab fits, which must be
refused before anything runs.
"""
import numpy as np
import pytest
import torch

from kda_inputs import BF16, FP32, make_problem
from kda_inputs.torch_io import problem_to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_03_amd as m
    return m


def run_both(kda, p, **kw):
    dev = torch.device("cuda:0")
    cfg, t = problem_to_device(p, dev, out_dtype=torch.float32, **kw)
    N = len(p.seqlens)
    outs = []
    for noalloc in (False, True):
        o = torch.full((p.total_T, p.H, p.dv), float("nan"), device=dev)
        S = torch.full((N, p.H, p.dk, p.dv), float("nan"), device=dev)
        cs = torch.full((N, 3, p.ctot), float("nan"), device=dev, dtype=cfg.io_dtype)
        args = (cfg, t["cu_seqlens"], t["q"], t["k"], t["v"], t["alpha"], t["b"], t["initial_state"],
                t["conv_state"])
        if noalloc:
            kda.kda_varlen_prefill_noalloc(*args, o=o, final_state=S, conv_state_out=cs)
        else:
            kda.kda_varlen_prefill(*args, o=o, final_state=S, conv_state_out=cs)
        torch.cuda.synchronize()
        outs.append((o, S, cs))
    (o1, S1, c1), (o2, S2, c2) = outs
    assert torch.isfinite(o1).all() and torch.isfinite(S1).all()
    assert torch.equal(o1, o2) and torch.equal(S1, S2) and torch.equal(c1, c2)


@pytest.mark.parametrize("io,d", [(BF16, 128), (FP32, 32)])
def test_noalloc_matches_workspace_call_twice(kda, io, d):
    big = make_problem(4500 + d, [700, 1, 0, 390, 64], 4, d, d, io, state_seqs=[0, 3], conv_state=True)
    run_both(kda, big)
    small = make_problem(4600 + d, [70, 5], 2, d, d, io, state_seqs=[1], conv_state=True)
    run_both(kda, small)


def test_noalloc_recurrent_form(kda):
    p = make_problem(4700, [150, 3, 64], 3, 64, 64, BF16, state_seqs=[0], conv_state=True)
    run_both(kda, p, gate_lower_bound=float("-inf"))


def test_noalloc_runs_batches_beyond_the_scratch_in_slabs(kda):
    """A batch whose one-pass workspace exceeds the scratch runs in slabs of
    positions, bit-identical to the one-pass call with a workspace."""
    p = make_problem(4900, [20000, 9000, 0, 77], 4, 128, 128, BF16, state_seqs=[0, 1], conv_state=True)
    cfg, _ = problem_to_device(p, torch.device("cuda:0"))
    assert kda.kda_varlen_workspace_bytes(cfg, 4, p.total_T) > kda.NOALLOC_SCRATCH_BYTES
    run_both(kda, p)


def test_noalloc_refuses_batches_beyond_one_slab(kda):
    """Refused before anything runs when not even a 64-token slab fits: 40
    sequences at H = 32, d = 128 need 6.5 MB each."""
    dev = torch.device("cuda:0")
    p = make_problem(4800, [64], 32, 128, 128, BF16)
    cfg, t = problem_to_device(p, dev)
    N, total = 40, 40 * 64
    assert kda.kda_prefill_slab_workspace_bytes(cfg, N, 64) > kda.NOALLOC_SCRATCH_BYTES
    cu = torch.arange(0, total + 1, 64, dtype=torch.int32, device=dev)
    q = torch.zeros((total, 32 * 128), dtype=torch.bfloat16, device=dev)
    b = torch.zeros((total, 32), dtype=torch.bfloat16, device=dev)
    o = torch.full((total, 32, 128), 7.0, device=dev)
    with pytest.raises(kda.KdaError) as ei:
        kda.kda_varlen_prefill_noalloc(cfg, cu, q, q, q, q.view(total, 32, 128), b, o=o)
    assert ei.value.status == kda.KDA_ERR_WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()
    assert bool((o == 7.0).all())
