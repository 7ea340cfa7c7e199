"""The chunked prefill in slabs (a workspace smaller than one pass needs):
windows of the positions of every sequence run one after the other, the
state carried between them.  The results must be bit-identical to one pass
(the state at a chunk boundary is the same fp32 value in memory as in
registers), and one pass is itself held to the oracle in test_gpu_parity.py;
one slab case is also checked against the oracle directly here."""
import numpy as np
import pytest
import torch

from kda_inputs import BF16, FP32, make_problem
from kda_inputs.torch_io import problem_to_device
from tests.test_gpu_parity import assert_parity, kda  # noqa: F401  (fixture)

pytestmark = pytest.mark.gpu


def varlen(kda, p, ws_bytes=None, with_state_out=True, out_dtype=torch.float32):
    dev = torch.device("cuda:0")
    cfg, t = problem_to_device(p, dev, out_dtype=out_dtype)
    N = len(p.seqlens)
    S = torch.full((N, p.H, p.dk, p.dv), float("nan"), device=dev) if with_state_out else None
    cs = torch.full((N, 3, p.ctot), float("nan"), device=dev, dtype=cfg.io_dtype)
    ws = None
    if ws_bytes is not None:
        full = kda.kda_varlen_workspace_bytes(cfg, N, p.total_T)
        assert ws_bytes < full, "the slab workspace must be smaller than one pass"
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    o, _, _ = kda.kda_varlen_prefill(cfg, t["cu_seqlens"], t["q"], t["k"], t["v"], t["alpha"], t["b"],
                                     t["initial_state"], t["conv_state"], final_state=S, conv_state_out=cs,
                                     workspace=ws)
    torch.cuda.synchronize()
    return o, S, cs, cfg


def assert_same(a, b):
    assert torch.equal(a[0], b[0]), "o differs from one pass"
    if a[1] is not None and b[1] is not None:
        assert torch.equal(a[1], b[1]), "final state differs from one pass"
    assert torch.equal(a[2], b[2]), "conv history differs from one pass"


@pytest.mark.parametrize("io,D", [(BF16, 128), (BF16, 64), (FP32, 32), (FP32, 16)])
def test_varlen_slabs_match_one_pass(kda, io, D):
    """Ragged lengths (empty, shorter than the conv history, around one chunk,
    several chunks with tails), initial states on some sequences and a conv
    history; slabs of 64 and 192 positions."""
    lens = [0, 1, 63, 64, 65, 300, 1000, 2]
    p = make_problem(9100 + D, lens, 2, D, D, io, state_seqs=[1, 3, 5, 6], conv_state=True)
    one = varlen(kda, p)
    for slab in (64, 192):
        need = kda.kda_prefill_slab_workspace_bytes(one[3], len(lens), slab)
        assert_same(varlen(kda, p, ws_bytes=need), one)


def test_uniform_slabs_match_one_pass_and_oracle(kda):
    """kda_prefill (B equal lengths, T not a multiple of the slab) in slabs of
    256 positions, against one pass and against the oracle."""
    dev = torch.device("cuda:0")
    p = make_problem(9200, [700, 700, 700], 4, 64, 64, BF16, state_seqs=[0, 2], conv_state=True)
    cfg, t = problem_to_device(p, dev, out_dtype=torch.float32)
    B, T = 3, 700
    args = [t[n].view(B, T, *t[n].shape[1:]) for n in ("q", "k", "v", "alpha", "b")]
    res = []
    for ws_bytes in (None, kda.kda_prefill_slab_workspace_bytes(cfg, B, 256)):
        S = torch.full((B, p.H, p.dk, p.dv), float("nan"), device=dev)
        cs = torch.full((B, 3, p.ctot), float("nan"), device=dev, dtype=cfg.io_dtype)
        ws = None if ws_bytes is None else torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        o, _, _ = kda.kda_prefill(cfg, *args, t["initial_state"], t["conv_state"], final_state=S,
                                  conv_state_out=cs, workspace=ws)
        torch.cuda.synchronize()
        res.append((o, S, cs))
    assert_same(res[1], res[0])
    o, S, cs = res[1]
    assert_parity(p, o.view(B * T, p.H, p.dv), S, cs)


def test_slabs_without_final_state_and_in_place_state(kda):
    """Without a final state the carried state lives in the workspace; with
    the final state aliasing the initial state the carry is in place."""
    p = make_problem(9300, [130, 5, 257], 2, 128, 128, BF16, state_seqs=[0, 1, 2], conv_state=True)
    one = varlen(kda, p)
    need = kda.kda_prefill_slab_workspace_bytes(one[3], 3, 64)
    no_state = varlen(kda, p, ws_bytes=need, with_state_out=False)
    assert torch.equal(no_state[0], one[0])
    # in place: the initial state buffer receives the final state
    dev = torch.device("cuda:0")
    cfg, t = problem_to_device(p, dev, out_dtype=torch.float32)
    S = t["initial_state"].clone()
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    o, _, _ = kda.kda_varlen_prefill(cfg, t["cu_seqlens"], t["q"], t["k"], t["v"], t["alpha"], t["b"], S,
                                     t["conv_state"], final_state=S, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o, one[0]) and torch.equal(S, one[1])
