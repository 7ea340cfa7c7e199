"""The oracle and the synthetic workloads use the constants the pages print."""
import json
import os

import numpy as np

import oracle
from kda_inputs import workload_decode
from tests.helpers import small_problem

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")))


def test_gate_bound_default():
    assert oracle.DEFAULT_LOWER_BOUND == GOLDEN["gate_lower_bound"]["value"]


def test_conv_reads_three_history_inputs(oracle_lib):
    # with taps only on the oldest position, the first output equals the
    # oldest history entry: the conv sees exactly kernel-1 = 3 past inputs
    assert GOLDEN["conv_kernel_size"]["value"] - 1 == GOLDEN["conv_history"]["value"] == 3
    p = small_problem(31, [5], H=1, dk=4, dv=4, state=False, conv=True)
    p.w_q = np.zeros_like(p.w_q); p.w_q[:, 0] = 1.0
    qh, _, _, _, _ = oracle.preprocess_head(p, 0, 0, flags=oracle.FLAG_SKIP_L2NORM)
    from kda_inputs import as_f64
    y = as_f64(p.conv_state, p.io)[0, 0, 0:4]
    assert np.allclose(qh[0], y / (1 + np.exp(-y)))
    _, _, cout, _ = oracle.forward(p)
    assert cout.shape[1] == GOLDEN["conv_history"]["value"]


def test_beta_in_unit_interval(oracle_lib):
    assert GOLDEN["beta_times_two"]["value"] is False
    p = small_problem(32, [50], H=2, dk=4, dv=4, state=False, conv=False)
    for h in range(2):
        beta = oracle.preprocess_head(p, 0, h)[4]
        assert (beta > 0).all() and (beta < 1).all()


def test_workload_geometry():
    H, d = GOLDEN["num_heads"]["value"], GOLDEN["head_dim"]["value"]
    dp = workload_decode(N=2, steps=1)
    assert (dp.H, dp.dk, dp.dv) == (H, d, d)
    assert dp.state.shape == (2, H, d, d)   # (batch, v_heads, k_dim, v_dim)
