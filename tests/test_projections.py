"""The projection check of the full-output GEMM tests (tests/projections.py),
on the CPU: it accepts the oracle's own product and catches one accumulator
off by one, in its row and its column, and nowhere else."""

import numpy as np

import oracle as O
from projections import project_expected, project_observed


def test_projections_catch_one_wrong_accumulator():
    """The check itself, on the CPU sizes of a small product: one accumulator
    off by one is caught by the projections of its row and its column."""
    rng = np.random.default_rng(3)
    M, K, N = 48, 256, 64
    X = rng.standard_normal((M, K)).astype(np.float16)
    W = rng.standard_normal((N, K)).astype(np.float16)
    x8, _ = O.quant_act_per_token(X)
    acc = O.gemm_exact(x8, O.encode_weight_g128(W)["w8"]).astype(np.int32)
    vals = np.array([-2, -1, 1, 2], np.int64)
    r_list = [np.ones(M, np.int64), rng.choice(vals, size=M)]
    c_list = [np.ones(N, np.int64), rng.choice(vals, size=N)]
    want_rt, want_ac = project_expected(x8, W, 128, r_list, c_list)
    got_rt, got_ac = project_observed(acc, r_list, c_list)
    assert all(np.array_equal(a, b) for a, b in zip(got_rt, want_rt))
    assert all(np.array_equal(a, b) for a, b in zip(got_ac, want_ac))
    acc[17, 41] += 1
    got_rt, got_ac = project_observed(acc, r_list, c_list)
    for a, b in zip(got_rt, want_rt):
        assert np.nonzero(a != b)[0].tolist() == [41]
    for a, b in zip(got_ac, want_ac):
        assert np.nonzero(a != b)[0].tolist() == [17]
