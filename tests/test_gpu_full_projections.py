"""Every INT32 accumulator of the largest workloads, checked through exact
linear projections.

The oracle cannot form the full 4096 x 24576 product over K = 8192 one
output at a time in a test's budget, but it can compute, exactly and cheaply,
what any product of the same operands must give when multiplied by a vector:
with acc = x8 @ w8^T ("QServe: W4A8KV4 Quantization and System Co-design for
Efficient LLM Serving", paperlayer.ai summary, §2 integer quantization: the
W4A8 GEMM is an INT8 x INT8 product into INT32 once the UINT4 weights are
dequantized to INT8),

    acc^T r = w8 @ (x8^T r)      (N equations per row weight vector r)
    acc c   = x8 @ (w8^T c)      (M equations per column weight vector c)

and the row and column sums (r, c all ones).  The weight vectors take values
in {-2, -1, 1, 2} (never 0), so any single wrong accumulator changes the
equation of its column (and of its row) and is caught; several wrong values
could only hide by cancelling in every one of the eight projections.  All
sums stay below 2^53, so the host side computes them exactly in float64 and
int64.  The oracle's w8 comes from its own encode of the synthetic weights,
in chunks of output channels; nothing on the expected side comes from the
GPU.
"""

import numpy as np
import pytest

import oracle as O
import synthetic
import w4a8_quantized_gemm_qoq_amd as q

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from projections import project_expected, project_observed  # noqa: E402


@pytest.mark.parametrize("name", ["ffn_large_g128", "ffn_large_perchannel"])
def test_full_output_projections(name):
    w = synthetic.get_workload(name)
    X, W = synthetic.make_inputs(w)
    print(f"[projections] {name} M={w.M} K={w.K} N={w.N} gs={w.group_size}", flush=True)
    p = q.qoq_pack_weights(W, w.group_size).to("cuda")
    x8_dev, _ = q.qoq_quant_act_per_token(torch.from_numpy(X).cuda())
    acc = q.qoq_w4a8_gemm_i32(x8_dev, p).cpu().numpy()
    del p
    torch.cuda.synchronize()
    ox8, _ = O.quant_act_per_token(X)
    assert np.array_equal(x8_dev.cpu().numpy(), ox8)

    rng = np.random.default_rng(2024)
    vals = np.array([-2, -1, 1, 2], np.int64)
    r_list = [np.ones(w.M, np.int64)] + [rng.choice(vals, size=w.M) for _ in range(3)]
    c_list = [np.ones(w.N, np.int64)] + [rng.choice(vals, size=w.N) for _ in range(3)]
    got_rt, got_ac = project_observed(acc, r_list, c_list)
    want_rt, want_ac = project_expected(ox8, W, w.group_size, r_list, c_list)
    for i in range(len(r_list)):
        bad = np.nonzero(got_rt[i] != want_rt[i])[0]
        assert bad.size == 0, f"acc^T r[{i}] differs in {bad.size} columns, first {bad[:8]}"
    for i in range(len(c_list)):
        bad = np.nonzero(got_ac[i] != want_ac[i])[0]
        assert bad.size == 0, f"acc c[{i}] differs in {bad.size} rows, first {bad[:8]}"
