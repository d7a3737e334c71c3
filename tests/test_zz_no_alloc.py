"""The allocation-free GEMM entry point (qoq_w4a8_gemm_noalloc) against the
workspace entry point (qoq_w4a8_gemm) on the same inputs, through the C ABI:
bit-identical FP16 outputs, and within one FP16 ulp of the oracle.  Two calls
in a row share the library's scratch; the second has a smaller input, so a
stale partial from the first call would show.  Collected last so that a
failure here cannot hide other tests."""

import numpy as np
import pytest

import oracle as O
import synthetic
import w4a8_quantized_gemm_qoq_amd as q

pytestmark = pytest.mark.gpu


def _ulp16(v):
    return 2.0 ** (np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -14))) - 10)


def _run_pair(torch, M, N, K, gs, seed):
    dev = torch.device("cuda")
    X = synthetic.make_x(M, K, "frac", seed=seed)
    W = synthetic.make_w(N, K, seed=seed)
    lib = q.load_library()
    need = lib.qoq_w4a8_gemm_workspace_size(M, N, K, gs)
    p = q.qoq_pack_weights(W, gs).to(dev)
    x8, sx = q.qoq_quant_act_per_token(torch.from_numpy(X).to(dev))
    y_ref = q.qoq_w4a8_gemm(x8, sx, p)
    y = torch.full((M, N), float("nan"), dtype=torch.float16, device=dev)
    q.qoq_w4a8_gemm_noalloc(x8, sx, p, y)
    torch.cuda.synchronize()
    return X, W, need, y.cpu().numpy(), y_ref.cpu().numpy()


@pytest.mark.parametrize("gs", [128, 0])
def test_noalloc_matches_workspace_entry_on_two_calls(gs):
    import torch
    # (M, N, K): both plans split K (16 MiB, then 9.4 MiB of partials); the
    # second input is smaller, so it reuses only part of what the first wrote
    shapes = [(512, 4096, 4096), (300, 4096, 4096)]
    for i, (M, N, K) in enumerate(shapes):
        print(f"noalloc case gs={gs} M={M} N={N} K={K}", flush=True)
        X, W, need, y, y_ref = _run_pair(torch, M, N, K, gs, seed=10 + i)
        assert 0 < need <= q.NOALLOC_SCRATCH_BYTES, need
        assert np.array_equal(y.view(np.uint16), y_ref.view(np.uint16)), f"call {i}: differs from qoq_w4a8_gemm"
        enc = O.encode_weight_g128(W) if gs else O.encode_weight_per_channel(W)
        _, _, _, oy = O.w4a8_forward(X, enc)
        yr = oy.astype(np.float64)
        assert np.all(np.abs(y.astype(np.float64) - yr) <= _ulp16(yr)), f"call {i}: off the oracle by > 1 ulp"


def test_noalloc_plans_without_scratch_and_rejects_oversized_shapes():
    import torch
    dev = torch.device("cuda")
    # a decode shape (no split, the scratch is not touched)
    print("noalloc case M=16 N=4096 K=4096 (no split)", flush=True)
    X, W, need, y, y_ref = _run_pair(torch, 16, 4096, 4096, 128, seed=12)
    assert need == 0
    assert np.array_equal(y.view(np.uint16), y_ref.view(np.uint16))
    # 768 x 4096 x 16384 would need 48 MiB of partials: rejected before launch
    lib = q.load_library()
    M, N, K = 768, 4096, 16384
    assert lib.qoq_w4a8_gemm_workspace_size(M, N, K, 128) > q.NOALLOC_SCRATCH_BYTES
    p = q.qoq_pack_weights(synthetic.make_w(N, K, seed=13), 128).to(dev)
    x8 = torch.zeros((M, K), dtype=torch.int8, device=dev)
    sx = torch.zeros((M,), dtype=torch.float16, device=dev)
    yb = torch.empty((M, N), dtype=torch.float16, device=dev)
    with pytest.raises(q.QoQError, match="split-K scratch"):
        q.qoq_w4a8_gemm_noalloc(x8, sx, p, yb)
