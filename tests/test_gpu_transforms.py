"""The W4A8 path on transformed tensors (offline rotation and smoothing):
GPU parity with the oracle on the oracle's own transformed inputs, and the
effect of the transforms on the activation quantization (printed)."""

import numpy as np
import pytest

import oracle as O
import synthetic
from test_gpu_parity import assert_fp16_within_1ulp, run_path

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def act_err(x8, sx, X):
    d = x8.astype(np.float64) * sx.astype(np.float64)[:, None]
    return np.linalg.norm(d - X.astype(np.float64)) / np.linalg.norm(X.astype(np.float64))


@pytest.mark.parametrize("M,K,N,transform", [(64, 4096, 512, "rotate"), (33, 14336, 256, "rotate"),
                                             (256, 4096, 1024, "smooth"), (16, 1024, 256, "rotate+smooth")])
def test_w4a8_on_transformed_tensors(M, K, N, transform):
    X = synthetic.make_x(M, K, "frac", seed=K)
    W = synthetic.make_w(N, K, seed=K)
    Xt, Wt = X, W
    if "rotate" in transform:
        Xt, Wt = O.rotate_rows(Xt), O.rotate_rows(Wt)
    if "smooth" in transform:
        lam = O.smoothing_factors(np.abs(Xt.astype(np.float32)).max(0), np.abs(Wt.astype(np.float32)).max(0), 0.5)
        Xt, Wt = O.scale_columns(Xt, lam, divide=True), O.scale_columns(Wt, lam)
    x8, sx, acc, y, _ = run_path(Xt, Wt, 128)
    ox8, osx, oacc, oy = O.w4a8_forward(Xt, O.encode_weight_g128(Wt))
    assert np.array_equal(x8, ox8) and np.array_equal(acc.astype(np.int64), oacc)
    assert_fp16_within_1ulp(y, oy)
    # effect on the per-token INT8 step (same vectors in the rotated basis;
    # for smoothing, relative to the smoothed activations)
    x8p, sxp, _, _, _ = run_path(X, W, 128)
    print(f"[transform] {transform} M={M} K={K}: activation error {act_err(x8p, sxp, X):.4f} -> "
          f"{act_err(x8, sx, Xt):.4f}", flush=True)
