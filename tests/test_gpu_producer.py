"""GPU parity of the fused producer (RMS normalization + per-token INT8
quantization) against the CPU oracle, through the C ABI: x8 and the FP16
scales bit for bit."""

import numpy as np
import pytest

import oracle as O
import synthetic
import w4a8_quantized_gemm_qoq_amd as q
from golden_io import read_fixture

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def gpu_rmsnorm_quant(X, g, eps, x=None):
    x = dev(X) if x is None else x
    x8, sx = q.qoq_rmsnorm_quant_per_token(x, dev(g), eps)
    return x8.cpu().numpy(), sx.cpu().numpy()


def check(X, g, eps, x=None):
    x8, sx = gpu_rmsnorm_quant(X, g, eps, x)
    ox8, osx = O.rmsnorm_quant_per_token(X, g, eps)
    assert np.array_equal(sx.view(np.uint16), osx.view(np.uint16))
    assert np.array_equal(x8, ox8)


def test_hand_worked_rows_gpu():
    fx = read_fixture("rmsnorm_quant_rows.txt")
    for r in "ab":
        X = np.array([fx["x" + r]], np.float16)
        x8, sx = gpu_rmsnorm_quant(X, np.array(fx["g" + r], np.float16), fx["eps"][0])
        assert float(sx[0]) == fx["s" + r][0]
        assert x8[0].tolist() == [int(v) for v in fx["q" + r]]


# register path (K up to 16384, 1 to 8 vectors per thread), streaming path
# (longer rows) and scalar path (K not a multiple of 8)
@pytest.mark.parametrize("M,K,eps", [(1, 4096, 1e-5), (16, 4096, 1e-6), (256, 4096, 1e-5), (7, 8192, 1e-5),
                                     (33, 14336, 1e-6), (3, 24576, 1e-5), (5, 1001, 1e-5), (4, 2048, 1e-5),
                                     (2, 16384, 1e-5), (9, 16392, 1e-5), (6, 8, 1e-3)])
def test_matches_oracle(M, K, eps):
    print(f"[rmsnorm] M={M} K={K}", flush=True)
    check(synthetic.make_x(M, K, "frac", seed=M + K), synthetic.make_gamma(K, seed=K), eps)


def test_strided_rows_and_edge_rows():
    M, K, ld = 8, 512, 520
    rng = np.random.default_rng(4)
    full = rng.standard_normal((M, ld)).astype(np.float16)
    full[0, :K] = 0                                  # zero row
    full[1, :K] = np.float16(6e-8)                   # FP16 subnormals only
    full[2, :K] = 2.0 ** -24; full[2, 0] = 60000.0   # one huge entry over tiny ones
    full[3, :K] = 0.25                               # constant power of two
    full[4, :K:3] *= 500                             # wide values
    full[5, :K] = 0; full[5, 7] = -3.0               # single spike
    g = synthetic.make_gamma(K, seed=1)
    x = dev(full)[:, :K]
    assert x.stride(0) == ld
    check(full[:, :K], g, 1e-5, x=x)
    check(full[:, :K], g, 2.0 ** -40, x=x)


@pytest.mark.parametrize("name", ["attn_proj", "ffn_gateup_prefill", "decode_m64", "ffn_large_g128"])
def test_full_size_rows(name):
    """The (M, K) of the layers a normalization feeds, all rows."""
    w = synthetic.get_workload(name)
    print(f"[rmsnorm full] {name} M={w.M} K={w.K}", flush=True)
    check(synthetic.make_x(w.M, w.K, w.outliers), synthetic.make_gamma(w.K), 1e-5)


def test_binding_rejects_bad_arguments():
    x = torch.zeros((4, 128), dtype=torch.float16, device="cuda")
    with pytest.raises(ValueError):
        q.qoq_rmsnorm_quant_per_token(x, torch.ones(64, dtype=torch.float16, device="cuda"), 1e-5)
    with pytest.raises(q.QoQError):
        q.qoq_rmsnorm_quant_per_token(x, torch.ones(128, dtype=torch.float16, device="cuda"), 0.0)


def boundary_rows(K, n, seed):
    """Rows whose exact mean square is an FP32 rounding tie (even rows) or
    lies 2^-48 / K above one (odd rows): [1, 1, m3 2^-12, m4 2^-12, (2^-24),
    0, ...] with m3, m4 odd, so S = 2 + (m3^2 + m4^2) 2^-24 with m3^2 + m4^2
    twice an odd number; for K a power of two, S / K is an odd multiple of
    half the FP32 spacing of its binade.  The kernel's FP64 sum cannot decide
    such rows and takes the exact 128-bit sum."""
    rng = np.random.default_rng(seed)
    X = np.zeros((n, K), np.float16)
    for r in range(n):
        m3, m4 = (2 * rng.integers(0, 1024, 2) + 1).tolist()
        X[r, 0] = X[r, 1] = 1.0
        X[r, 2], X[r, 3] = m3 * 2.0 ** -12, -m4 * 2.0 ** -12
        if r % 2:
            X[r, 4] = 2.0 ** -24
        perm = rng.permutation(K)
        X[r] = X[r, perm]
        # the tie property, from the exact sum (every FP16 value is an integer times 2^-24)
        units = (X[r].astype(np.float64) * 2.0 ** 24).astype(np.int64).tolist()
        S = sum(v * v for v in units)                     # units of 2^-48
        half = 2 ** 25                                    # half the FP32 spacing of [2, 4) (2^-23), units of 2^-48
        assert (S - 2 * 2 ** 48) % half == (0 if r % 2 == 0 else 1) and ((S - 2 * 2 ** 48) // half) % 2 == 1
    return X


@pytest.mark.parametrize("K", [1024, 4096, 8192, 16384])
def test_mean_square_at_fp32_rounding_boundaries(K):
    """Rows the FP64 fast path must hand to the exact sum (ties and near-ties
    of the FP32 mean square), through every register-path width; the oracle
    rounds the exact S."""
    print(f"[rmsnorm ties] K={K}", flush=True)
    X = boundary_rows(K, 12, seed=K)
    g = synthetic.make_gamma(K, seed=3)
    check(X, g, 1e-5)
    check(X, g, 2.0 ** -40)
