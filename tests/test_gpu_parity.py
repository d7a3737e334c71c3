"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Bar: bit-exact for the INT8 activations, FP16 activation scales and INT32
accumulators; within one FP16 ulp of the oracle's correctly rounded value for
the FP16 outputs.
"""

import numpy as np
import pytest

import oracle as O
import synthetic
import w4a8_quantized_gemm_qoq_amd as q

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def ulp16(v):
    """One FP16 ulp at the magnitude of v (2^-24 in the subnormal range)."""
    a = np.abs(np.asarray(v, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
    return 2.0 ** (e - 10)


def assert_fp16_within_1ulp(y_gpu, y_ref):
    yg = np.asarray(y_gpu, np.float16).astype(np.float64)
    yr = np.asarray(y_ref, np.float16).astype(np.float64)
    assert np.all(np.isfinite(yg)), "non-finite output"
    d = np.abs(yg - yr)
    tol = ulp16(yr)
    bad = d > tol
    assert not bad.any(), f"{bad.sum()} outputs off by more than 1 ulp; worst {d[bad].max()}"


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def gpu_quant(X):
    x = dev(X)
    x8, sx = q.qoq_quant_act_per_token(x)
    return x8, sx


def run_path(X, W, group_size):
    """GPU path: pack on host, quantize + GEMM (+ INT32 debug) on the GPU."""
    p = q.qoq_pack_weights(W, group_size).to("cuda")
    x8, sx = gpu_quant(X)
    y = q.qoq_w4a8_gemm(x8, sx, p)
    acc = q.qoq_w4a8_gemm_i32(x8, p)
    torch.cuda.synchronize()
    return x8.cpu().numpy(), sx.cpu().numpy(), acc.cpu().numpy(), y.cpu().numpy(), p


def oracle_path(X, W, group_size):
    enc = O.encode_weight_g128(W) if group_size else O.encode_weight_per_channel(W)
    return O.w4a8_forward(X, enc)


# ------------------------------------------------------------- activation quant

def test_act_quant_hand_worked_rows_gpu():
    from golden_io import read_fixture
    fx = read_fixture("act_quant_rows.txt")
    X = np.array([fx[f"x{i}"] for i in range(5)], dtype=np.float16)
    for K in (12, 128):   # scalar path (K = 12) and vector path (zero padded)
        Xp = np.zeros((5, K), np.float16)
        Xp[:, :12] = X
        x8, sx = gpu_quant(Xp)
        x8 = x8.cpu().numpy()
        sx = sx.cpu().numpy()
        for i in range(5):
            assert float(sx[i]) == fx[f"s{i}"][0]
            assert x8[i, :12].tolist() == [int(v) for v in fx[f"q{i}"]]
            assert not x8[i, 12:].any()


@pytest.mark.parametrize("M,K", [(1, 128), (16, 256), (7, 1000), (64, 4096), (33, 8192), (5, 14336), (3, 24576)])
def test_act_quant_bit_exact(M, K):
    X = synthetic.make_x(M, K, "frac", seed=M + K)
    x8, sx = gpu_quant(X)
    ox8, osx = O.quant_act_per_token(X)
    assert np.array_equal(x8.cpu().numpy(), ox8)
    assert np.array_equal(sx.cpu().numpy().view(np.uint16), osx.view(np.uint16))


def test_act_quant_strided_rows_and_edge_values():
    M, K, ld = 9, 512, 520
    rng = np.random.default_rng(5)
    full = rng.standard_normal((M, ld)).astype(np.float16)
    full[0, :K] = 0                         # zero row
    full[1, :K] = 0; full[1, 17] = -65504   # negative max at the FP16 extreme
    full[2, :K] = np.float16(6e-8)          # subnormals
    full[3, :K] = 0; full[3, 3] = 2.0 ** -17
    full[4, :K:2] *= 300
    x = dev(full)[:, :K]
    assert x.stride(0) == ld
    x8, sx = q.qoq_quant_act_per_token(x)
    ox8, osx = O.quant_act_per_token(full[:, :K])
    assert np.array_equal(x8.cpu().numpy(), ox8)
    assert np.array_equal(sx.cpu().numpy().view(np.uint16), osx.view(np.uint16))


# ------------------------------------------------------------- GEMM, small shapes

from gemm_cases import SMALL  # noqa: E402  (shapes and the launch plan each reaches)


@pytest.mark.parametrize("M,K,N,gs,plan", SMALL)
def test_gemm_small_shapes_match_oracle(M, K, N, gs, plan):
    assert q.qoq_w4a8_gemm_plan(M, N, K, gs) == plan
    X = synthetic.make_x(M, K, "frac", seed=M)
    W = synthetic.make_w(N, K, seed=N)
    x8, sx, acc, y, _ = run_path(X, W, gs)
    ox8, osx, oacc, oy = oracle_path(X, W, gs)
    assert np.array_equal(x8, ox8)
    assert np.array_equal(sx.view(np.uint16), osx.view(np.uint16))
    assert np.array_equal(acc.astype(np.int64), oacc)
    assert_fp16_within_1ulp(y, oy)


@pytest.mark.parametrize("gs", [128, 0])
def test_tiny_workload_full_parity(gs):
    X, W = synthetic.make_inputs("tiny")
    x8, sx, acc, y, _ = run_path(X, W, gs)
    ox8, osx, oacc, oy = oracle_path(X, W, gs)
    assert np.array_equal(x8, ox8) and np.array_equal(acc.astype(np.int64), oacc)
    assert_fp16_within_1ulp(y, oy)


@pytest.mark.parametrize("M", [1, 16, 64, 128, 256])
def test_identity_probe_pins_layout(M):
    # one-hot activation rows x8 = 127 * e_k give acc[m, :] = 127 * w8[:, k]
    N, K = 48, 384
    W = synthetic.make_w(N, K, seed=21)
    enc = O.encode_weight_g128(W)
    p = q.qoq_pack_weights(W, 128).to("cuda")
    ks = np.random.default_rng(M).integers(0, K, size=M)
    x8 = np.zeros((M, K), np.int8)
    x8[np.arange(M), ks] = 127
    acc = q.qoq_w4a8_gemm_i32(dev(x8), p).cpu().numpy()
    assert np.array_equal(acc.astype(np.int64), 127 * enc["w8"][:, ks].T)


@pytest.mark.parametrize("M", [3, 64, 200])
def test_textbook_int8_gemm_reduction(M):
    # s1 = 1 and z = 8 everywhere: W4A8 reduces to a plain INT8 GEMM with
    # weights q4 - 8 in [-8, 7], checked against an int64 matmul
    N, K = 80, 512
    rng = np.random.default_rng(M)
    q4 = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    p = q.qoq_pack_codes(q4, np.ones((N, K // 128), np.uint8), np.full((N, K // 128), 8, np.uint8),
                         np.ones(N, np.float16), 128).to("cuda")
    x8 = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    acc = q.qoq_w4a8_gemm_i32(dev(x8), p).cpu().numpy()
    ref = x8.astype(np.int64) @ (q4.astype(np.int64) - 8).T
    assert np.array_equal(acc.astype(np.int64), ref)


@pytest.mark.parametrize("M", [16, 96])
def test_extreme_valid_bytes(M):
    # the byte extremes of the packed dequantization: w8 = -128 (z*s1 = 128,
    # q4 = 0), w8 = 112, w8 = +-121-range products, x8 = +-127
    N, K = 32, 256
    G = K // 128
    rng = np.random.default_rng(7)
    s1 = np.full((N, G), 16, np.uint8)
    z = np.full((N, G), 8, np.uint8)
    q4 = rng.choice(np.array([0, 15, 8, 1], np.uint8), size=(N, K))
    s1[::2] = 11; z[::2] = 11     # w8 in [-121, 44]
    q4[::2] = rng.choice(np.array([0, 15], np.uint8), size=(N // 2, K))
    p = q.qoq_pack_codes(q4, s1, z, np.ones(N, np.float16), 128).to("cuda")
    x8 = rng.choice(np.array([-127, 127], np.int8), size=(M, K))
    acc = q.qoq_w4a8_gemm_i32(dev(x8), p).cpu().numpy()
    w8 = (q4.astype(np.int64) - np.repeat(z, 128, 1)) * np.repeat(s1, 128, 1)
    assert w8.min() == -128
    assert np.array_equal(acc.astype(np.int64), x8.astype(np.int64) @ w8.T)


@pytest.mark.parametrize("M", [1, 24, 64, 300])  # strip, 32-row skinny, 64-row skinny, large kernel
def test_every_valid_metadata_byte(M):
    # Every (s1, z) pair whose dequantized bytes q4*s1 + 128 - z*s1 stay in
    # [0, 255] for all q4 (the condition of the carry-free packed form), cycled
    # over 48 channels x 8 groups, through each kernel's metadata decode;
    # INT32 accumulators against an int64 matmul.
    N, K = 48, 1024
    G = K // 128
    pairs = [(s, zz) for s in range(1, 17) for zz in range(16) if zz * s <= 128 and s * (15 - zz) <= 127]
    assert len(pairs) == 177
    rng = np.random.default_rng(M)
    idx = (np.arange(N * G) + M) % len(pairs)
    s1 = np.array([pairs[i][0] for i in idx], np.uint8).reshape(N, G)
    z = np.array([pairs[i][1] for i in idx], np.uint8).reshape(N, G)
    q4 = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    p = q.qoq_pack_codes(q4, s1, z, np.ones(N, np.float16), 128).to("cuda")
    x8 = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    print(f"[meta bytes] M={M}", flush=True)
    acc = q.qoq_w4a8_gemm_i32(dev(x8), p).cpu().numpy()
    w8 = (q4.astype(np.int64) - np.repeat(z, 128, 1)) * np.repeat(s1, 128, 1).astype(np.int64)
    assert w8.min() >= -128 and w8.max() <= 127
    assert np.array_equal(acc.astype(np.int64), x8.astype(np.int64) @ w8.T)


# largest multiple of 128 with 127 * 127 * K below 2^31 (the INT32 bound the packer enforces)
KMAX = 133120


@pytest.mark.parametrize("M,N", [(1, 40),     # strip kernel, activations and metadata fill 147 KB of LDS
                                 (16, 48),    # activations exceed LDS: 16-row skinny kernel
                                 (64, 40),    # 64-row skinny kernel, 260 groups per wave
                                 (300, 64)])  # large kernel, small tile, K split 128 ways + reduction
def test_max_k_near_int32_bound(M, N):
    # K at the INT32 limit through every launch plan.  Row 0 of the weights is
    # w8 = 121 throughout and row 0 of the activations 127, so accumulator
    # (0, 0) is 127 * 121 * K, 95% of 2^31.  Sampled rows against an int64
    # matmul of the reconstructed INT8 weights.
    K = KMAX
    G = K // 128
    rng = np.random.default_rng(M + N)
    q4 = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    s1 = rng.integers(1, 9, size=(N, G)).astype(np.uint8)   # |w8| <= 120, bytes in [8, 248]
    z = rng.integers(0, 16, size=(N, G)).astype(np.uint8)
    q4[0] = 11
    s1[0] = 11
    z[0] = 0
    p = q.qoq_pack_codes(q4, s1, z, np.ones(N, np.float16), 128).to("cuda")
    x8 = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    x8[0] = 127
    print(f"[max K] M={M} N={N} K={K}", flush=True)
    acc = q.qoq_w4a8_gemm_i32(dev(x8), p).cpu().numpy()
    rows = sorted({0, M // 2, M - 1})
    w8 = (q4.astype(np.int64) - np.repeat(z, 128, 1)) * np.repeat(s1, 128, 1).astype(np.int64)
    ref = x8[rows].astype(np.int64) @ w8.T
    assert ref[0, 0] == 127 * 121 * K
    assert np.array_equal(acc[rows].astype(np.int64), ref)


def test_output_canaries_and_determinism():
    M, K, N = 70, 512, 100
    X = synthetic.make_x(M, K, "frac", seed=1)
    W = synthetic.make_w(N, K, seed=2)
    p = q.qoq_pack_weights(W, 128).to("cuda")
    x8, sx = gpu_quant(X)
    ld = N + 24
    yfull = torch.full((M, ld), float("nan"), dtype=torch.float16, device="cuda")
    y = yfull[:, :N]
    q.qoq_w4a8_gemm(x8, sx, p, y=y)
    y2 = q.qoq_w4a8_gemm(x8, sx, p)
    torch.cuda.synchronize()
    yf = yfull.cpu().numpy()
    assert np.all(np.isfinite(yf[:, :N]))
    assert np.all(np.isnan(yf[:, N:]))          # nothing written past N
    assert np.array_equal(yf[:, :N].view(np.uint16), y2.cpu().numpy().view(np.uint16))
    a1 = q.qoq_w4a8_gemm_i32(x8, p).cpu().numpy()
    a2 = q.qoq_w4a8_gemm_i32(x8, p).cpu().numpy()
    assert np.array_equal(a1, a2)


def test_python_binding_rejects_bad_tensors():
    p = q.qoq_pack_weights(synthetic.make_w(16, 128), 128).to("cuda")
    x8 = torch.zeros((4, 256), dtype=torch.int8, device="cuda")
    with pytest.raises(ValueError):
        q.qoq_w4a8_gemm_i32(x8, p)       # K mismatch
    with pytest.raises(ValueError):
        q.qoq_quant_act_per_token(torch.zeros((4, 128), dtype=torch.float32, device="cuda"))


# ------------------------------------------------------------- full-size workloads

FULL = ["attn_proj", "attn_qkv", "ffn_gateup_prefill", "ffn_down_prefill", "decode_m1", "decode_m16",
        "decode_m64", "ffn_large_g128", "ffn_large_perchannel"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_workload_parity(name):
    """Full-size run in the benchmark's launch configuration.  Activations are
    checked in full.  Accumulators and outputs are checked in full where the
    weight matrix has at most 64M entries, otherwise on 256 sampled output
    channels x up to 256 tokens that the oracle computes one by one (its
    weight quantization is local to an output channel, its activation
    quantization local to a token)."""
    w = synthetic.get_workload(name)
    X, W = synthetic.make_inputs(w)
    print(f"[full] {name} M={w.M} K={w.K} N={w.N} gs={w.group_size}", flush=True)
    x8, sx, acc, y, _ = run_path(X, W, w.group_size)
    ox8, osx = O.quant_act_per_token(X)
    assert np.array_equal(x8, ox8)
    assert np.array_equal(sx.view(np.uint16), osx.view(np.uint16))
    if w.N * w.K <= 64 * 2 ** 20:
        ms, ns = np.arange(w.M), np.arange(w.N)
    else:
        rng = np.random.default_rng(99)
        ns = np.unique(np.r_[rng.choice(w.N, size=254, replace=False), 0, w.N - 1])
        ms = np.arange(w.M) if w.M <= 256 else np.unique(np.r_[rng.choice(w.M, 254, replace=False), 0, w.M - 1])
    enc = O.encode_weight_g128(W[ns]) if w.group_size else O.encode_weight_per_channel(W[ns])
    oacc = O.gemm_exact(ox8[ms], enc["w8"])
    assert np.array_equal(acc[np.ix_(ms, ns)].astype(np.int64), oacc)
    assert_fp16_within_1ulp(y[np.ix_(ms, ns)], O.epilogue(oacc, osx[ms], enc["scale"]))
