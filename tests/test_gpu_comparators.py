"""GPU parity of the two comparators of the W4A8 GEMM, through the C ABI.

  * W8A8: per-channel INT8 weights in the same kernels and plans; checked
    against the oracle's INT8 weights and exact GEMM (bit-exact INT32, one
    FP16 ulp on outputs).
  * Saturating ablation: the g128 GEMM with a clamping dequantization.  On
    weights from the encoder it must equal the plain GEMM bit for bit; on
    codes whose products leave INT8 it must match the oracle's clamped
    dequantization exactly.
"""

import numpy as np
import pytest

import oracle as O
import synthetic
import w4a8_quantized_gemm_qoq_amd as q
from test_gpu_parity import SMALL, assert_fp16_within_1ulp, dev, gpu_quant

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

# shapes reaching every kernel and launch plan: strip (M <= 16), skinny with
# 16 / 32 / 64-row tiles, skinny up to 256 rows, the three large-M tiles, K
# split over blocks, ragged M and N
W8_SMALL = [s[:4] for s in SMALL if s[3] == 128] + [(1, 256, 27990, 128), (7, 1664, 17000, 128),
                                                    (520, 384, 24400, 128), (1000, 8192, 4000, 128)]


def w8_path(X, W):
    p = q.qoq_pack_weights_w8(W).to("cuda")
    x8, sx = gpu_quant(X)
    y = q.qoq_w8a8_gemm(x8, sx, p)
    acc = q.qoq_w8a8_gemm_i32(x8, p)
    torch.cuda.synchronize()
    return x8.cpu().numpy(), sx.cpu().numpy(), acc.cpu().numpy(), y.cpu().numpy()


@pytest.mark.parametrize("M,K,N,gs", W8_SMALL)
def test_w8a8_small_shapes_match_oracle(M, K, N, gs):
    X = synthetic.make_x(M, K, "frac", seed=M)
    W = synthetic.make_w(N, K, seed=N)
    print(f"[w8a8] M={M} K={K} N={N}", flush=True)
    x8, sx, acc, y = w8_path(X, W)
    ox8, osx, oacc, oy = O.w4a8_forward(X, O.encode_weight_w8(W))
    assert np.array_equal(x8, ox8)
    assert np.array_equal(acc.astype(np.int64), oacc)
    assert_fp16_within_1ulp(y, oy)


@pytest.mark.parametrize("M", [1, 16, 48, 200, 300])
def test_w8a8_full_int8_range(M):
    # random INT8 weights over the whole [-127, 127] range, one scale per
    # channel: the comparator contracts them as they are
    N, K = 96, 640
    rng = np.random.default_rng(M)
    W = (rng.integers(-127, 128, size=(N, K)) / 64.0).astype(np.float16)
    W[:, 0] = 127 / 64.0          # scale = 1/64 exactly, codes = W * 64
    p = q.qoq_pack_weights_w8(W).to("cuda")
    x8 = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    acc = q.qoq_w8a8_gemm_i32(dev(x8), p).cpu().numpy()
    w8 = np.rint(W.astype(np.float64) * 64).astype(np.int64)
    assert np.abs(w8).max() == 127
    assert np.array_equal(acc.astype(np.int64), x8.astype(np.int64) @ w8.T)


W8_FULL = ["attn_proj", "attn_qkv", "ffn_gateup_prefill", "ffn_down_prefill", "decode_m1", "decode_m16",
           "decode_m64", "ffn_large_g128"]


def _sample(w):
    if w.N * w.K <= 64 * 2 ** 20:
        return np.arange(w.M), np.arange(w.N)
    rng = np.random.default_rng(98)
    ns = np.unique(np.r_[rng.choice(w.N, size=254, replace=False), 0, w.N - 1])
    ms = np.arange(w.M) if w.M <= 256 else np.unique(np.r_[rng.choice(w.M, 254, replace=False), 0, w.M - 1])
    return ms, ns


@pytest.mark.parametrize("name", W8_FULL)
def test_w8a8_full_size_sampled(name):
    """The benchmark's shapes, sampled as in the W4A8 full-size test."""
    w = synthetic.get_workload(name)
    X, W = synthetic.make_inputs(w)
    print(f"[w8a8 full] {name} M={w.M} K={w.K} N={w.N}", flush=True)
    x8, sx, acc, y = w8_path(X, W)
    ms, ns = _sample(w)
    ox8, osx = O.quant_act_per_token(X)
    enc = O.encode_weight_w8(W[ns])
    oacc = O.gemm_exact(ox8[ms], enc["w8"])
    assert np.array_equal(acc[np.ix_(ms, ns)].astype(np.int64), oacc)
    assert_fp16_within_1ulp(y[np.ix_(ms, ns)], O.epilogue(oacc, osx[ms], enc["scale"]))


# ------------------------------------------------------------- saturating ablation

SAT_SMALL = [s[:4] for s in SMALL if s[3] == 128]


@pytest.mark.parametrize("M,K,N,gs", SAT_SMALL)
def test_saturating_equals_plain_on_encoded_weights(M, K, N, gs):
    X = synthetic.make_x(M, K, "frac", seed=M + 1)
    W = synthetic.make_w(N, K, seed=N + 1)
    print(f"[sat] M={M} K={K} N={N}", flush=True)
    p = q.qoq_pack_weights(W, 128).to("cuda")
    x8, sx = gpu_quant(X)
    a_plain = q.qoq_w4a8_gemm_i32(x8, p).cpu().numpy()
    a_sat = q.qoq_w4a8_gemm_saturating_i32(x8, p).cpu().numpy()
    y_plain = q.qoq_w4a8_gemm(x8, sx, p).cpu().numpy()
    y_sat = q.qoq_w4a8_gemm_saturating(x8, sx, p).cpu().numpy()
    assert np.array_equal(a_sat, a_plain)
    assert np.array_equal(y_sat.view(np.uint16), y_plain.view(np.uint16))
    enc = O.encode_weight_g128(W)
    assert np.array_equal(a_sat.astype(np.int64), O.gemm_exact(O.quant_act_per_token(X)[0], enc["w8"]))


def meta_offset(n, g, G):
    """Byte of (channel n, group g) in the g128 metadata, as documented in qoq.h."""
    G4 = (G + 3) // 4 * 4
    strip, c = divmod(n, 16)
    return ((strip * (G4 // 4) + g // 4) * 16 + c) * 4 + g % 4


@pytest.mark.parametrize("M,K,N", [(5, 512, 96), (40, 512, 200), (300, 512, 640), (512, 256, 24576)])
def test_saturating_clamps_out_of_range_products(M, K, N):
    """Metadata rewritten to s1 = 16 with z = 0 or 15 (and s1 = 9, z = 0):
    (q4 - z) * s1 reaches +-240, far outside INT8; the saturating GEMM must
    contract clamp((q4 - z) * s1, -128, 127)."""
    G = K // 128
    rng = np.random.default_rng(M + N)
    W = synthetic.make_w(N, K, seed=3)
    enc = O.encode_weight_g128(W)
    p = q.qoq_pack_weights(W, 128)
    s1 = enc["s1"].astype(np.int64).copy()
    z = enc["z"].astype(np.int64).copy()
    meta = np.array(p.meta, copy=True)
    kinds = rng.integers(0, 4, size=(N, G))   # 0: unchanged, 1: (16, 0), 2: (16, 15), 3: (9, 0)
    for n in range(N):
        for g in range(G):
            k = kinds[n, g]
            if k == 0:
                continue
            s1[n, g], z[n, g] = {1: (16, 0), 2: (16, 15), 3: (9, 0)}[int(k)]
            meta[meta_offset(n, g, G)] = (s1[n, g] - 1) | (z[n, g] << 4)
    pd = q.PackedWeight(p.qweight, meta, p.scale, N, K, 128).to("cuda")
    w8 = O.dequant_level1_saturating(enc["q4"], s1, z)
    assert w8.max() == 127 and w8.min() == -128
    x8 = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    print(f"[sat clamp] M={M} K={K} N={N}", flush=True)
    acc = q.qoq_w4a8_gemm_saturating_i32(dev(x8), pd).cpu().numpy()
    assert np.array_equal(acc.astype(np.int64), O.gemm_exact(x8, w8))


SAT_FULL = ["attn_proj", "ffn_gateup_prefill", "decode_m16", "decode_m64", "ffn_large_g128"]


@pytest.mark.parametrize("name", SAT_FULL)
def test_saturating_full_size_equals_plain(name):
    """The benchmark's shapes: the ablation's output equals the plain GEMM's
    bit for bit over the whole output (the plain one is checked against the
    oracle by the W4A8 full-size test)."""
    w = synthetic.get_workload(name)
    X, W = synthetic.make_inputs(w)
    print(f"[sat full] {name} M={w.M} K={w.K} N={w.N}", flush=True)
    p = q.qoq_pack_weights(W, 128).to("cuda")
    x8, sx = gpu_quant(X)
    y_plain = q.qoq_w4a8_gemm(x8, sx, p)
    y_sat = q.qoq_w4a8_gemm_saturating(x8, sx, p)
    assert torch.equal(y_plain.view(torch.int16), y_sat.view(torch.int16))
    a_plain = q.qoq_w4a8_gemm_i32(x8, p)
    a_sat = q.qoq_w4a8_gemm_saturating_i32(x8, p)
    assert torch.equal(a_plain, a_sat)
