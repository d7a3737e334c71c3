"""GPU parity of the KV4 kernels against the CPU oracle, through the C ABI.

  * Quantization: codes, FP16 scales and zero points bit for bit.
  * Decode attention: the oracle evaluates it in FP64 from its own quantized
    cache (packed here into the documented byte layout); the kernel computes
    in FP32.  Per (sequence, head) the bar is
        |o_gpu - o_ref| <= ulp16(o_ref) + 2^-12 * max_t |v_t|
    -- one FP16 rounding of the output plus the FP32 error of the scores
    (about K * 2^-24 relative to sum |q k|), of exp, and of a sum of up to
    T weighted values, each bounded well below 2^-12 of the value range.
"""

import numpy as np
import pytest

import oracle as O
import w4a8_quantized_gemm_qoq_amd as q
from kv4_cases import EDGE, PLAIN, SPLIT

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SCALE = float(np.float32(1.0 / np.sqrt(128.0)))


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def pack_codes(c):
    """Documented cache byte layout: byte j = code(2j) | code(2j+1) << 4."""
    c = np.asarray(c, np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def ulp16(v):
    a = np.abs(np.asarray(v, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
    return 2.0 ** (e - 10)


def rows(n, seed, kind="normal"):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((n, 128)).astype(np.float32)
    if kind == "outliers":
        X[:, rng.choice(128, 3, replace=False)] *= 20
    return X.astype(np.float16)


@pytest.mark.parametrize("n,kind", [(1, "normal"), (64, "normal"), (1000, "outliers"), (4096 * 3, "normal")])
def test_kv4_quant_bit_exact(n, kind):
    X = rows(n, seed=n, kind=kind)
    codes, s, z = q.qoq_kv4_quant(dev(X))
    oq, os_, oz = O.kv4_quant_per_head(X)
    assert np.array_equal(codes.cpu().numpy(), pack_codes(oq))
    assert np.array_equal(s.cpu().numpy().view(np.uint16), os_.view(np.uint16))
    assert np.array_equal(z.cpu().numpy(), oz)


def test_kv4_quant_edge_rows():
    X = rows(8, seed=1)
    X[0] = 0                              # zero row: zero scale and codes
    X[1] = 3.0                            # constant row: zero range
    X[2] = np.float16(6e-8)               # subnormals
    X[3, :] = 0; X[3, 5] = -65504         # FP16 extreme, one sign
    X[4, ::2] = 65504; X[4, 1::2] = -65504
    X[5] = np.linspace(-1, 1, 128)
    codes, s, z = q.qoq_kv4_quant(dev(X))
    oq, os_, oz = O.kv4_quant_per_head(X)
    assert np.array_equal(codes.cpu().numpy(), pack_codes(oq))
    assert np.array_equal(s.cpu().numpy().view(np.uint16), os_.view(np.uint16))
    assert np.array_equal(z.cpu().numpy(), oz)


def make_cache(B, Hkv, T, seed, peak=1.0):
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((B, Hkv, T, 128)).astype(np.float16)
    V = rng.standard_normal((B, Hkv, T, 128)).astype(np.float16)
    return O.kv4_quant_per_head(K), O.kv4_quant_per_head(V)


def run_attention(Q, kk, vv, lengths, split=False):
    k = (dev(pack_codes(kk[0])), dev(kk[1]), dev(kk[2]))
    v = (dev(pack_codes(vv[0])), dev(vv[1]), dev(vv[2]))
    o = q.qoq_kv4_decode_attention(dev(Q), k, v, dev(np.asarray(lengths, np.int32)), SCALE, split=split)
    return o.cpu().numpy()


def check_attention(Q, kk, vv, lengths, split=False):
    o = run_attention(Q, kk, vv, lengths, split).astype(np.float64)
    ref = O.kv4_decode_attention(Q, *kk, *vv, lengths, SCALE).astype(np.float64)
    B, H, _ = Q.shape
    Hkv = kk[0].shape[1]
    vmax = np.zeros((B, H))
    Vd = np.abs(O.kv4_dequant(*vv))
    for b in range(B):
        L = min(max(int(lengths[b]), 0), kk[0].shape[2])
        for h in range(H):
            vmax[b, h] = Vd[b, h // (H // Hkv), :L].max() if L else 0.0
    tol = ulp16(ref) + 2.0 ** -12 * vmax[..., None]
    err = np.abs(o - ref)
    worst = float((err / tol).max())
    print(f"[kv4 attn] B={B} H={H} Hkv={Hkv} split={split} worst err/tol = {worst:.3f}", flush=True)
    assert np.all(np.isfinite(o))
    assert np.all(err <= tol), f"worst err/tol {worst}"
    for b in range(B):
        if int(lengths[b]) <= 0:
            assert not o[b].any()


def assert_plan(B, H, Hkv, T, split, plan):
    """The launch plan the shape reaches (pinned in kv4_cases.py)."""
    assert q.qoq_kv4_decode_attention_plan(B, H, Hkv, T, split=split) == tuple(plan)


@pytest.mark.parametrize("B,H,Hkv,T,lengths,peak,plan", PLAIN)
def test_kv4_attention_matches_oracle(B, H, Hkv, T, lengths, peak, plan):
    assert_plan(B, H, Hkv, T, False, plan)
    kk, vv = make_cache(B, Hkv, T, seed=T + H)
    Q = (np.random.default_rng(B).standard_normal((B, H, 128)) * peak).astype(np.float16)
    check_attention(Q, kk, vv, lengths)


@pytest.mark.parametrize("B,H,Hkv,T,split,plan", EDGE)
def test_kv4_attention_query_edge_cases(B, H, Hkv, T, split, plan):
    """Queries that stress the three-piece INT8 split of the scaled query: a
    zero head (all pieces zero: uniform weights), one FP16-max entry, FP16
    subnormals only, all dims equal, and alternating signs at the FP16 max;
    once for every kernel family (1, 2 and 4 heads a workgroup, split or not)."""
    assert_plan(B, H, Hkv, T, split, plan)
    kk, vv = make_cache(B, Hkv, T, seed=77)
    Q = np.random.default_rng(77).standard_normal((B, H, 128)).astype(np.float16)
    Q[0, 0] = 0
    Q[0, 1] = 0
    Q[0, 1, 17] = 65504
    Q[0, 2] = np.float16(6e-8) * np.sign(np.random.default_rng(1).standard_normal(128)).astype(np.float16)
    Q[0, 3] = np.float16(0.3)
    Q[0, 4, ::2] = 65504
    Q[0, 4, 1::2] = -65504
    lengths = [T - 1] + [T] * (B - 1)
    check_attention(Q, kk, vv, lengths, split=split)


def test_kv4_attention_lengths_clamped_to_cache():
    kk, vv = make_cache(2, 2, 32, seed=3)
    Q = np.random.default_rng(0).standard_normal((2, 2, 128)).astype(np.float16)
    o = run_attention(Q, kk, vv, [100, -5])
    ref = O.kv4_decode_attention(Q, *kk, *vv, [32, 0], SCALE)
    assert np.array_equal(o[1], ref[1])          # negative length: zeros
    check_attention(Q, kk, vv, [32, 0])


@pytest.mark.parametrize("H,Hkv", [(32, 32), (32, 8)])
def test_kv4_attention_bench_shape(H, Hkv):
    """The benchmark's decode shape (64 sequences x 1024 cached tokens),
    every head checked."""
    B, T = 64, 1024
    kk, vv = make_cache(B, Hkv, T, seed=H + Hkv)
    Q = np.random.default_rng(7).standard_normal((B, H, 128)).astype(np.float16)
    check_attention(Q, kk, vv, [T] * B)


# Token-split attention: chunks of the cache over more workgroups, their
# softmax partials combined afterwards.  Same oracle, same tolerance.
@pytest.mark.parametrize("B,H,Hkv,T,lengths,peak,plan", SPLIT)
def test_kv4_attention_split_matches_oracle(B, H, Hkv, T, lengths, peak, plan):
    assert_plan(B, H, Hkv, T, True, plan)
    assert q.qoq_kv4_decode_attention_workspace_size(B, H, Hkv, T) > 0
    kk, vv = make_cache(B, Hkv, T, seed=T + 3 * H)
    Q = (np.random.default_rng(B + 11).standard_normal((B, H, 128)) * peak).astype(np.float16)
    check_attention(Q, kk, vv, lengths, split=True)


def test_kv4_attention_split_entry_without_split_is_the_plain_kernel():
    """Shapes that are not split (here 64 x 32 heads: 512 workgroups already)
    run the single-pass kernel through the split entry: identical bits."""
    B, H, Hkv, T = 64, 32, 8, 600
    assert q.qoq_kv4_decode_attention_workspace_size(B, H, Hkv, T) == 0
    kk, vv = make_cache(B, Hkv, T, seed=5)
    Q = np.random.default_rng(5).standard_normal((B, H, 128)).astype(np.float16)
    lengths = np.random.default_rng(6).integers(0, T + 1, B).astype(np.int32)
    a = run_attention(Q, kk, vv, lengths, split=False)
    b = run_attention(Q, kk, vv, lengths, split=True)
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


def test_kv4_attention_split_agrees_with_single_pass():
    """Split and single-pass results differ only by FP32 summation order, so
    by at most the attention tolerance: one FP16 ulp plus 2^-12 of the
    largest |v| (outputs near cancellation lose relative accuracy)."""
    B, H, Hkv, T = 1, 32, 8, 8192
    kk, vv = make_cache(B, Hkv, T, seed=9)
    Q = np.random.default_rng(9).standard_normal((B, H, 128)).astype(np.float16)
    a = run_attention(Q, kk, vv, [T], split=False).astype(np.float64)
    b = run_attention(Q, kk, vv, [T], split=True).astype(np.float64)
    vmax = float(np.abs(O.kv4_dequant(*vv)).max())
    assert np.all(np.abs(a - b) <= ulp16(a) + 2.0 ** -12 * vmax)
