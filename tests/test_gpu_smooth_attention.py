"""SmoothAttention on the KV4 path, through the C ABI.

"QServe: W4A8KV4 Quantization and System Co-design for Efficient LLM Serving"
(paperlayer.ai summary), §4 SmoothAttention: outlier key channels are scaled
down and the queries, which stay unquantized, take the factor instead, with
alpha = 0.5; §5 KV4 attention: the smoothed keys are what the per-head INT4
cache holds.  Per kv head h and channel d the factor is
    lambda[h, d] = max_{b,t} |K[b, t, h, d]| ^ 0.5        (weight side w = 1),
keys are divided by it before qoq_kv4_quant and every query head of that kv
head is multiplied by it, so q . k is unchanged before rounding.

The library path (qoq_smoothing_factors, qoq_scale_columns on the host; the
KV4 quantizer and attention on the GPU) is compared with the oracle's own
composition of the same steps: codes, scales and zeros of the smoothed keys
bit for bit, the attention output within the KV4 bar
    |o_gpu - o_ref| <= ulp16(o_ref) + 2^-12 * max_t |v_t|.
The accuracy effect on synthetic outlier keys is printed and checked loosely
(information about the transform, not parity).
"""

import numpy as np
import pytest

import oracle as O
import w4a8_quantized_gemm_qoq_amd as q

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SCALE = float(np.float32(1.0 / np.sqrt(128.0)))
ALPHA = 0.5


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def ulp16(v):
    a = np.abs(np.asarray(v, np.float64))
    return 2.0 ** (np.floor(np.log2(np.maximum(a, 2.0 ** -14))) - 10)


def pack_codes(c):
    c = np.asarray(c, np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def make_qkv(B, T, H, Hkv, seed):
    """Keys [B, T, Hkv, 128] with 4 fixed outlier channels per kv head (x20,
    the same for every token, as key outliers are), values [B, T, Hkv, 128]
    and queries [B, H, 128], all N(0, 1) FP16 otherwise."""
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((B, T, Hkv, 128)).astype(np.float32)
    for h in range(Hkv):
        K[:, :, h, rng.choice(128, 4, replace=False)] *= 20
    V = rng.standard_normal((B, T, Hkv, 128)).astype(np.float16)
    Q = rng.standard_normal((B, H, 128)).astype(np.float16)
    return K.astype(np.float16), V, Q


def smooth_library(K, Q, H):
    B, T, Hkv, D = K.shape
    kabs = np.abs(K.astype(np.float32)).max(axis=(0, 1)).reshape(-1)
    lam = q.qoq_smoothing_factors(kabs, np.ones_like(kabs), ALPHA)
    Ks = q.qoq_scale_columns(K.reshape(B * T, Hkv * D), lam, divide=True).reshape(B, T, Hkv, D)
    lam_q = np.repeat(lam.reshape(Hkv, D), H // Hkv, axis=0).reshape(-1)
    Qs = q.qoq_scale_columns(Q.reshape(B, H * D), lam_q).reshape(B, H, D)
    return lam, Ks, Qs


def smooth_oracle(K, Q, H):
    B, T, Hkv, D = K.shape
    kabs = np.abs(K.astype(np.float64)).max(axis=(0, 1)).reshape(-1)
    lam = O.smoothing_factors(kabs, np.ones_like(kabs), ALPHA)
    Ks = O.scale_columns(K.reshape(B * T, Hkv * D), lam, divide=True).reshape(B, T, Hkv, D)
    lam_q = np.repeat(lam.reshape(Hkv, D), H // Hkv, axis=0).reshape(-1)
    Qs = O.scale_columns(Q.reshape(B, H * D), lam_q).reshape(B, H, D)
    return lam, Ks, Qs


def cache_layout(X):
    """[B, T, Hkv, 128] -> the cache's [B, Hkv, T, 128]."""
    return np.ascontiguousarray(X.transpose(0, 2, 1, 3))


def gpu_attention(Qs, Kc, Vc, lengths, split):
    kq = q.qoq_kv4_quant(dev(Kc))
    vq = q.qoq_kv4_quant(dev(Vc))
    o = q.qoq_kv4_decode_attention(dev(Qs), kq, vq, dev(np.asarray(lengths, np.int32)), SCALE, split=split)
    torch.cuda.synchronize()
    return o.cpu().numpy(), [t.cpu().numpy() for t in kq]


def exact_attention(Q, K, V, lengths, H):
    """FP64 decode attention over the unquantized keys and values (no
    smoothing: the reference the quantized paths approximate)."""
    B, T, Hkv, D = K.shape
    out = np.zeros((B, H, D))
    for b in range(B):
        L = int(lengths[b])
        for h in range(H):
            g = h // (H // Hkv)
            k = K[b, :L, g].astype(np.float64)
            v = V[b, :L, g].astype(np.float64)
            s = SCALE * (k @ Q[b, h].astype(np.float64))
            e = np.exp(s - s.max())
            out[b, h] = (e / e.sum()) @ v
    return out


@pytest.mark.parametrize("B,T,H,Hkv,lengths,split", [
    (4, 512, 32, 8, [512, 300, 1, 511], False),   # Llama-3-8B heads (GQA)
    (2, 300, 4, 4, [300, 77], False),             # MHA
    (1, 4096, 32, 8, [4096], True),               # one long sequence, token-split entry
])
def test_smooth_attention_matches_oracle(B, T, H, Hkv, lengths, split):
    K, V, Q = make_qkv(B, T, H, Hkv, seed=T + H)
    lam, Ks, Qs = smooth_library(K, Q, H)
    lam_o, Ks_o, Qs_o = smooth_oracle(K, Q, H)
    # both sides evaluate lambda in FP64 and round once to FP32
    assert np.array_equal(lam.view(np.uint32), lam_o.view(np.uint32))
    assert np.array_equal(Ks.view(np.uint16), Ks_o.view(np.uint16))
    assert np.array_equal(Qs.view(np.uint16), Qs_o.view(np.uint16))

    Kc, Vc = cache_layout(Ks), cache_layout(V)
    o, (kc, ks, kz) = gpu_attention(Qs, Kc, Vc, lengths, split)
    kk = O.kv4_quant_per_head(cache_layout(Ks_o))
    vv = O.kv4_quant_per_head(Vc)
    assert np.array_equal(kc, pack_codes(kk[0]))
    assert np.array_equal(ks.view(np.uint16), kk[1].view(np.uint16))
    assert np.array_equal(kz, kk[2])

    ref = O.kv4_decode_attention(Qs_o, *kk, *vv, lengths, SCALE).astype(np.float64)
    Vd = np.abs(O.kv4_dequant(*vv))
    vmax = np.zeros((B, H))
    for b in range(B):
        L = int(lengths[b])
        for h in range(H):
            vmax[b, h] = Vd[b, h // (H // Hkv), :L].max() if L else 0.0
    tol = ulp16(ref) + 2.0 ** -12 * vmax[..., None]
    err = np.abs(o.astype(np.float64) - ref)
    print(f"[smooth attn] B={B} T={T} H={H} Hkv={Hkv} split={split} worst err/tol = {float((err / tol).max()):.3f}",
          flush=True)
    assert np.all(err <= tol)


def test_smooth_attention_reduces_kv4_error_on_outlier_keys():
    """Information about the transform on synthetic outlier keys: the INT4
    key error and the attention output error against FP64 attention over the
    unquantized cache, without and with SmoothAttention (both on the GPU)."""
    B, T, H, Hkv = 8, 1024, 32, 8
    lengths = [T] * B
    K, V, Q = make_qkv(B, T, H, Hkv, seed=5)
    exact = exact_attention(Q, K, V, lengths, H)
    Vc = cache_layout(V)

    o_plain, (kc, ks, kz) = gpu_attention(Q, cache_layout(K), Vc, lengths, False)
    lam, Ks, Qs = smooth_library(K, Q, H)
    o_smooth, (kc2, ks2, kz2) = gpu_attention(Qs, cache_layout(Ks), Vc, lengths, False)

    def key_error(codes, s, z, factor):
        c = np.stack([codes & 15, codes >> 4], axis=-1).reshape(codes.shape[:-1] + (128,))
        deq = (c.astype(np.float64) - z[..., None]) * s.astype(np.float64)[..., None]
        deq = deq * factor.reshape(1, Hkv, 1, 128)
        ref = cache_layout(K).astype(np.float64)
        return np.linalg.norm(deq - ref) / np.linalg.norm(ref)

    ek_plain = key_error(kc, ks, kz, np.ones(Hkv * 128))
    ek_smooth = key_error(kc2, ks2, kz2, lam.astype(np.float64))
    ea_plain = np.linalg.norm(o_plain - exact) / np.linalg.norm(exact)
    ea_smooth = np.linalg.norm(o_smooth - exact) / np.linalg.norm(exact)
    print(f"[smooth attn] INT4 key error {ek_plain:.4f} -> {ek_smooth:.4f}; "
          f"attention output error {ea_plain:.4f} -> {ea_smooth:.4f}", flush=True)
    assert ek_smooth < ek_plain
    assert ea_smooth < ea_plain
