"""Fused SiLU(gate) * up + per-token quantization on the GPU, through the C ABI.

"QServe: W4A8KV4 Quantization and System Co-design for Efficient LLM Serving"
(paperlayer.ai summary), §5 runtime and precision mapping: the per-token
quantizer also runs inside the activation-function kernel that produces a
layer's input -- here the down projection's input SiLU(gate) * up.  Against
oracle.swiglu_quant_per_token: x8, s_x and the FP16 activations h bit for
bit, including the SiLU of every finite FP16 value.
"""

import numpy as np
import pytest

import oracle as O
import w4a8_quantized_gemm_qoq_amd as q

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def bits(a):
    return np.asarray(a, np.float16).view(np.uint16)


def check(G, U, x8, sx, h):
    ox8, osx, oh = O.swiglu_quant_per_token(G, U)
    assert np.array_equal(bits(h), bits(oh))
    assert np.array_equal(sx.view(np.uint16), osx.view(np.uint16))
    assert np.array_equal(x8, ox8)


def run(G, U):
    x8, sx, h = q.qoq_swiglu_quant_per_token(dev(G), dev(U), want_h=True)
    torch.cuda.synchronize()
    return x8.cpu().numpy(), sx.cpu().numpy(), h.cpu().numpy()


def test_silu_of_every_finite_half():
    # all 63488 finite FP16 gate values with up = 1: h is the FP16 SiLU itself
    g = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    g = g[np.isfinite(g)]
    G = g.reshape(62, 1024)
    U = np.ones_like(G)
    x8, sx, h = run(G, U)
    assert np.array_equal(bits(h), bits(O.silu_fp16(G)))
    check(G, U, x8, sx, h)


def test_hand_worked_rows():
    from golden_io import read_fixture
    fx = read_fixture("swiglu_rows.txt")
    for K in (6, 16):   # scalar path, and the vector path (zero gates pad the rows)
        G = np.zeros((2, K), np.float16)
        U = np.zeros((2, K), np.float16)
        for r in range(2):
            G[r, :6] = fx[f"g{r}"]
            U[r, :6] = fx[f"u{r}"]
        x8, sx, h = run(G, U)
        for r in range(2):
            assert h[r, :6].astype(np.float64).tolist() == fx[f"h{r}"]
            assert float(sx[r]) == fx[f"s{r}"][0]
            assert x8[r, :6].tolist() == [int(v) for v in fx[f"q{r}"]]
            assert not x8[r, 6:].any()


@pytest.mark.parametrize("M,K", [(4, 128), (3, 4096), (5, 14336), (2, 32000), (2, 32008), (3, 1000), (1, 8)])
def test_random_rows(M, K):
    # the LDS-row path (up to 32000 channels, the longest row), the streaming
    # path (K = 32008) and the scalar path (K not a multiple of 8)
    rng = np.random.default_rng(M * K)
    G = (rng.standard_normal((M, K)) * 2).astype(np.float16)
    U = rng.standard_normal((M, K)).astype(np.float16)
    G[0, :7] = [0, -0.0, 16, -16, 11.5, -20.5, 6e-8]   # zeros, saturating SiLU, a subnormal gate
    check(G, U, *run(G, U))


def test_fused_gate_up_layout_and_strided_output():
    # gate and up as the two halves of one [M, 2K] tensor (leading dimension
    # 2K), h written into a wider buffer
    M, K = 6, 2048
    rng = np.random.default_rng(1)
    GU = rng.standard_normal((M, 2 * K)).astype(np.float16)
    gu = dev(GU)
    hbuf = torch.zeros((M, K + 64), dtype=torch.float16, device="cuda")
    x8, sx, h = q.qoq_swiglu_quant_per_token(gu[:, :K], gu[:, K:], h=hbuf[:, :K])
    torch.cuda.synchronize()
    check(GU[:, :K], GU[:, K:], x8.cpu().numpy(), sx.cpu().numpy(), hbuf[:, :K].cpu().numpy())
    assert not hbuf[:, K:].cpu().numpy().any()


def test_down_projection_input_at_full_size():
    # the c2 down projection's input: 1024 tokens x 14336 (Llama-3-8B FFN)
    M, K = 1024, 14336
    rng = np.random.default_rng(7)
    G = (rng.standard_normal((M, K)) * 1.5).astype(np.float16)
    U = rng.standard_normal((M, K)).astype(np.float16)
    print(f"[swiglu] M={M} K={K}", flush=True)
    x8, sx = q.qoq_swiglu_quant_per_token(dev(G), dev(U))
    torch.cuda.synchronize()
    ox8, osx, _ = O.swiglu_quant_per_token(G, U)
    assert np.array_equal(sx.cpu().numpy().view(np.uint16), osx.view(np.uint16))
    assert np.array_equal(x8.cpu().numpy(), ox8)


def test_rejections():
    g = torch.zeros((2, 16), dtype=torch.float16, device="cuda")
    with pytest.raises(ValueError):
        q.qoq_swiglu_quant_per_token(g, torch.zeros((2, 8), dtype=torch.float16, device="cuda"))
    with pytest.raises(ValueError):
        q.qoq_swiglu_quant_per_token(g.float(), g.float())
