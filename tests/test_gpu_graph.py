"""The device entry points inside a captured HIP graph: every replay must
reproduce the eager result bit for bit, with eager work and synchronizations
between the replays.  No entry point records a memset, and the GEMM's split-K
workspace is an ordinary allocation of the capturing pool."""

import numpy as np
import pytest

import synthetic
import w4a8_quantized_gemm_qoq_amd as q

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.mark.parametrize("M,K,N", [(256, 4096, 4096),   # skinny, K split in LDS
                                   (300, 2048, 96),     # large kernel, K split over blocks + reduction
                                   (520, 512, 24576),   # big 128x512 tiles
                                   (1024, 8320, 4096),  # K-set 128x128 tile, odd group count
                                   (16, 2048, 20000),   # strip kernel (16-row groups)
                                   (40, 1024, 20000),   # ring kernel, one wave a strip
                                   (20, 8192, 24000)])  # ring kernel, two waves a strip
def test_quant_gemm_graph_replays(M, K, N):
    X = synthetic.make_x(M, K, "frac", seed=M)
    W = synthetic.make_w(N, K, seed=N)
    p = q.qoq_pack_weights(W, 128).to("cuda")
    p8 = q.qoq_pack_weights_w8(W).to("cuda")
    x = torch.from_numpy(X).cuda()
    gamma = torch.from_numpy(synthetic.make_gamma(K)).cuda()
    x8 = torch.empty((M, K), dtype=torch.int8, device="cuda")
    sx = torch.empty((M,), dtype=torch.float16, device="cuda")
    y = torch.empty((M, N), dtype=torch.float16, device="cuda")
    y8 = torch.empty((M, N), dtype=torch.float16, device="cuda")

    def step():
        q.qoq_rmsnorm_quant_per_token(x, gamma, 1e-5, x8, sx)
        q.qoq_quant_act_per_token(x, x8, sx)
        q.qoq_w4a8_gemm(x8, sx, p, y=y)
        q.qoq_w8a8_gemm(x8, sx, p8, y=y8)

    step()
    torch.cuda.synchronize()
    ref, ref8 = y.clone(), y8.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(4):
        y.fill_(float("nan"))
        y8.fill_(float("nan"))
        x8.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), f"replay {i}"
        assert torch.equal(y8.view(torch.int16), ref8.view(torch.int16)), f"replay {i}"
        step()                       # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("split", [False, True])
def test_kv4_graph_replays(split):
    B, H, Hkv, T = 4, 8, 2, 600
    rng = np.random.default_rng(0)
    kv = torch.from_numpy(rng.standard_normal((2, B, Hkv, T, 128)).astype(np.float16)).cuda()
    qq = torch.from_numpy(rng.standard_normal((B, H, 128)).astype(np.float16)).cuda()
    lengths = torch.tensor([600, 1, 0, 357], dtype=torch.int32, device="cuda")
    o = torch.empty((B, H, 128), dtype=torch.float16, device="cuda")
    need = q.qoq_kv4_decode_attention_workspace_size(B, H, Hkv, T)
    assert need > 0                  # this shape is split when asked
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    caches = [q.qoq_kv4_quant(kv[0]), q.qoq_kv4_quant(kv[1])]

    def step():
        for i, c in enumerate(caches):
            q.qoq_kv4_quant(kv[i], *c)
        q.qoq_kv4_decode_attention(qq, caches[0], caches[1], lengths, 0.0883883476, o=o, split=split, workspace=ws)

    step()
    torch.cuda.synchronize()
    ref = o.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(4):
        o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), ref.view(torch.int16)), f"replay {i}"
        step()
        torch.cuda.synchronize()
