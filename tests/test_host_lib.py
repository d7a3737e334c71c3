"""Host-side checks of libqoq.so that need no GPU: the library loads with
torch's HIP runtime, exports every entry point of include/qoq.h, and its
offline packer produces exactly the oracle's codes in the documented layout.
"""

import os
import re

import numpy as np
import pytest

import oracle as O
import synthetic
import w4a8_quantized_gemm_qoq_amd as q
from w4a8_quantized_gemm_qoq_amd import _native
from golden_io import read_fixture

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_symbols():
    txt = open(os.path.join(ROOT, "include", "qoq.h")).read()
    return sorted(set(re.findall(r"QOQ_API\s+[\w\s\*]*?\b(qoq_\w+)\s*\(", txt)))


def test_library_exports_every_header_symbol():
    lib = q.load_library()
    syms = header_symbols()
    assert len(syms) == 28, syms
    assert sorted(_native.EXPORTS) == syms
    for s in syms:
        assert hasattr(lib, s), s


def test_library_shares_torchs_hip_runtime():
    import torch  # noqa: F401
    q.load_library()
    maps = open("/proc/self/maps").read()
    hip = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    assert len(hip) == 1, hip  # one HIP runtime in the process: torch's
    assert "torch" in next(iter(hip))


def test_status_strings():
    lib = q.load_library()
    for s in range(6):
        assert lib.qoq_status_string(s)
    assert lib.qoq_status_string(99) == b"unknown status"


def test_layout_query_sizes():
    L = q.qoq_weight_layout_query(28672, 8192, 128)
    assert L["layout_id"] == 1 and L["N_pad"] == 28672 and L["n_groups"] == 64
    assert L["qweight_bytes"] == 28672 * 8192 // 2
    assert L["meta_bytes"] == 28672 * 64          # one byte per (channel, group)
    assert L["scale_bytes"] == 2 * 28672
    L = q.qoq_weight_layout_query(100, 256, 128)   # N padded to 112, G = 2 padded to 4
    assert L["N_pad"] == 112 and L["qweight_bytes"] == 112 * 128 and L["meta_bytes"] == 7 * 4 * 16
    L = q.qoq_weight_layout_query(24576, 8192, 0)
    assert L["meta_bytes"] == 24576 and L["group_size"] == 0


@pytest.mark.parametrize("N,K,G,args", [
    (16, 100, 128, "K not multiple of 128"),
    (16, 0, 128, "K zero"),
    (0, 128, 128, "N zero"),
    (16, 128, 64, "group size"),
    (16, 133248, 128, "K over the INT32 bound"),
])
def test_layout_query_rejects(N, K, G, args):
    with pytest.raises(q.QoQError):
        q.qoq_weight_layout_query(N, K, G)


def _documented_position(n, k):
    """Byte offset and nibble of code (n, k) per the layout text in qoq.h."""
    strip, c = divmod(n, 16)
    g, kl = divmod(k, 128)
    half, r = divmod(kl, 64)
    j, t = divmod(r, 16)
    # low nibble of byte b of dword p: k = 64*(p//2) + 16j + 8*(p%2) + b; high = that + 4
    sub, b = divmod(t, 4)          # t = 8*(p%2) + 4*high + b
    p2, high = divmod(sub, 2)
    p = 2 * half + p2
    slot = c + 16 * j
    return ((strip * (K_G[0]) + g) * 64 + slot) * 16 + 4 * p + b, high


K_G = [0]


def test_packed_layout_matches_documentation():
    N, K = 40, 384
    K_G[0] = K // 128
    rng = np.random.default_rng(0)
    for _ in range(200):
        n, k = int(rng.integers(N)), int(rng.integers(K))
        q4 = np.zeros((N, K), np.uint8)
        q4[n, k] = 9
        p = q.qoq_pack_codes(q4, np.ones((N, K // 128), np.uint8), np.zeros((N, K // 128), np.uint8),
                             np.ones(N, np.float16), 128)
        nz = np.flatnonzero(p.qweight)
        assert nz.size == 1
        off, high = _documented_position(n, k)
        assert nz[0] == off
        assert p.qweight[off] == (0x90 if high else 0x09)


def test_meta_layout_matches_documentation():
    N, K = 48, 768  # G = 6, G4 = 8
    G, G4 = 6, 8
    q4 = np.zeros((N, K), np.uint8)
    s1 = np.ones((N, G), np.uint8)
    z = np.zeros((N, G), np.uint8)
    s1[37, 5] = 11
    z[37, 5] = 3
    p = q.qoq_pack_codes(q4, s1, z, np.ones(N, np.float16), 128)
    strip, c = divmod(37, 16)
    off = ((strip * (G4 // 4) + 5 // 4) * 16 + c) * 4 + 5 % 4
    assert np.flatnonzero(p.meta).tolist() == [off]
    assert p.meta[off] == (11 - 1) | (3 << 4)


def _oracle_codes(W, group_size):
    if group_size:
        e = O.encode_weight_g128(W)
        return e["q4"], e["s1"], e["z"], e["s0"]
    e = O.encode_weight_per_channel(W)
    return e["q4"], None, e["z"], e["s_w"]


def _check_pack_matches_oracle(W, group_size):
    p = q.qoq_pack_weights(W, group_size)
    q4, s1, z, sc = q.qoq_unpack_weights(p)
    oq4, os1, oz, osc = _oracle_codes(W, group_size)
    assert np.array_equal(q4, oq4)
    if group_size:
        assert np.array_equal(s1, os1)
    assert np.array_equal(z, oz)
    assert np.array_equal(sc.view(np.uint16), osc.view(np.uint16))
    # padding channels are zero codes with zero scale
    L = q.qoq_weight_layout_query(W.shape[0], W.shape[1], group_size)
    assert np.all(np.asarray(p.scale)[W.shape[0]:L["N_pad"]] == 0)
    return p


@pytest.mark.parametrize("group_size", [128, 0])
@pytest.mark.parametrize("name", ["tiny"])
def test_pack_weights_matches_oracle_tiny(name, group_size):
    _, W = synthetic.make_inputs(name)
    _check_pack_matches_oracle(W, group_size)


@pytest.mark.parametrize("group_size", [128, 0])
def test_pack_weights_matches_oracle_ragged(group_size):
    W = synthetic.make_w(77, 1152, seed=4)   # N not a multiple of 16, G = 9
    _check_pack_matches_oracle(W, group_size)


@pytest.mark.parametrize("group_size", [128, 0])
def test_pack_weights_matches_oracle_attention_shape(group_size):
    W = synthetic.make_w(4096, 4096, seed=0)
    _check_pack_matches_oracle(W, group_size)


@pytest.mark.parametrize("group_size", [128, 0])
def test_pack_weights_edge_rows(group_size):
    K = 256
    rows = [
        np.zeros(K),                                   # zero row
        np.full(K, 3.0),                               # constant row
        np.r_[np.full(K - 1, 1e-7), 6e-8],             # FP16 subnormals
        np.r_[65504.0, -65504.0, np.zeros(K - 2)],     # FP16 extremes
        np.r_[np.full(K // 2, 0.25), np.full(K // 2, -7.0)],  # groups of one sign each
        np.linspace(-1, 1, K),
        np.r_[1.0, np.zeros(K - 1)],                   # single spike
        np.r_[-0.0, np.full(K - 1, -2.5)],
    ]
    W = np.array(rows, dtype=np.float16)
    _check_pack_matches_oracle(W, group_size)


def test_pack_weights_rejects_nonfinite():
    W = synthetic.make_w(16, 128)
    W[3, 7] = np.float16(np.inf)
    with pytest.raises(q.QoQError):
        q.qoq_pack_weights(W, 128)
    W[3, 7] = np.float16(np.nan)
    with pytest.raises(q.QoQError):
        q.qoq_pack_weights(W, 0)


def test_pack_codes_roundtrip_and_validation():
    rng = np.random.default_rng(1)
    N, K = 35, 512
    G = K // 128
    s1 = rng.integers(1, 17, size=(N, G)).astype(np.uint8)
    z = np.minimum(rng.integers(0, 16, size=(N, G)), 128 // s1).astype(np.uint8)
    z = np.minimum(z, 15).astype(np.uint8)
    # choose codes inside the INT8 bound for each group
    q4 = np.zeros((N, K), np.uint8)
    for n in range(N):
        for g in range(G):
            hi = min(15, int(z[n, g]) + 127 // int(s1[n, g]))
            q4[n, g * 128:(g + 1) * 128] = rng.integers(0, hi + 1, size=128)
    sc = rng.standard_normal(N).astype(np.float16)
    p = q.qoq_pack_codes(q4, s1, z, sc, 128)
    uq4, us1, uz, usc = q.qoq_unpack_weights(p)
    assert np.array_equal(uq4, q4) and np.array_equal(us1, s1) and np.array_equal(uz, z)
    assert np.array_equal(usc.view(np.uint16), sc.view(np.uint16))
    bad = s1.copy(); bad[0, 0] = 0
    with pytest.raises(q.QoQError):
        q.qoq_pack_codes(q4, bad, z, sc, 128)
    bad = s1.copy(); bad[0, 0] = 17
    with pytest.raises(q.QoQError):
        q.qoq_pack_codes(q4, bad, z, sc, 128)
    # w8 = (15 - 0) * 16 = 240 breaks the INT8 bound
    q4b = q4.copy(); q4b[0, 0] = 15
    s1b = s1.copy(); s1b[0, 0] = 16
    zb = z.copy(); zb[0, 0] = 0
    with pytest.raises(q.QoQError):
        q.qoq_pack_codes(q4b, s1b, zb, sc, 128)
    # z * s1 = 9 * 16 = 144 > 128
    zb[0, 0] = 9; q4b[0, 0] = 9
    with pytest.raises(q.QoQError):
        q.qoq_pack_codes(q4b, s1b, zb, sc, 128)
    # per-channel roundtrip
    zc = rng.integers(0, 16, size=N).astype(np.uint8)
    p = q.qoq_pack_codes(q4, None, zc, sc, 0)
    uq4, us1, uz, usc = q.qoq_unpack_weights(p)
    assert us1 is None and np.array_equal(uq4, q4) and np.array_equal(uz, zc)


def test_pack_codes_accepts_extreme_valid_bytes():
    # w8 = -128 (z*s1 = 128, q4 = 0) and w8 = 127 are the byte extremes the
    # packed dequantization must still represent
    N, K = 16, 128
    q4 = np.zeros((N, K), np.uint8)
    s1 = np.full((N, 1), 16, np.uint8)
    z = np.full((N, 1), 8, np.uint8)
    q4[:, 1] = 15  # (15 - 8) * 16 = 112
    q.qoq_pack_codes(q4, s1, z, np.ones(N, np.float16), 128)
    s1[:] = 1; z[:] = 0; q4[:] = 15
    q.qoq_pack_codes(q4, s1, z, np.ones(N, np.float16), 128)


def test_device_entry_points_validate_before_launch():
    # argument errors are reported synchronously, without touching a GPU
    lib = q.load_library()
    assert lib.qoq_quant_act_per_token(None, 4, 128, 128, None, None, None) == 1
    assert lib.qoq_w4a8_gemm(None, None, None, None, None, None, 4, 16, 128, 16, 128, None, 0, None) == 1
    # K not a multiple of 128 (non-null dummy pointers are never dereferenced)
    d = 4096
    assert lib.qoq_w4a8_gemm_i32(d, d, d, d, 4, 16, 100, 16, 128, None, 0, None) == 2
    # ldacc < N
    assert lib.qoq_w4a8_gemm_i32(d, d, d, d, 4, 16, 128, 8, 128, None, 0, None) == 1
    # misaligned qweight
    assert lib.qoq_w4a8_gemm_i32(d, d + 4, d, d, 4, 16, 128, 16, 128, None, 0, None) == 3
    assert lib.qoq_w4a8_gemm_workspace_size(4, 16, 128, 128) == 0


@pytest.mark.parametrize("M", [0, -1])
def test_device_entry_points_reject_row_counts_below_one(M):
    # M >= 1 is part of every device call's contract; an empty or negative
    # batch is an unsupported shape (status 2), reported before any launch
    lib = q.load_library()
    d = 4096
    assert lib.qoq_quant_act_per_token(d, M, 128, 128, d, d, None) == 2
    assert lib.qoq_w4a8_gemm(d, d, d, d, d, d, M, 16, 128, 16, 128, None, 0, None) == 2
    assert lib.qoq_w4a8_gemm_i32(d, d, d, d, M, 16, 128, 16, 128, None, 0, None) == 2
    assert lib.qoq_w4a8_gemm_noalloc(d, d, d, d, d, d, M, 16, 128, 16, 128, None) == 2
    assert lib.qoq_rmsnorm_quant_per_token(d, d, 1e-5, M, 128, 128, d, d, None) == 2
    assert lib.qoq_w8a8_gemm(d, d, d, d, d, M, 16, 128, 16, None, 0, None) == 2
    assert lib.qoq_w8a8_gemm_i32(d, d, d, M, 16, 128, 16, None, 0, None) == 2
    assert lib.qoq_w4a8_gemm_saturating(d, d, d, d, d, d, M, 16, 128, 16, None, 0, None) == 2
    assert lib.qoq_w4a8_gemm_saturating_i32(d, d, d, d, M, 16, 128, 16, None, 0, None) == 2
    with pytest.raises(q.QoQError):
        q.qoq_w4a8_gemm_plan(M, 16, 128)


# ------------------------------------------------------------ comparators (f1)

def _documented_w8_blocks(w8, N, K):
    """Scatter INT8 codes by the layout comment of qoq_pack_weights_w8."""
    N_pad = (N + 15) // 16 * 16
    G = K // 128
    out = np.zeros(N_pad * K, np.uint8)
    for n in range(N):
        strip, c = divmod(n, 16)
        for g in range(G):
            for h in range(2):
                for j in range(4):
                    slot = c + 16 * j + 64 * h
                    k0 = 128 * g + 64 * h + 16 * j
                    off = ((strip * G + g) * 128 + slot) * 16
                    out[off:off + 16] = w8[n, k0:k0 + 16].astype(np.int8).view(np.uint8)
    return out


@pytest.mark.parametrize("N,K,seed", [(16, 256, 0), (77, 1152, 4), (40, 384, 9)])
def test_pack_weights_w8_matches_oracle_and_layout(N, K, seed):
    W = synthetic.make_w(N, K, seed=seed)
    p = q.qoq_pack_weights_w8(W)
    w8, s = O.quant_weight_w8(W)
    assert np.array_equal(np.asarray(p.scale)[:N].view(np.float16), s)
    assert not np.asarray(p.scale)[N:].any()
    assert np.array_equal(p.qweight, _documented_w8_blocks(w8, N, K))


def test_pack_weights_w8_edge_rows_and_rejects():
    K = 256
    rows = [np.zeros(K), np.full(K, 3.0), np.r_[65504.0, -65504.0, np.zeros(K - 2)],
            np.r_[np.full(K - 1, 1e-7), 6e-8], np.linspace(-1, 1, K)]
    W = np.array(rows, dtype=np.float16)
    p = q.qoq_pack_weights_w8(W)
    w8, s = O.quant_weight_w8(W)
    assert np.array_equal(np.asarray(p.scale)[:len(rows)].view(np.float16), s)
    assert np.array_equal(p.qweight, _documented_w8_blocks(w8, len(rows), K))
    W[2, 3] = np.float16(np.nan)
    with pytest.raises(q.QoQError):
        q.qoq_pack_weights_w8(W)
    with pytest.raises(q.QoQError):
        q.qoq_pack_weights_w8(np.zeros((4, 100), np.float16))


def test_comparator_entry_points_validate_before_launch():
    lib = q.load_library()
    d = 4096
    # null pointers
    assert lib.qoq_w8a8_gemm(None, None, None, None, None, 4, 16, 128, 16, None, 0, None) == 1
    assert lib.qoq_w4a8_gemm_saturating(None, None, None, None, None, None, 4, 16, 128, 16, None, 0, None) == 1
    # K not a multiple of 128, ldacc < N, misaligned weights
    assert lib.qoq_w8a8_gemm_i32(d, d, d, 4, 16, 100, 16, None, 0, None) == 2
    assert lib.qoq_w8a8_gemm_i32(d, d, d, 4, 16, 128, 8, None, 0, None) == 1
    assert lib.qoq_w8a8_gemm_i32(d, d + 4, d, 4, 16, 128, 16, None, 0, None) == 3
    assert lib.qoq_w4a8_gemm_saturating_i32(d, d, d, d, 4, 16, 100, 16, None, 0, None) == 2
    assert lib.qoq_w8a8_gemm_workspace_size(4, 16, 128) == 0
    assert lib.qoq_w8a8_gemm_workspace_size(300, 96, 2048) == lib.qoq_w4a8_gemm_workspace_size(300, 96, 2048, 128)


def test_rmsnorm_quant_validates_before_launch():
    lib = q.load_library()
    d = 4096
    assert lib.qoq_rmsnorm_quant_per_token(None, d, 1e-5, 4, 128, 128, d, d, None) == 1
    assert lib.qoq_rmsnorm_quant_per_token(d, d, 0.0, 4, 128, 128, d, d, None) == 1       # eps must be > 0
    assert lib.qoq_rmsnorm_quant_per_token(d, d, float("inf"), 4, 128, 128, d, d, None) == 1
    assert lib.qoq_rmsnorm_quant_per_token(d, d, 1e-5, 4, 128, 64, d, d, None) == 1       # ldx < K
    assert lib.qoq_rmsnorm_quant_per_token(d, d, 1e-5, 0, 128, 128, d, d, None) == 2
    assert lib.qoq_rmsnorm_quant_per_token(d + 1, d, 1e-5, 4, 128, 128, d, d, None) == 3  # odd FP16 pointer


def test_kv4_entry_points_validate_before_launch():
    lib = q.load_library()
    d = 4096
    assert lib.qoq_kv4_quant(None, 4, 128, 128, d, d, d, None) == 1
    assert lib.qoq_kv4_quant(d, 4, 64, 64, d, d, d, None) == 2            # head_dim must be 128
    assert lib.qoq_kv4_quant(d, 4, 128, 130, d, d, d, None) == 1          # ldx not a multiple of 8
    assert lib.qoq_kv4_quant(d + 4, 4, 128, 128, d, d, d, None) == 3      # x needs 16-byte alignment
    args = [d] * 8
    assert lib.qoq_kv4_decode_attention(*args, 2, 4, 3, 16, 128, 0.1, d, None) == 2      # H % Hkv
    assert lib.qoq_kv4_decode_attention(*args, 2, 4, 2, 40000, 128, 0.1, d, None) == 2   # T_max too large
    assert lib.qoq_kv4_decode_attention(*args, 2, 4, 2, 16, 64, 0.1, d, None) == 2       # head_dim
    assert lib.qoq_kv4_decode_attention(*args, 2, 4, 2, 16, 128, float("nan"), d, None) == 1
    assert lib.qoq_kv4_decode_attention(d + 8, *args[1:], 2, 4, 2, 16, 128, 0.1, d, None) == 3
    assert lib.qoq_kv4_decode_attention(None, *args[1:], 2, 4, 2, 16, 128, 0.1, d, None) == 1
    # empty or negative sizes: unsupported shapes, and no workspace
    assert lib.qoq_kv4_quant(d, 0, 128, 128, d, d, d, None) == 2
    for B, H, Hkv, T in [(0, 4, 2, 16), (-1, 4, 2, 16), (2, 0, 2, 16), (2, 4, 0, 16), (2, 4, 2, 0)]:
        assert lib.qoq_kv4_decode_attention(*args, B, H, Hkv, T, 128, 0.1, d, None) == 2
        assert lib.qoq_kv4_decode_attention_workspace_size(B, H, Hkv, T) == 0
    # the token-split entry: same checks, plus its workspace
    assert lib.qoq_kv4_decode_attention_split(*args, 2, 4, 3, 16, 128, 0.1, d, d, 1 << 20, None) == 2
    need = lib.qoq_kv4_decode_attention_workspace_size(1, 32, 8, 4096)
    assert need > 0
    assert lib.qoq_kv4_decode_attention_split(*args, 1, 32, 8, 4096, 128, 0.1, d, d, need - 1, None) == 1
    assert lib.qoq_kv4_decode_attention_split(*args, 1, 32, 8, 4096, 128, 0.1, d, None, need, None) == 1
    assert lib.qoq_kv4_decode_attention_split(*args, 1, 32, 8, 4096, 128, 0.1, d, d + 4, need, None) == 3


def test_kv4_attention_split_plan():
    """Workspace of the token-split attention: nc chunks x B x H x (128 outputs
    + max + sum) FP32.  Nothing is split once (sequence, head group)
    workgroups alone reach 256, or below 512 cached tokens; otherwise chunks
    are 1024 tokens, halved (down to 256) while fewer than 512 workgroups
    would result.  A GQA group is taken 4 or 2 heads a workgroup: of the plans
    that reach 512 workgroups the one with the longest chunks, else the one
    with the most workgroups."""
    ws = q.load_library().qoq_kv4_decode_attention_workspace_size

    def chunks(B, H, Hkv, T):
        n = ws(B, H, Hkv, T)
        assert n % (B * H * 130 * 4) == 0
        return n // (B * H * 130 * 4)

    # 1 x 32 heads over 8 kv heads: 16 two-head workgroups; 256-token chunks
    # still give only 256 workgroups (128 with four heads)
    assert chunks(1, 32, 8, 32768 // 8) == 16
    # 512 workgroups either way: four heads with 512-token chunks, two heads
    # with 1024-token chunks (longer, chosen)
    assert chunks(1, 32, 8, 32768) == 32
    # MHA, 2 x 32 one-head workgroups: 1024 -> 192, 512 -> 384, 256 -> 768
    assert chunks(2, 32, 32, 3000) == 12
    assert chunks(4, 32, 32, 4096) == 4        # 128 workgroups x 4 chunks of 1024
    assert chunks(1, 4, 1, 32768) == 128       # one four-head workgroup: 256-token chunks
    assert chunks(1, 4, 1, 511) == 0           # too short to split
    assert chunks(1, 4, 1, 512) == 2
    assert chunks(64, 32, 8, 1024) == 0        # 512 workgroups already
    assert chunks(32, 32, 8, 1024) == 0        # 256: one per CU
    assert chunks(8, 32, 1, 4096) == 4         # 8 x 16 two-head workgroups x 4 chunks of 1024
    assert chunks(4, 64, 8, 8192) == 8         # 64 four-head workgroups x 8 chunks of 1024
    assert chunks(1, 6, 2, 2000) == 8          # 3 heads per kv head: one a workgroup
    assert ws(2, 4, 3, 4096) == 0              # invalid shapes: 0
    assert ws(1, 4, 1, 40000) == 0


# ------------------------------------------------- offline transforms (f4)

def _within_1ulp16(a, b):
    a = np.asarray(a, np.float16).astype(np.float64)
    b = np.asarray(b, np.float16).astype(np.float64)
    e = np.floor(np.log2(np.maximum(np.abs(b), 2.0 ** -14)))
    return np.all(np.abs(a - b) <= 2.0 ** (e - 10))


@pytest.mark.parametrize("rows,K,seed", [(8, 4096, 0), (4, 14336, 1), (16, 384, 2), (3, 8, 3), (5, 7, 4)])
def test_hadamard_rotate_matches_oracle(rows, K, seed):
    X = synthetic.make_x(rows, K, "frac", seed=seed)
    got = q.qoq_hadamard_rotate(X)
    ref = O.rotate_rows(X)
    assert _within_1ulp16(got, ref)
    assert int(np.count_nonzero(got.view(np.uint16) != ref.view(np.uint16))) <= max(1, got.size // 100000)


def test_hadamard_rotate_is_an_involution_up_to_rounding():
    # H is symmetric and orthogonal (H H = I for the Sylvester blocks)
    X = synthetic.make_w(4, 2048, seed=5)
    back = q.qoq_hadamard_rotate(q.qoq_hadamard_rotate(X)).astype(np.float64)
    X64 = X.astype(np.float64)
    # the FP16 rounding of the rotated row (2^-11 relative) spreads over the
    # whole row when rotated back: bound it by the row's RMS
    rms = np.sqrt((X64 ** 2).mean(axis=1, keepdims=True))
    assert np.all(np.abs(back - X64) <= 2.0 ** -8 * rms)


def test_scale_columns_bit_exact_and_smoothing_factors():
    X = synthetic.make_x(6, 512, "frac", seed=6)
    W = synthetic.make_w(10, 512, seed=6)
    a = np.abs(X.astype(np.float32)).max(0)
    w = np.abs(W.astype(np.float32)).max(0)
    lam = q.qoq_smoothing_factors(a, w, 0.5)
    ref = O.smoothing_factors(a, w, 0.5)
    assert np.all(np.abs(lam.astype(np.float64) - ref) <= np.spacing(np.abs(ref)).astype(np.float64))
    assert np.array_equal(q.qoq_scale_columns(W, ref).view(np.uint16), O.scale_columns(W, ref).view(np.uint16))
    assert np.array_equal(q.qoq_scale_columns(X, ref, divide=True).view(np.uint16),
                          O.scale_columns(X, ref, divide=True).view(np.uint16))
    # FP16 edge values: subnormal results, overflow to inf, exact halving
    E = np.array([[6e-8, 65504.0, -1.0, 3.0]], np.float16)
    f = np.array([0.5, 2.0, 1.0, 1.0 / 3.0], np.float32)
    with np.errstate(over="ignore"):   # 65504 * 2 overflows FP16 to inf on purpose
        ref_e = O.scale_columns(E, f)
    assert np.array_equal(q.qoq_scale_columns(E, f).view(np.uint16), ref_e.view(np.uint16))


def test_library_refuses_a_build_of_other_sources(monkeypatch):
    # load_library() compares the source hash recorded by build() with the
    # sources in the tree and refuses a library built from anything else
    import w4a8_quantized_gemm_qoq_amd.build as b
    monkeypatch.setattr(_native, "_lib", None)
    monkeypatch.setattr(b, "source_hash", lambda arch="gfx950": "0" * 64)
    with pytest.raises(RuntimeError, match="not built from the sources"):
        _native.load_library()


def test_scale_columns_hand_worked_cases():
    # the library against the hand-worked fixture directly (not only against
    # the oracle)
    fx = read_fixture("scale_columns.txt")
    for x, f, d, y in zip(fx["x"], fx["f"], fx["divide"], fx["y"]):
        got = q.qoq_scale_columns(np.array([[x]], np.float16), np.array([f], np.float32), divide=bool(d))
        assert got[0, 0].view(np.uint16) == np.float16(y).view(np.uint16), (x, f, d, y, got[0, 0])
    X = np.array(fx["mat_x"], np.float16).reshape(2, 2)
    got = q.qoq_scale_columns(X, np.array(fx["mat_f"], np.float32))
    assert np.array_equal(got, np.array(fx["mat_y"], np.float16).reshape(2, 2))


def test_transforms_validate_arguments():
    lib = q.load_library()
    d = 4096
    assert lib.qoq_hadamard_rotate(None, 1, 8, 8, d) == 1
    assert lib.qoq_hadamard_rotate(d, 1, 8, 4, d) == 1
    assert lib.qoq_smoothing_factors(d, d, 4, 1.5, d) == 1
    with pytest.raises(q.QoQError):
        q.qoq_scale_columns(np.ones((2, 4), np.float16), np.array([1, 0, 1, 1], np.float32))
