"""Launch plans of the W4A8 GEMM (host query, no GPU): every parity shape
reaches the plan pinned for it in gemm_cases.py, and together the shapes
reach every kernel variant -- the strip kernel with one and several strips
per block and with K parts, the ring kernel with one and two waves a strip,
the skinny kernel with 16-, 32- and 64-row tiles and 4 or 8 K parts per
block, and the three large-M tiles with and without a K split."""

import pytest

import w4a8_quantized_gemm_qoq_amd as q
from gemm_cases import SMALL


@pytest.mark.parametrize("M,K,N,gs,plan", SMALL)
def test_parity_shape_plans(M, K, N, gs, plan):
    assert q.qoq_w4a8_gemm_plan(M, N, K, gs) == plan


def test_parity_shapes_reach_every_kernel_variant():
    plans = {c[-1] for c in SMALL}
    kinds = {(k, t if k == "large" else None, s > 1) for k, t, s in plans}
    want = {("strip", None, True), ("strip", None, False), ("skinny16", None, True),
            ("skinny32", None, True), ("skinny64", None, True), ("ring", None, False), ("ring", None, True)}
    want |= {("large", t, False) for t in (0, 1, 2)} | {("large", t, True) for t in (1, 2)}
    assert want <= kinds, sorted(want - kinds)
    # the skinny kernel with several strips per block, with 4 and with 8 K
    # parts per block, and both weight formats on the large tiles
    assert any(k == "skinny64" and t > 1 for k, t, _ in plans)
    assert {s for k, _, s in plans if k.startswith("skinny")} == {4, 8}
    assert any(k == "skinny64" and t > 1 and s == 8 for k, t, s in plans)
    for t in (0, 1, 2):
        assert {c[3] for c in SMALL if c[-1][0] == "large" and c[-1][1] == t} == {0, 128}
    # the ring kernel with 16-, 32- and 64-row tiles, both weight formats, and
    # one, several and a partial last batch of groups
    ring = [c for c in SMALL if c[-1][0] == "ring"]
    tiles = lambda cs: {(m + 15) // 16 if m <= 16 else (2 if m <= 32 else 4) for m, *_ in cs}
    ring1 = [c for c in ring if c[-1][2] == 1]
    ring2 = [c for c in ring if c[-1][2] == 2]
    assert tiles(ring1) == {2, 4} and tiles(ring2) == {1, 2}
    assert {c[3] for c in ring1} == {0, 128} and {c[3] for c in ring2} == {0, 128}
    assert {k // 1024 for _, k, *_ in ring1} >= {1, 2, 3, 5}
    assert {t for *_, (k, t, _) in ring} == {5, 6, 7, 8}


def test_headline_and_decode_plans():
    # the measured workloads: M=4096 on the big tile, the down projection on
    # the K-set tile, decode M = 1 and 16 on the strip kernel, M = 64 on the
    # ring kernel
    assert q.qoq_w4a8_gemm_plan(4096, 24576, 8192) == ("large", 0, 1)
    assert q.qoq_w4a8_gemm_plan(1024, 4096, 14336) == ("large", 2, 1)
    assert q.qoq_w4a8_gemm_plan(1024, 28672, 4096) == ("large", 0, 1)
    assert q.qoq_w4a8_gemm_plan(1, 28672, 8192) == ("strip", 7, 1)
    assert q.qoq_w4a8_gemm_plan(16, 28672, 8192) == ("strip", 7, 1)
    assert q.qoq_w4a8_gemm_plan(64, 28672, 8192) == ("ring", 7, 1)


def test_plan_query_rejects_bad_shapes():
    with pytest.raises(q.QoQError):
        q.qoq_w4a8_gemm_plan(16, 64, 100)   # K not a multiple of 128
    with pytest.raises(q.QoQError):
        q.qoq_w4a8_gemm_plan(0, 64, 128)
