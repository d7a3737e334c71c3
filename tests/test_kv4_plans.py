"""Launch plans of the KV4 decode attention (host query, no GPU): every
parity case reaches the plan pinned for it in kv4_cases.py, and together the
cases reach every kernel the attention has -- 1, 2 and 4 query heads a
workgroup, each with and without token chunks -- and the query edge cases do
too."""

import pytest

import w4a8_quantized_gemm_qoq_amd as q
from kv4_cases import EDGE, PLAIN, SPLIT


@pytest.mark.parametrize("B,H,Hkv,T,lengths,peak,plan", PLAIN)
def test_plain_case_plans(B, H, Hkv, T, lengths, peak, plan):
    assert q.qoq_kv4_decode_attention_plan(B, H, Hkv, T, split=False) == plan


@pytest.mark.parametrize("B,H,Hkv,T,lengths,peak,plan", SPLIT)
def test_split_case_plans(B, H, Hkv, T, lengths, peak, plan):
    assert q.qoq_kv4_decode_attention_plan(B, H, Hkv, T, split=True) == plan
    assert plan[1] > 1


def kernel(plan):
    r, nc = plan
    return r, nc > 1


def test_cases_reach_every_kernel():
    want = {(r, s) for r in (1, 2, 4) for s in (False, True)}
    got = {kernel(c[-1]) for c in PLAIN + SPLIT}
    assert got == want, sorted(want - got)
    assert {kernel(c[-1]) for c in EDGE} == want


@pytest.mark.parametrize("B,H,Hkv,T,split,plan", EDGE)
def test_edge_case_plans(B, H, Hkv, T, split, plan):
    assert q.qoq_kv4_decode_attention_plan(B, H, Hkv, T, split=split) == plan


def test_plan_query_rejects_bad_shapes():
    with pytest.raises(q.QoQError):
        q.qoq_kv4_decode_attention_plan(1, 6, 4, 100)     # H not a multiple of Hkv
    with pytest.raises(q.QoQError):
        q.qoq_kv4_decode_attention_plan(1, 8, 2, 40000)   # longer than the cache limit
