"""Pins for the CPU oracle: hand-worked values, closed forms, invariants,
exhaustive scans and brute force.  None of these re-types the oracle's own
formula; each would fail on a plausible slip (a dropped term, a wrong sign or
index, the wrong rounding mode, a transposed operand).

CPU only.
"""

from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
import synthetic
from golden_io import read_fixture

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# ---------------------------------------------------------------- rounding

def test_fp16_rounding_is_single_step_half_even():
    # 1 + 2^-11 + 2^-40 is just above the tie between FP16 1.0 and 1.0009765625.
    # A detour through FP32 would drop 2^-40, land on the tie and round to 1.0.
    v = np.float64(1.0) + np.float64(2.0) ** -11 + np.float64(2.0) ** -40
    assert float(O.fp16_rne(v)) == 1.0009765625
    # exact ties go to the even significand
    assert float(O.fp16_rne(np.float64(1.0) + 2.0 ** -11)) == 1.0
    assert float(O.fp16_rne(np.float64(1.0) + 3 * 2.0 ** -11)) == 1.001953125


def test_rne_div_matches_exact_fractions():
    from fractions import Fraction
    a = np.arange(-300, 301)
    for s in range(1, 18):
        got = O.rne_div(a, s)
        for ai, gi in zip(a.tolist(), got.tolist()):
            f = Fraction(ai, s)
            fl = f.numerator // f.denominator
            rem = f - fl
            if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
                fl += 1
            assert gi == fl, (ai, s, gi, fl)


# ------------------------------------------------------ activation quantizer

def test_act_quant_hand_worked_rows():
    fx = read_fixture("act_quant_rows.txt")
    X = np.array([fx[f"x{i}"] for i in range(5)], dtype=np.float16)
    x8, s = O.quant_act_per_token(X)
    for i in range(5):
        assert float(s[i]) == fx[f"s{i}"][0], i
        assert x8[i].tolist() == [int(v) for v in fx[f"q{i}"]], i
    assert int(s.view(np.uint16)[2]) == 0x260C


def test_act_quant_invariants_on_workload_rows():
    X = synthetic.make_x(64, 4096, "frac", seed=3)
    x8, s = O.quant_act_per_token(X)
    assert x8.dtype == np.int8 and s.dtype == np.float16
    assert np.abs(x8.astype(np.int32)).max() <= 127
    # each token reaches +-127 at its largest-magnitude entry (normal-range scale)
    am = np.argmax(np.abs(X.astype(np.float32)), axis=1)
    hit = x8[np.arange(64), am].astype(np.int32)
    assert np.all(np.abs(hit) == 127)
    assert np.all(np.sign(hit) == np.sign(X[np.arange(64), am].astype(np.float32)))
    # every code is within half a step of x/s (no clamping away from the max)
    err = np.abs(x8.astype(np.float64) * s.astype(np.float64)[:, None] - X.astype(np.float64))
    assert np.all(err <= 0.5 * s.astype(np.float64)[:, None] * (1 + 2.0 ** -20))


def test_act_quant_is_row_local_and_sign_symmetric():
    X = synthetic.make_x(8, 512, "fixed", seed=1)
    x8, s = O.quant_act_per_token(X)
    x8n, sn = O.quant_act_per_token(-X)
    assert np.array_equal(s, sn) and np.array_equal(x8n.astype(int), -x8.astype(int))
    x8p, sp = O.quant_act_per_token(X[::-1])
    assert np.array_equal(x8p, x8[::-1]) and np.array_equal(sp, s[::-1])


# ------------------------------------------------------ weight level 0

def test_level0_hand_worked_row():
    fx = read_fixture("weight_level0_row.txt")
    W = np.array([fx["w"]], dtype=np.float16)
    q8, s0 = O.quant_weight_level0(W)
    assert float(s0[0]) == fx["s0"][0]
    assert q8[0].tolist() == [int(v) for v in fx["q8"]]


def test_level0_invariants_and_error_bound():
    W = synthetic.make_w(256, 1024, seed=5)
    q8, s0 = O.quant_weight_level0(W)
    assert np.abs(q8.astype(int)).max() <= 119
    am = np.argmax(np.abs(W.astype(np.float32)), axis=1)
    assert np.all(np.abs(q8[np.arange(256), am].astype(int)) == 119)
    err = np.abs(q8.astype(np.float64) * s0.astype(np.float64)[:, None] - W.astype(np.float64))
    assert np.all(err <= 0.5 * s0.astype(np.float64)[:, None])


def test_level0_zero_row_and_nonfinite():
    W = np.zeros((2, 128), np.float16)
    W[1, 5] = 1.0
    q8, s0 = O.quant_weight_level0(W)
    assert float(s0[0]) == 0 and not q8[0].any()
    assert q8[1, 5] == 119
    W[0, 0] = np.inf
    with pytest.raises(ValueError):
        O.quant_weight_level0(W)


# ------------------------------------------------------ weight level 1

def test_level1_hand_worked_groups():
    fx = read_fixture("level1_groups.txt")
    for g in "ABCDEFG":
        vals = [int(v) for v in fx[f"{g}.q8"]]
        row = np.array(vals + [vals[0]] * (128 - len(vals)), dtype=np.int8)[None, :]
        q4, s1, z = O.quant_weight_level1(row, 128)
        w8 = O.dequant_level1(q4, s1, z, 128)
        assert int(s1[0, 0]) == int(fx[f"{g}.s1"][0]), g
        assert int(z[0, 0]) == int(fx[f"{g}.z"][0]), g
        n = len(vals)
        assert q4[0, :n].tolist() == [int(v) for v in fx[f"{g}.q4"]], g
        assert w8[0, :n].tolist() == [int(v) for v in fx[f"{g}.w8"]], g


def _scan_level1(R):
    """Every (lo, hi, q8) with -R <= lo <= q8 <= hi <= R through the level-1 code."""
    worst = 0
    viol = 0
    max_s1 = 0
    max_zs = 0
    max_prod = 0
    for lo in range(-R, R + 1):
        hi = np.arange(lo, R + 1)[:, None]
        q8 = np.arange(-R, R + 1)[None, :]
        mask = (q8 >= lo) & (q8 <= hi)
        s1, z = O.group_scale_zero(np.full(hi.shape, lo), hi)
        q4 = O.group_codes(q8, s1, z)
        w8 = (q4 - z) * s1
        w8 = np.where(mask, w8, 0)
        worst = max(worst, int(np.abs(w8).max()))
        viol += int(((w8 > 127) | (w8 < -128)).sum())
        max_s1 = max(max_s1, int(s1.max()))
        max_zs = max(max_zs, int((z * s1).max()))
        max_prod = max(max_prod, int(np.where(mask, q4 * s1, 0).max()))
        assert s1.min() >= 1 and z.min() >= 0 and z.max() <= 15
        assert q4.min() >= 0 and q4.max() <= 15
    return worst, viol, max_s1, max_zs, max_prod


def test_protective_range_119_is_safe_exhaustively():
    # The pages: shrinking the level-0 range to [-119, 119] keeps the level-1
    # dequantized intermediates inside INT8 (no saturation needed).
    worst, viol, max_s1, max_zs, max_prod = _scan_level1(119)
    assert viol == 0
    assert worst <= 127
    assert max_s1 == 16          # an 8-bit group scale is needed, 4 bits cannot hold 16
    # properties the packed-byte dequantization relies on:
    assert max_zs <= 127         # z*s1 fits a byte with room for a +128 bias
    assert max_prod <= 255       # q4*s1 never carries out of its byte


@pytest.mark.parametrize("R", [120, 127])
def test_wider_level0_range_overflows_int8(R):
    worst, viol, *_ = _scan_level1(R)
    assert viol > 0 and worst > 127


def test_level1_error_bound_and_roundtrip_on_workload_rows():
    W = synthetic.make_w(64, 2048, seed=7)
    enc = O.encode_weight_g128(W)
    q8, q4, s1, z, w8 = (enc[k].astype(np.int64) for k in ("q8", "q4", "s1", "z", "w8"))
    s1e = np.repeat(s1, 128, axis=1)
    ze = np.repeat(z, 128, axis=1)
    assert np.abs(w8).max() <= 127
    unclamped = (q4 > 0) & (q4 < 15)
    assert np.all(np.abs(w8 - q8)[unclamped] * 2 <= s1e[unclamped])
    # UINT4 -> INT8 in byte lanes mod 256 equals the wide-integer w8
    byte = ((q4 * s1e - ze * s1e) % 256).astype(np.uint8).view(np.int8)
    assert np.array_equal(byte.astype(np.int64), w8)


# ------------------------------------------------------ per-channel W4

def test_per_channel_hand_worked_row():
    fx = read_fixture("per_channel_row.txt")
    W = np.array([fx["w"]], dtype=np.float16)
    q4, s_w, z = O.quant_weight_per_channel(W)
    assert float(s_w[0]) == fx["s_w"][0] and int(s_w.view(np.uint16)[0]) == 0x3266
    assert int(z[0]) == int(fx["z"][0])
    assert q4[0].tolist() == [int(v) for v in fx["q4"]]


def test_per_channel_invariants():
    W = synthetic.make_w(128, 1024, seed=9)
    enc = O.encode_weight_per_channel(W)
    w8 = enc["w8"]
    assert np.abs(w8).max() <= 15
    q4 = enc["q4"].astype(np.int64)
    err = np.abs((q4 - enc["z"].astype(np.int64)[:, None]) * enc["s_w"].astype(np.float64)[:, None]
                 - W.astype(np.float64))
    inner = (q4 > 0) & (q4 < 15)
    assert np.all(err[inner] <= 0.5 * np.broadcast_to(enc["s_w"].astype(np.float64)[:, None], err.shape)[inner] * (1 + 2.0 ** -20))
    # acc through (q4 - z) equals sum x8*q4 - z * sum x8 (zero applied after the contraction)
    X = synthetic.make_x(8, 1024, "frac", seed=2)
    x8, sx = O.quant_act_per_token(X)
    acc = O.gemm_exact(x8, w8)
    alt = O.gemm_int64(x8, q4) - x8.astype(np.int64).sum(1)[:, None] * enc["z"].astype(np.int64)[None, :]
    assert np.array_equal(acc, alt)


# ------------------------------------------------------ GEMM and epilogue

def test_gemm_matches_python_int_bruteforce():
    rng = np.random.default_rng(11)
    x8 = rng.integers(-127, 128, size=(5, 256), dtype=np.int64).astype(np.int8)
    w8 = rng.integers(-121, 122, size=(7, 256), dtype=np.int64)
    assert np.array_equal(O.gemm_exact(x8, w8), O.gemm_bruteforce(x8, w8))
    # extreme magnitudes
    x8 = np.full((2, 384), 127, np.int8); x8[1] = -127
    w8 = np.full((3, 384), 121); w8[1] = -121; w8[2, ::2] = -121
    assert np.array_equal(O.gemm_exact(x8, w8), O.gemm_bruteforce(x8, w8))


def test_gemm_tiny_workload_bruteforce():
    X, W = synthetic.make_inputs("tiny")
    enc = O.encode_weight_g128(W)
    x8, _ = O.quant_act_per_token(X)
    assert np.array_equal(O.gemm_exact(x8[:4], enc["w8"][:9]), O.gemm_bruteforce(x8[:4], enc["w8"][:9]))


def test_gemm_fp64_form_equals_int64_at_attention_size():
    rng = np.random.default_rng(12)
    x8 = rng.integers(-127, 128, size=(256, 4096)).astype(np.int8)
    w8 = rng.integers(-121, 122, size=(128, 4096))
    assert np.array_equal(O.gemm_exact(x8, w8), O.gemm_int64(x8, w8))


def test_gemm_orientation_and_linearity():
    # acc[m, n] contracts row m of x8 with row n of w8 (not a transposed operand)
    x8 = np.zeros((3, 128), np.int8)
    w8 = np.zeros((4, 128), np.int64)
    x8[1, 7] = 127
    w8[2, 7] = -5
    acc = O.gemm_exact(x8, w8)
    assert acc[1, 2] == -635 and np.count_nonzero(acc) == 1
    rng = np.random.default_rng(13)
    a = rng.integers(-60, 61, size=(4, 256)).astype(np.int8)
    b = rng.integers(-60, 61, size=(4, 256)).astype(np.int8)
    w = rng.integers(-121, 122, size=(6, 256))
    assert np.array_equal(O.gemm_exact((a.astype(int) + b).astype(np.int8), w),
                          O.gemm_exact(a, w) + O.gemm_exact(b, w))
    perm = np.concatenate([np.arange(128, 256), np.arange(0, 128)])
    assert np.array_equal(O.gemm_exact(a[:, perm], w[:, perm]), O.gemm_exact(a, w))


def test_epilogue_hand_worked_cases():
    fx = read_fixture("epilogue_cases.txt")
    for i in range(len(fx["acc"])):
        acc = np.array([[int(fx["acc"][i])]], dtype=np.int64)
        y = O.epilogue(acc, np.array([fx["s_x"][i]], np.float16), np.array([fx["s_w"][i]], np.float16))
        assert float(y[0, 0]) == fx["y"][i], i


def test_epilogue_equals_dequantize_then_matmul():
    X, W = synthetic.make_inputs("tiny")
    enc = O.encode_weight_g128(W)
    x8, s_x, acc, y = O.w4a8_forward(X, enc)
    ystar = O.dequant_matmul_fp64(x8, s_x, enc["w8"], enc["s0"])
    exact = acc.astype(np.float64) * s_x.astype(np.float64)[:, None] * enc["s0"].astype(np.float64)[None, :]
    assert np.array_equal(ystar, exact)
    assert np.array_equal(y, ystar.astype(np.float16))
    # and the per-channel variant
    encp = O.encode_weight_per_channel(W)
    _, _, accp, yp = O.w4a8_forward(X, encp)
    assert np.array_equal(yp, O.dequant_matmul_fp64(x8, s_x, encp["w8"], encp["s_w"]).astype(np.float16))


def test_quantized_gemm_tracks_fp_gemm_loosely():
    # Information-level sanity of the whole encoding (the pages give no error
    # bound for one GEMM; this only rules out gross slips such as a lost zero
    # point or a wrong scale).
    X, W = synthetic.make_inputs("tiny")
    ref = X.astype(np.float64) @ W.astype(np.float64).T
    for enc in (O.encode_weight_g128(W), O.encode_weight_per_channel(W)):
        _, _, _, y = O.w4a8_forward(X, enc)
        rel = np.linalg.norm(y.astype(np.float64) - ref) / np.linalg.norm(ref)
        assert rel < 0.2, rel


def test_synthetic_prefix_and_determinism():
    a = synthetic.make_x(64, 512, "frac", 0)
    b = synthetic.make_x(16, 512, "frac", 0)
    assert np.array_equal(a[:16], b)
    assert np.array_equal(synthetic.make_w(32, 256), synthetic.make_w(32, 256))
    cols = synthetic.outlier_channels(8192, "frac")
    assert cols.size == 41 and np.unique(cols).size == 41


# ------------------------------------------------------------ comparators (f1)

def test_w8_hand_worked_row():
    fx = read_fixture("weight_w8_row.txt")
    W = np.array([fx["w"]], dtype=np.float16)
    w8, s = O.quant_weight_w8(W)
    assert float(s[0]) == fx["s"][0]
    assert w8[0].tolist() == [int(v) for v in fx["w8"]]


def test_w8_invariants_and_error_bound():
    W = synthetic.make_w(256, 1024, seed=6)
    w8, s = O.quant_weight_w8(W)
    assert np.abs(w8.astype(int)).max() <= 127
    # each row's largest magnitude lands on the range end
    am = np.argmax(np.abs(W.astype(np.float32)), axis=1)
    assert np.all(np.abs(w8[np.arange(256), am].astype(int)) == 127)
    s64 = s.astype(np.float64)[:, None]
    err = np.abs(w8.astype(np.float64) * s64 - W.astype(np.float64))
    inside = np.abs(W.astype(np.float64)) <= 126.5 * s64
    assert np.all(err[inside] <= 0.5 * s64.repeat(W.shape[1], 1)[inside])
    # a finer grid than the protective level-0 one on the same rows
    _, s0 = O.quant_weight_level0(W)
    assert np.all(s.astype(np.float64) <= s0.astype(np.float64))


def test_w8_zero_row_and_nonfinite():
    W = np.zeros((2, 128), np.float16)
    W[1, 5] = 3.0
    w8, s = O.quant_weight_w8(W)
    assert float(s[0]) == 0 and not w8[0].any()
    assert w8[1, 5] == 127 and int(np.count_nonzero(w8[1])) == 1
    W[1, 7] = np.float16(np.inf)
    with pytest.raises(ValueError):
        O.quant_weight_w8(W)


def test_w8a8_forward_matches_bruteforce():
    X, W = synthetic.make_inputs("tiny")
    enc = O.encode_weight_w8(W)
    x8, s_x, acc, y = O.w4a8_forward(X, enc)
    assert np.array_equal(acc, O.gemm_bruteforce(x8, enc["w8"]))
    yd = O.dequant_matmul_fp64(x8, s_x, enc["w8"], enc["scale"])
    assert np.array_equal(y, O.fp16_rne(yd))


def test_saturating_dequant_hand_cases():
    fx = read_fixture("saturating_dequant.txt")
    q4 = np.array([fx["q4"]], np.uint8)
    s1 = np.array([fx["s1"]], np.uint8)
    z = np.array([fx["z"]], np.uint8)
    assert O.dequant_level1(q4, s1, z, group=1)[0].tolist() == [int(v) for v in fx["plain"]]
    assert O.dequant_level1_saturating(q4, s1, z, group=1)[0].tolist() == [int(v) for v in fx["sat"]]


def test_saturating_dequant_is_exact_inside_the_protective_range():
    W = synthetic.make_w(128, 2048, seed=8)
    enc = O.encode_weight_g128(W)
    sat = O.dequant_level1_saturating(enc["q4"], enc["s1"], enc["z"])
    assert np.array_equal(sat, enc["w8"])


# ------------------------------------------------------- fused producer (f2)

def test_rmsnorm_quant_hand_worked_rows():
    fx = read_fixture("rmsnorm_quant_rows.txt")
    eps = fx["eps"][0]
    assert eps == 2.0 ** -40
    for r in "ab":
        X = np.array([fx["x" + r]], np.float16)
        g = np.array(fx["g" + r], np.float16)
        h = O.rmsnorm_fp16(X, g, eps)
        assert h[0].astype(np.float64).tolist() == fx["h" + r]
        x8, sx = O.rmsnorm_quant_per_token(X, g, eps)
        assert float(sx[0]) == fx["s" + r][0]
        assert x8[0].tolist() == [int(v) for v in fx["q" + r]]


def test_rmsnorm_power_of_two_row_scaling_is_invisible():
    # scaling a row by 2^j scales the exact mean square by 4^j and the rms by
    # 2^j exactly, so with eps below the last bit nothing downstream changes
    X = synthetic.make_x(8, 512, "frac", seed=3)
    g = (synthetic.make_w(1, 512, seed=4)[0] * 40).astype(np.float16)
    x8, sx = O.rmsnorm_quant_per_token(X, g, 2.0 ** -60)
    for j in (-3, 2):
        x8j, sxj = O.rmsnorm_quant_per_token((X.astype(np.float32) * 2.0 ** j).astype(np.float16), g, 2.0 ** -60)
        assert np.array_equal(x8j, x8) and np.array_equal(sxj, sx)


def test_rmsnorm_constant_row_reduces_to_plain_quantizer():
    # a constant row of c = +-2^j has rms |c|, so x * r = +-1 exactly and the
    # fused producer must equal the plain per-token quantizer of +-gamma
    K = 384
    g = (synthetic.make_w(1, K, seed=11)[0] * 100).astype(np.float16)
    for c in (0.125, -4.0, 1.0):
        X = np.full((1, K), c, np.float16)
        x8, sx = O.rmsnorm_quant_per_token(X, g, 2.0 ** -50)
        ref8, refs = O.quant_act_per_token((np.sign(c) * g.astype(np.float32))[None, :].astype(np.float16))
        assert np.array_equal(x8, ref8) and np.array_equal(sx, refs)


def test_rmsnorm_mean_square_is_exact():
    # small integers: the FP64 mean of squares is exact, so ms must equal it;
    # and one huge plus many tiny entries, where the exact sum still rounds
    # to the same FP32 as the huge square alone
    rng = np.random.default_rng(2)
    X = rng.integers(-30, 31, size=(5, 256)).astype(np.float16)
    g = np.ones(256, np.float16)
    h = O.rmsnorm_fp16(X, g, 2.0 ** -60)
    ms = np.mean(X.astype(np.float64) ** 2, axis=1).astype(np.float32)
    r = np.float32(1) / np.sqrt(ms)
    assert np.array_equal(h, (X.astype(np.float32) * r[:, None]).astype(np.float16))
    Y = np.full((1, 1024), 2.0 ** -24, np.float16)
    Y[0, 0] = 60000.0
    hy = O.rmsnorm_fp16(Y, np.ones(1024, np.float16), 2.0 ** -60)
    assert float(hy[0, 0]) == 32.0       # 60000 / (60000 / 32) = 32: rms = 60000 / sqrt(1024)
    assert float(hy[0, 1]) == 0.0        # 2^-24 / 1875 underflows FP16


def test_rmsnorm_zero_row_and_bad_args():
    X = np.zeros((2, 128), np.float16)
    X[1, 3] = 1.0
    x8, sx = O.rmsnorm_quant_per_token(X, np.ones(128, np.float16), 1e-5)
    assert float(sx[0]) == 0 and not x8[0].any()
    assert x8[1, 3] == 127 and int(np.count_nonzero(x8[1])) == 1
    with pytest.raises(ValueError):
        O.rmsnorm_fp16(X, np.ones(128, np.float16), 0.0)
    with pytest.raises(ValueError):
        O.rmsnorm_fp16(X, np.ones(64, np.float16), 1e-5)


def _fp16_nearest_exact(val, candidates):
    """The FP16 value among candidates nearest to the exact value val
    (a Decimal or a Fraction), ties to the even mantissa."""
    v = Fraction(val)
    return min(candidates, key=lambda c: (abs(Fraction(float(c)) - v), int(np.array(c, np.float16).view(np.uint16)) & 1))


def _fp16_neighbours(x):
    c = np.float16(x)
    with np.errstate(over="ignore"):
        cands = [c, np.nextafter(c, np.float16(np.inf)), np.nextafter(c, np.float16(-np.inf))]
    return [v for v in cands if np.isfinite(v)]


def test_silu_fp16_every_finite_half_against_decimal():
    # silu(g) = g / (1 + e^-g) to 50 significant digits (Decimal's exp is
    # correctly rounded), then the nearest FP16: must equal the oracle's
    # FP64 evaluation for every finite FP16 input
    getcontext().prec = 50
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    g = bits.view(np.float16)
    g = g[np.isfinite(g)]
    got = O.silu_fp16(g)
    bad = 0
    for gv, out in zip(g.tolist(), got.tolist()):
        d = Decimal(gv)
        if d < -200:      # |silu| < 2^-200: rounds to -0 (the oracle's e^-g overflows to inf)
            want = -0.0
        else:
            ex = Decimal(float(d)).__neg__().exp()
            val = d / (1 + ex)
            want = float(_fp16_nearest_exact(val, _fp16_neighbours(float(val))))
            if want == 0:
                want = -0.0 if val < 0 or d.is_signed() else 0.0
        bad += np.float16(want).view(np.uint16) != np.float16(out).view(np.uint16)
    assert bad == 0
    # sign and size: 0 <= silu(g) <= g above zero, g <= silu(g) <= 0 below
    g64, s64 = g.astype(np.float64), got.astype(np.float64)
    assert np.all((s64 >= np.minimum(g64, 0)) & (s64 <= np.maximum(g64, 0)))


def test_swiglu_product_rounds_once_half_to_even():
    # h = fp16(s * u) with s = silu_fp16(g): against exact rational products
    rng = np.random.default_rng(8)
    G = rng.standard_normal(4000).astype(np.float16) * np.float16(3)
    U = (rng.standard_normal(4000) * 7).astype(np.float16)
    h = O.swiglu_fp16(G, U)
    s = O.silu_fp16(G)
    for sv, uv, hv in zip(s.tolist(), U.tolist(), h.tolist()):
        exact = Fraction(sv) * Fraction(uv)
        assert hv == float(_fp16_nearest_exact(exact, _fp16_neighbours(float(exact))))


def test_swiglu_quant_hand_worked_rows():
    fx = read_fixture("swiglu_rows.txt")
    for r in range(2):
        G = np.array([fx[f"g{r}"]], np.float16)
        U = np.array([fx[f"u{r}"]], np.float16)
        x8, sx, h = O.swiglu_quant_per_token(G, U)
        assert h[0].astype(np.float64).tolist() == fx[f"h{r}"]
        assert float(sx[0]) == fx[f"s{r}"][0]
        assert x8[0].tolist() == [int(v) for v in fx[f"q{r}"]]
    with pytest.raises(ValueError):   # 300 * 300 overflows FP16
        O.swiglu_quant_per_token(np.full((1, 4), 300, np.float16), np.full((1, 4), 300, np.float16))


def test_swiglu_with_large_gate_reduces_to_plain_quantizer_of_up_times_gate():
    # for g >= 24 (an FP16 value), silu(g) rounds to g itself (g e^-g is far
    # below half an ulp), so h = fp16(g * u) and the fused producer equals
    # the plain quantizer of that product
    rng = np.random.default_rng(5)
    G = np.full((3, 256), 32.0, np.float16)
    U = rng.standard_normal((3, 256)).astype(np.float16)
    assert np.array_equal(O.silu_fp16(G), G)
    x8, sx, h = O.swiglu_quant_per_token(G, U)
    ref8, refs = O.quant_act_per_token((G.astype(np.float64) * U.astype(np.float64)).astype(np.float16))
    assert np.array_equal(x8, ref8) and np.array_equal(sx, refs)


# ------------------------------------------------------------------ KV4 (f3)

def test_kv4_quant_hand_worked_row():
    fx = read_fixture("kv4_row.txt")
    q, sc, z = O.kv4_quant_per_head(np.array([fx["x"]], np.float16))
    assert q[0].tolist() == [int(v) for v in fx["q"]]
    assert float(sc[0]) == fx["s"][0] and int(z[0]) == fx["z"][0]


def test_kv4_quant_is_per_row_over_leading_axes():
    X = synthetic.make_x(2 * 3 * 5, 128, "frac", seed=2).reshape(2, 3, 5, 128)
    q, sc, z = O.kv4_quant_per_head(X)
    assert q.shape == X.shape and sc.shape == (2, 3, 5) and z.shape == (2, 3, 5)
    q2, s2, z2 = O.quant_weight_per_channel(X[1, 2])
    assert np.array_equal(q[1, 2], q2) and np.array_equal(sc[1, 2], s2) and np.array_equal(z[1, 2], z2)
    deq = O.kv4_dequant(q, sc, z)
    err = np.abs(deq - X.astype(np.float64))
    assert np.all(err <= 0.5 * sc.astype(np.float64)[..., None] + 1e-12)


def _kv_case(B, H, Hkv, T, d=128, seed=0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, d)).astype(np.float16)
    K = rng.standard_normal((B, Hkv, T, d)).astype(np.float16)
    V = rng.standard_normal((B, Hkv, T, d)).astype(np.float16)
    return q, O.kv4_quant_per_head(K), O.kv4_quant_per_head(V)


def _attn(q, kk, vv, lengths, scale=0.08838834764831845):
    return O.kv4_decode_attention(q, *kk, *vv, lengths, scale)


def test_kv4_attention_single_token_returns_its_value():
    q, kk, vv = _kv_case(2, 2, 2, 1, seed=1)
    o = _attn(q, kk, vv, [1, 1])
    assert np.array_equal(o, O.fp16_rne(O.kv4_dequant(*vv)[:, :, 0]))


def test_kv4_attention_zero_query_averages_values():
    q, kk, vv = _kv_case(1, 2, 2, 37, seed=2)
    o = _attn(np.zeros_like(q), kk, vv, [37])
    assert np.array_equal(o, O.fp16_rne(O.kv4_dequant(*vv).mean(axis=2)))
    assert np.array_equal(o, _attn(q, kk, vv, [37], scale=0.0))


def test_kv4_attention_token_order_does_not_matter():
    q, kk, vv = _kv_case(1, 3, 3, 50, seed=3)
    perm = np.random.default_rng(0).permutation(50)
    pk = tuple(a[:, :, perm] for a in kk)
    pv = tuple(a[:, :, perm] for a in vv)
    a, b = _attn(q, kk, vv, [50]).astype(np.float64), _attn(q, pk, pv, [50]).astype(np.float64)
    assert np.all(np.abs(a - b) <= 2.0 ** -10 * np.abs(a) + 2.0 ** -24)


def test_kv4_attention_dominant_key_selects_its_value():
    q, kk, vv = _kv_case(1, 1, 1, 20, seed=4)
    kq, ks, kz = (a.copy() for a in kk)
    j = 13
    qs = np.sign(q[0, 0].astype(np.float64))
    kq[0, 0, j] = np.where(qs > 0, 15, 0)      # key aligned with q at the range ends
    kz[0, 0, j] = 8
    ks[0, 0, j] = np.float16(8.0)               # score ~ 8 * 7.5 * sum|q| * scale: hundreds
    o = _attn(q, (kq, ks, kz), vv, [20])
    assert np.array_equal(o[0, 0], O.fp16_rne(O.kv4_dequant(*vv)[0, 0, j]))
    # the opposite sign picks some other token instead
    o2 = _attn(-q, (kq, ks, kz), vv, [20])
    assert not np.array_equal(o2[0, 0], o[0, 0])


def test_kv4_attention_gqa_equals_duplicated_heads():
    q, kk, vv = _kv_case(2, 4, 2, 9, seed=5)
    dup = lambda t: tuple(np.repeat(a, 2, axis=1) for a in t)
    assert np.array_equal(_attn(q, kk, vv, [9, 9]), _attn(q, dup(kk), dup(vv), [9, 9]))


def test_kv4_attention_lengths_are_prefixes():
    q, kk, vv = _kv_case(3, 2, 2, 16, seed=6)
    o = _attn(q, kk, vv, [16, 5, 0])
    cut = lambda t, n: tuple(a[:, :, :n] for a in t)
    assert np.array_equal(o[1], _attn(q[1:2], cut(tuple(a[1:2] for a in kk), 5), cut(tuple(a[1:2] for a in vv), 5), [5])[0])
    assert not o[2].any()


def test_kv4_attention_query_scale_equals_softmax_scale():
    q, kk, vv = _kv_case(1, 2, 2, 30, seed=7)
    a = _attn(q, kk, vv, [30], scale=0.25)
    b = _attn((q.astype(np.float32) * 2).astype(np.float16), kk, vv, [30], scale=0.125)
    assert np.array_equal(a, b)


# ------------------------------------------------- offline transforms (f4)

def test_hadamard_closed_form_and_orthogonality():
    # entry (i, j) of the normalized Sylvester matrix is (-1)^popcount(i & j) / sqrt(n)
    n = 64
    H = O.hadamard_matrix(n)
    i, j = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")
    par = np.vectorize(lambda v: bin(int(v)).count("1") & 1)(i & j)
    assert np.array_equal(H, np.where(par, -1.0, 1.0) / 8.0)
    assert np.allclose(H @ H.T, np.eye(n), atol=1e-15)
    assert np.array_equal(O.hadamard_matrix(2), np.array([[1.0, 1.0], [1.0, -1.0]]) / np.sqrt(2.0))


def test_hadamard_blocks_for_non_power_of_two():
    assert O.hadamard_block_size(14336) == 2048 and O.hadamard_block_size(4096) == 4096
    assert O.hadamard_block_size(384) == 128
    H = O.hadamard_matrix(384)
    assert np.allclose(H @ H.T, np.eye(384), atol=1e-14)
    assert not H[:128, 128:].any() and np.array_equal(H[128:256, 128:256], O.hadamard_matrix(128))


def test_rotation_and_smoothing_leave_the_product_unchanged():
    X = synthetic.make_x(8, 256, "frac", seed=1).astype(np.float64)
    W = synthetic.make_w(16, 256, seed=1).astype(np.float64)
    H = O.hadamard_matrix(256)
    assert np.allclose((X @ H) @ (W @ H).T, X @ W.T, rtol=0, atol=1e-12)
    lam = O.smoothing_factors(np.abs(X).max(0), np.abs(W).max(0), 0.5).astype(np.float64)
    assert np.allclose((X / lam) @ (W * lam).T, X @ W.T, rtol=0, atol=1e-12)


def test_smoothing_factor_hand_cases():
    lam = O.smoothing_factors([4.0, 9.0, 0.0, 2.0, 16.0], [1.0, 4.0, 3.0, 0.0, 1.0], 0.5)
    assert lam.tolist() == [2.0, 1.5, 1.0, 1.0, 4.0]
    assert O.smoothing_factors([8.0], [2.0], 1.0).tolist() == [8.0]   # alpha = 1: all on the activation side
    assert O.smoothing_factors([8.0], [2.0], 0.0).tolist() == [0.5]   # alpha = 0: 1 / w


def test_scale_columns_hand_worked_cases():
    # tests/golden/scale_columns.txt: orientation (multiply against divide),
    # one FP16 rounding of the exact FP64 product (case 4 would round to the
    # other neighbour through FP32), overflow to inf, a subnormal tie, exact
    # halvings, and the factor running along the last axis
    fx = read_fixture("scale_columns.txt")
    for x, f, d, y in zip(fx["x"], fx["f"], fx["divide"], fx["y"]):
        got = O.scale_columns(np.array([[x]], np.float16), np.array([f]), divide=bool(d))
        assert got.dtype == np.float16
        assert got[0, 0].view(np.uint16) == np.float16(y).view(np.uint16), (x, f, d, y, got[0, 0])
    X = np.array(fx["mat_x"], np.float16).reshape(2, 2)
    got = O.scale_columns(X, np.array(fx["mat_f"]))
    assert np.array_equal(got, np.array(fx["mat_y"], np.float16).reshape(2, 2))
    # divide=True with the same factors undoes it exactly here (powers of two and
    # small integers)
    assert np.array_equal(O.scale_columns(got, np.array(fx["mat_f"]), divide=True), X)


def test_smooth_attention_keeps_scores_and_lowers_key_error():
    # SmoothAttention: keys / lambda, queries * lambda with lambda = max|k|^0.5
    # per channel (w = 1).  The scores are unchanged before rounding, and on
    # keys with fixed outlier channels the INT4 key error drops (information
    # about the transform on synthetic keys)
    rng = np.random.default_rng(3)
    K = rng.standard_normal((512, 128)).astype(np.float32)
    K[:, [5, 40, 77, 100]] *= 20
    K = K.astype(np.float16)
    qv = rng.standard_normal(128).astype(np.float16)
    lam = O.smoothing_factors(np.abs(K.astype(np.float64)).max(0), np.ones(128), 0.5).astype(np.float64)
    K64, q64 = K.astype(np.float64), qv.astype(np.float64)
    assert np.allclose((K64 / lam) @ (q64 * lam), K64 @ q64, rtol=0, atol=1e-10)

    def key_err(Kq, factor):
        d = O.kv4_dequant(*O.kv4_quant_per_head(Kq)) * factor
        return np.linalg.norm(d - K64) / np.linalg.norm(K64)

    plain = key_err(K, 1.0)
    smooth = key_err(O.scale_columns(K, lam, divide=True), lam)
    assert smooth < 0.5 * plain, (plain, smooth)


def test_rotation_spreads_activation_outliers():
    # synthetic rows with x20 outlier channels: after the rotation no channel
    # dominates, so the per-token INT8 step is finer (information about the
    # value of the transform, on synthetic data; the rotation is orthogonal,
    # so the norms compared are those of the same vectors)
    X = synthetic.make_x(64, 1024, "frac", seed=2)

    def act_err(Xi):
        x8, sx = O.quant_act_per_token(Xi)
        d = x8.astype(np.float64) * sx.astype(np.float64)[:, None]
        return np.linalg.norm(d - Xi.astype(np.float64)) / np.linalg.norm(Xi.astype(np.float64))

    e_plain, e_rot = act_err(X), act_err(O.rotate_rows(X))
    assert e_rot < 0.25 * e_plain, (e_plain, e_rot)
