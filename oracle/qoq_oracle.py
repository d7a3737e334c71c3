"""QoQ W4A8 oracle: plain CPU reference of the W4A8 GEMM path.

ORACLE -- TEST INFRASTRUCTURE ONLY.  Nothing in the product library imports,
links or calls this file; only the tests, the smoke check and the benchmark's
``cpu_baseline`` leg do.  It shares no code with the HIP library.

Sources followed (cited by tag in each docstring):

  [PL]   "QServe: W4A8KV4 Quantization and System Co-design for Efficient LLM
         Serving" -- section-by-section summary page, paperlayer.ai
         abs/2405.04532v3.  Cited as [PL §n, <bullet topic>].
  [ABS]  the arXiv abstract of the same paper (mlsanity.com index page).
  [SS]   study.space summary page of the same paper.

Notation.  X[M,K] FP16 activations (tokens x input channels), W[N,K] FP16
weights (output x input channels), Y[M,N] = X W^T.  The [PL §2] summary calls
the token count N; this file uses M for tokens and N for output channels.

Precision.  The pages fix FP16 for the per-channel weight scale
([PL §4, progressive group quantization]).  Every
step that decides an integer code (activation and weight quantization) is
taken in IEEE FP32 with round-half-to-even, the precision the GPU kernel uses;
the epilogue is evaluated exactly in FP64 and rounded once to FP16.

Readings taken where the pages are silent or garbled, those that shape the
arithmetic here:
  * group scale stored as an 8-bit integer in [1, 16] (one page calls the
    group scales 4-bit, which cannot hold 16), rounded to nearest;
  * round half to even everywhere;
  * level-1 code = round(q8 / s1) + z, rounding before adding the zero;
  * plain min/max group range (0 not forced in), zero clamped to [0, 15];
  * zero-range rows/tokens get scale 0 and all-zero codes;
  * activation scale stored as FP16 and the quantizer divides by the stored
    value.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "ACT_QMAX",
    "W8_PROTECT",
    "U4_MAX",
    "GROUP",
    "fp16_rne",
    "rne_div",
    "quant_act_per_token",
    "quant_weight_level0",
    "group_scale_zero",
    "group_codes",
    "quant_weight_level1",
    "dequant_level1",
    "encode_weight_g128",
    "quant_weight_per_channel",
    "encode_weight_per_channel",
    "gemm_exact",
    "gemm_int64",
    "gemm_bruteforce",
    "epilogue",
    "dequant_matmul_fp64",
    "w4a8_forward",
    "W8_QMAX",
    "quant_weight_w8",
    "encode_weight_w8",
    "dequant_level1_saturating",
    "rmsnorm_fp16",
    "rmsnorm_quant_per_token",
    "silu_fp16",
    "swiglu_fp16",
    "swiglu_quant_per_token",
    "kv4_quant_per_head",
    "kv4_dequant",
    "kv4_decode_attention",
    "hadamard_block_size",
    "hadamard_matrix",
    "rotate_rows",
    "smoothing_factors",
    "scale_columns",
]

ACT_QMAX = 127   # symmetric INT8 activation range [-127, 127]
W8_PROTECT = 119  # protective INT8 range for the level-0 weight codes
U4_MAX = 15       # UINT4 code range [0, 15]
GROUP = 128       # group size along K of the level-1 (g128) quantization
W8_QMAX = 127     # symmetric INT8 range of the W8A8 comparator's weights


def fp16_rne(a) -> np.ndarray:
    """Round FP32/FP64 values to FP16, round-half-to-even, in one step.

    NumPy converts float64 and float32 to float16 directly (no intermediate
    float32 rounding of a float64), with IEEE round-half-to-even, subnormals
    and overflow to +-inf.
    """
    return np.asarray(a).astype(np.float16)


def rne_div(a, s):
    """Integer a / s (s > 0) rounded to nearest, ties to even, exactly.

    Floor division gives a = q*s + r with 0 <= r < s; the quotient is rounded
    up when the remainder is more than half of s, or exactly half and q odd.
    """
    a = np.asarray(a, dtype=np.int64)
    s = np.asarray(s, dtype=np.int64)
    q, r = np.divmod(a, s)
    up = (2 * r > s) | ((2 * r == s) & (q % 2 == 1))
    return q + up.astype(np.int64)


def quant_act_per_token(X):
    """Per-token symmetric INT8 activation quantization.

    [PL §6, experimental setup]: activations are quantized per token to INT8;
    [PL §5, runtime and precision mapping]: the W4A8 GEMM consumes INT8
    activations.  Per row m:  a = max_k |X[m,k]|,  s_x = fp16(a / 127),
    x8 = clamp(round(X / s_x), -127, 127); a zero scale gives a zero row.

    Returns (x8 int8 [M,K], s_x float16 [M]).
    """
    X32 = np.asarray(X, dtype=np.float16).astype(np.float32)
    a = np.max(np.abs(X32), axis=1) if X32.shape[1] else np.zeros(X32.shape[0], np.float32)
    s_x = fp16_rne(a / np.float32(ACT_QMAX))
    s32 = s_x.astype(np.float32)
    safe = np.where(s32 == 0, np.float32(1), s32)
    q = np.rint(X32 / safe[:, None])
    q = np.clip(q, -ACT_QMAX, ACT_QMAX)
    q[s32 == 0, :] = 0
    return q.astype(np.int8), s_x


def _per_channel_symmetric(W, qmax):
    """Per-output-channel symmetric INT8: s = fp16(max|W| / qmax),
    q = clamp(round(W / s), -qmax, qmax); a zero scale gives a zero row.
    The division and the rounding are taken in FP32 (the precision that
    decides the codes on the device too)."""
    W32 = np.asarray(W, dtype=np.float16).astype(np.float32)
    if not np.all(np.isfinite(W32)):
        raise ValueError("non-finite weight")
    b = np.max(np.abs(W32), axis=1)
    s = fp16_rne(b / np.float32(qmax))
    s32 = s.astype(np.float32)
    safe = np.where(s32 == 0, np.float32(1), s32)
    q = np.clip(np.rint(W32 / safe[:, None]), -qmax, qmax)
    q[s32 == 0, :] = 0
    return q.astype(np.int8), s


def quant_weight_level0(W):
    """Progressive quantization, level 0: per-output-channel symmetric INT8.

    [PL §4, progressive group quantization]: weights are first quantized per
    channel to INT8 with channel-wise FP16 scales, and the INT8 range is shrunk
    to the protective range [-119, 119] so that the level-1 dequantized values
    cannot overflow INT8.  [SS]: first to 8 bits with per-channel FP16 scales.
    Per row n:  b = max_k |W[n,k]|,  s0 = fp16(b / 119),
    q8 = clamp(round(W / s0), -119, 119); a zero scale gives a zero row.

    Returns (q8 int8 [N,K], s0 float16 [N]).
    """
    return _per_channel_symmetric(W, W8_PROTECT)


def group_scale_zero(lo, hi):
    """Level-1 group scale and zero point from the group's INT8 min and max.

    [PL §4, progressive group quantization]: the INT8 intermediates are
    quantized per group to 4 bits with an integer group scale and a zero
    point; [PL §2, integer quantization]: asymmetric quantization maps a range
    onto the n-bit levels with a scale and a zero point.  With d = hi - lo:
      s1 = max(1, round(d / 15))   -- d is an integer and 15 is odd, so
                                      d / 15 is never a tie and
                                      round(d / 15) == (d + 7) // 15
      z  = clamp(round(-lo / s1), 0, 15)
    """
    lo = np.asarray(lo, dtype=np.int64)
    hi = np.asarray(hi, dtype=np.int64)
    s1 = np.maximum(1, (hi - lo + 7) // U4_MAX)
    z = np.clip(rne_div(-lo, s1), 0, U4_MAX)
    return s1, z


def group_codes(q8, s1, z):
    """Level-1 UINT4 code of an INT8 intermediate: clamp(round(q8/s1) + z, 0, 15)."""
    return np.clip(rne_div(q8, s1) + np.asarray(z, dtype=np.int64), 0, U4_MAX)


def quant_weight_level1(q8, group=GROUP):
    """Progressive quantization, level 1: per-group (g128) asymmetric UINT4.

    [PL §2, integer quantization]: with group quantization each run of g
    consecutive input channels of a row gets its own scale and zero point;
    [PL §6, experimental setup]: the g128 variant uses group size 128.

    Returns (q4 uint8 [N,K], s1 uint8 [N,K/g], z uint8 [N,K/g]).
    """
    q8 = np.asarray(q8, dtype=np.int64)
    N, K = q8.shape
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    g = q8.reshape(N, K // group, group)
    lo = g.min(axis=2)
    hi = g.max(axis=2)
    s1, z = group_scale_zero(lo, hi)
    q4 = group_codes(g, s1[..., None], z[..., None]).reshape(N, K)
    return q4.astype(np.uint8), s1.astype(np.uint8), z.astype(np.uint8)


def dequant_level1(q4, s1, z, group=GROUP):
    """INT8 intermediate the GEMM multiplies: w8 = (q4 - z) * s1.

    [PL §5, W4A8 GEMM optimization]: subtraction after multiplication,
    w8 = q4*s1 - z*s1, on the integer codes; the protective level-0 range keeps
    it inside INT8.  Returned as int64 so an overflow would be visible.
    """
    q4 = np.asarray(q4, dtype=np.int64)
    N, K = q4.shape
    s1e = np.repeat(np.asarray(s1, dtype=np.int64), group, axis=1)
    ze = np.repeat(np.asarray(z, dtype=np.int64), group, axis=1)
    return q4 * s1e - ze * s1e


def encode_weight_g128(W, group=GROUP):
    """Full progressive group quantization of W (level 0 then level 1).

    Returns a dict with q8, s0 (level 0), q4, s1, z (level 1) and w8, the
    INT8 intermediate that the GEMM consumes.
    """
    q8, s0 = quant_weight_level0(W)
    q4, s1, z = quant_weight_level1(q8, group)
    w8 = dequant_level1(q4, s1, z, group)
    return {"q8": q8, "s0": s0, "q4": q4, "s1": s1, "z": z, "w8": w8,
            "scale": s0, "group_size": group}


def quant_weight_per_channel(W):
    """Per-channel W4 (the pages' "W4A8KV4" variant without the g128 level).

    [PL §6, experimental setup]: the per-channel counterpart of the g128
    variant quantizes weights per output channel.  Direct FP16 -> UINT4,
    asymmetric, with an FP16 scale and a UINT4 zero per channel:
      s_w = fp16((max W - min W) / 15),  z = clamp(round(-min W / s_w), 0, 15),
      q4 = clamp(round(W / s_w) + z, 0, 15);  a zero scale gives zero codes.

    Returns (q4 uint8 [N,K], s_w float16 [N], z uint8 [N]).
    """
    W32 = np.asarray(W, dtype=np.float16).astype(np.float32)
    if not np.all(np.isfinite(W32)):
        raise ValueError("non-finite weight")
    hi = W32.max(axis=1)
    lo = W32.min(axis=1)
    s_w = fp16_rne((hi - lo) / np.float32(U4_MAX))
    s32 = s_w.astype(np.float32)
    safe = np.where(s32 == 0, np.float32(1), s32)
    z = np.clip(np.rint(-lo / safe), 0, U4_MAX)
    q4 = np.clip(np.rint(W32 / safe[:, None]) + z[:, None], 0, U4_MAX)
    dead = s32 == 0
    z[dead] = 0
    q4[dead, :] = 0
    return q4.astype(np.uint8), s_w, z.astype(np.uint8)


def encode_weight_per_channel(W):
    """Per-channel W4 encode; w8 = q4 - z lies in [-15, 15]."""
    q4, s_w, z = quant_weight_per_channel(W)
    w8 = q4.astype(np.int64) - z.astype(np.int64)[:, None]
    return {"q4": q4, "s_w": s_w, "z": z, "w8": w8, "scale": s_w, "group_size": 0}


def gemm_exact(x8, w8):
    """acc[m,n] = sum_k x8[m,k] * w8[n,k], exactly, as int64.

    [PL §1/§8]: progressive quantization keeps the W4A8 GEMM on INT8 tensor
    cores with one INT32 accumulator over all of K.  Evaluated as an FP64
    matrix product: every product and partial sum is an integer of magnitude
    at most 127*127*K < 2**53, so the FP64 result is exact whatever the
    summation order.  Asserts the INT32 range.
    """
    a = np.asarray(x8, dtype=np.float64)
    b = np.asarray(w8, dtype=np.float64)
    K = a.shape[1]
    if 127 * 127 * K >= 2 ** 53:
        raise ValueError("K too large for the exact FP64 form")
    acc = a @ b.T
    out = acc.astype(np.int64)
    if out.size and np.max(np.abs(out)) >= 2 ** 31:
        raise OverflowError("accumulator leaves INT32")
    return out


def gemm_int64(x8, w8):
    """Same contraction in int64 arithmetic (NumPy integer matmul, no BLAS)."""
    return np.asarray(x8, dtype=np.int64) @ np.asarray(w8, dtype=np.int64).T


def gemm_bruteforce(x8, w8):
    """Same contraction with Python integers in a triple loop (tiny shapes)."""
    xl = np.asarray(x8).tolist()
    wl = np.asarray(w8).tolist()
    M, N = len(xl), len(wl)
    out = np.zeros((M, N), dtype=np.int64)
    for m in range(M):
        xr = xl[m]
        for n in range(N):
            wr = wl[n]
            s = 0
            for k in range(len(xr)):
                s += int(xr[k]) * int(wr[k])
            out[m, n] = s
    return out


def epilogue(acc, s_x, s_w):
    """y[m,n] = fp16(acc[m,n] * s_x[m] * s_w[n]).

    [PL §5, W4A8 GEMM optimization]: the per-channel scale is fused into the
    GEMM epilogue; [PL §5, runtime and precision mapping]: the W4A8 GEMM
    writes FP16.  The FP64 products are exact (|acc| < 2**28 times two 11-bit
    significands fits in 53 bits), so y is the correctly rounded FP16 of the
    exact dequantized product.
    """
    a = np.asarray(acc, dtype=np.float64)
    sx = np.asarray(s_x, dtype=np.float16).astype(np.float64)
    sw = np.asarray(s_w, dtype=np.float16).astype(np.float64)
    return fp16_rne(a * sx[:, None] * sw[None, :])


def dequant_matmul_fp64(x8, s_x, w8, s_w):
    """Y* = (diag(s_x) x8)(diag(s_w) w8)^T in FP64, before any FP16 rounding.

    A second route to the same value: dequantize both operands to real
    numbers, then multiply.  Exact in FP64 for the same reason as
    ``epilogue``: every term shares the factor s_x[m]*s_w[n].
    """
    xd = np.asarray(x8, dtype=np.float64) * np.asarray(s_x, np.float16).astype(np.float64)[:, None]
    wd = np.asarray(w8, dtype=np.float64) * np.asarray(s_w, np.float16).astype(np.float64)[:, None]
    return xd @ wd.T


def w4a8_forward(X, enc):
    """The whole online path: per-token quant, exact integer GEMM, epilogue.

    ``enc`` is the dict returned by ``encode_weight_g128`` or
    ``encode_weight_per_channel``.  Returns (x8, s_x, acc, y).
    """
    x8, s_x = quant_act_per_token(X)
    acc = gemm_exact(x8, enc["w8"])
    y = epilogue(acc, s_x, enc["scale"])
    return x8, s_x, acc, y


# ------------------------------------------------------------------ comparators

def quant_weight_w8(W):
    """Per-channel symmetric INT8 weights of the W8A8 comparator GEMM.

    [SS]: the W4A8 GEMM is compared with an INT8 (W8A8) library GEMM;
    [PL §6, accuracy evaluation]: W8A8 SmoothQuant is the 8-bit baseline;
    [PL §2, integer quantization]: symmetric quantization with one scale per
    output channel.  The full INT8 range is used (there is no second level to
    protect).  Per row n:  s_w = fp16(max_k |W[n,k]| / 127),
    w8 = clamp(round(W / s_w), -127, 127); a zero scale gives a zero row.

    Returns (w8 int8 [N,K], s_w float16 [N]).
    """
    return _per_channel_symmetric(W, W8_QMAX)


def encode_weight_w8(W):
    """W8A8 comparator weights in the form ``w4a8_forward`` takes."""
    w8, s_w = quant_weight_w8(W)
    return {"w8": w8.astype(np.int64), "scale": s_w, "group_size": None}


def dequant_level1_saturating(q4, s1, z, group=GROUP):
    """Level-1 dequantization clamped to INT8: clip((q4 - z) * s1, -128, 127).

    [PL §4, progressive group quantization]: without the protective level-0
    range the dequantized intermediates can leave INT8 and the GEMM would have
    to saturate them, which the pages report as costly.  This is that
    saturating form; on codes from ``encode_weight_g128`` it equals
    ``dequant_level1`` (their values stay within [-121, 121]).
    """
    return np.clip(dequant_level1(q4, s1, z, group), -128, 127)


# ------------------------------------------------------- fused producer (f2)

def rmsnorm_fp16(X, gamma, eps):
    """RMS normalization of FP16 token rows, rounded to FP16.

    [PL §5, runtime and precision mapping]: the per-token quantizer runs
    inside the normalization that produces the activations; here that is the
    RMS normalization of the token (x / rms(x) * gamma, the Llama-family norm)
    followed by the per-token INT8 quantization.  The pages give no
    arithmetic, so the statistic is taken exactly and rounded once:
      S    = sum_k x_k^2, exact (every FP16 value is an integer times 2^-24,
             so S is an integer times 2^-48: Python integers hold it);
      ms   = fp32(fp64(S) / K)        -- S rounded to FP64, IEEE division;
      r    = 1 / sqrt(ms + eps)       -- FP32 add, sqrt and division;
      h_k  = fp16((x_k * r) * gamma_k) -- two FP32 products, then FP16.
    Every step is a single correctly rounded IEEE operation, so the result
    does not depend on any summation order.

    Returns h float16 [M, K].
    """
    X16 = np.asarray(X, dtype=np.float16)
    g32 = np.asarray(gamma, dtype=np.float16).astype(np.float32)
    M, K = X16.shape
    if g32.shape != (K,):
        raise ValueError("gamma must have K entries")
    eps32 = np.float32(eps)
    if not eps32 > 0:
        raise ValueError("eps must be positive")
    units = (X16.astype(np.float64) * 2.0 ** 24).astype(np.int64)  # exact integers
    h = np.empty((M, K), np.float16)
    for m in range(M):
        S = sum(v * v for v in units[m].tolist())
        ms = np.float32(float(S) * 2.0 ** -48 / K)
        r = np.float32(1.0) / np.sqrt(np.float32(ms + eps32))
        h[m] = ((X16[m].astype(np.float32) * r) * g32).astype(np.float16)
    return h


def rmsnorm_quant_per_token(X, gamma, eps):
    """Fused producer: RMS normalization then per-token INT8 quantization.

    The quantization is ``quant_act_per_token`` applied to the FP16
    normalized rows of ``rmsnorm_fp16`` -- fusing the two moves no value.
    Returns (x8 int8 [M,K], s_x float16 [M]).
    """
    return quant_act_per_token(rmsnorm_fp16(X, gamma, eps))


def silu_fp16(G):
    """SiLU of FP16 values, rounded once to FP16.

    [PL §5, runtime and precision mapping]: activation quantization also runs
    inside the activation-function kernel that produces a layer's input.  In
    the Llama-family FFN the down projection's input is SiLU(gate) * up.  The
    pages give no arithmetic for it; the reading taken here rounds each FP16
    step once:  silu(g) = g / (1 + e^-g)  evaluated in FP64 and rounded to
    FP16.  For every finite FP16 g the exact value lies at least 4.8e-12
    (relative) from the nearest FP16 rounding boundary, far beyond the FP64
    evaluation's error, so the result is the correctly rounded FP16 value
    (checked against 60-digit decimal arithmetic in the tests).

    Returns float16, the shape of G.
    """
    g = np.asarray(G, dtype=np.float16).astype(np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        s = g / (1.0 + np.exp(-g))
    return fp16_rne(s)


def swiglu_fp16(G, U):
    """h = fp16(silu_fp16(g) * u): the product of two FP16 values is exact in
    FP64 and is rounded once to FP16 (round half to even).

    Returns float16 [M, K].
    """
    s = silu_fp16(G).astype(np.float64)
    u = np.asarray(U, dtype=np.float16).astype(np.float64)
    if s.shape != u.shape:
        raise ValueError("gate and up must have the same shape")
    return fp16_rne(s * u)


def swiglu_quant_per_token(G, U):
    """Fused producer of the down projection's input: h = SiLU(gate) * up
    (``swiglu_fp16``), then the per-token INT8 quantization of those FP16
    values (``quant_act_per_token``).  The activations must stay finite.

    Returns (x8 int8 [M,K], s_x float16 [M], h float16 [M,K]).
    """
    h = swiglu_fp16(G, U)
    if not np.all(np.isfinite(h)):
        raise ValueError("SiLU(gate) * up overflows FP16")
    x8, s_x = quant_act_per_token(h)
    return x8, s_x, h


# ------------------------------------------------------------------ KV4 (f3)

def kv4_quant_per_head(X):
    """Per-head dynamic asymmetric INT4 quantization of key or value vectors.

    [PL §6, experimental setup]: the KV cache is per-head asymmetric INT4;
    [PL §5, KV4 attention]: the scaling factors and zero points are per head
    and computed at run time.  Every row of X (last axis = one head's vector
    of one token) gets its own FP16 scale and UINT4 zero point, by the same
    asymmetric UINT4 map as the per-channel weights:
      s = fp16((max x - min x) / 15),  z = clamp(round(-min x / s), 0, 15),
      q = clamp(round(x / s) + z, 0, 15);  a zero scale gives zero codes.

    X: float16 [..., d].  Returns (q uint8 [..., d], s float16 [...],
    z uint8 [...]).
    """
    X16 = np.asarray(X, dtype=np.float16)
    lead, d = X16.shape[:-1], X16.shape[-1]
    q4, s, z = quant_weight_per_channel(X16.reshape(-1, d))
    return q4.reshape(*lead, d), s.reshape(lead), z.reshape(lead)


def kv4_dequant(q4, s, z):
    """(q - z) * s, exactly, in FP64 (broadcast over the last axis)."""
    q = np.asarray(q4, dtype=np.float64)
    zz = np.asarray(z, dtype=np.float64)[..., None]
    ss = np.asarray(s, dtype=np.float16).astype(np.float64)[..., None]
    return (q - zz) * ss


def kv4_decode_attention(q, kq, ks, kz, vq, vs, vz, lengths, softmax_scale):
    """Decode attention over a KV4 cache, in FP64, rounded once to FP16.

    [PL §5, KV4 attention]: the attention of the newest token reads the INT4
    cache, dequantizes it with the per-head scales and zero points, and
    computes in floating point; [PL §4, SmoothAttention]: queries stay
    unquantized.  Per sequence b and query head h, with kv head
    g = h // (H / Hkv) and L = lengths[b] cached tokens:
      k_t = (kq - kz) * ks, v_t = (vq - vz) * vs       (t < L)
      a_t = softmax_t(scale * <q[b,h], k_t>)
      o[b,h] = fp16(sum_t a_t v_t);  L = 0 gives o = 0.

    q float16 [B, H, d]; kq/vq uint8 codes [B, Hkv, T, d]; ks/vs float16 and
    kz/vz uint8 [B, Hkv, T]; lengths int [B]; softmax_scale a float (taken
    as FP32).  Returns float16 [B, H, d].
    """
    q64 = np.asarray(q, dtype=np.float16).astype(np.float64)
    B, H, d = q64.shape
    Hkv = np.asarray(kq).shape[1]
    if H % Hkv:
        raise ValueError("query heads must be a multiple of kv heads")
    scale = float(np.float32(softmax_scale))
    out = np.zeros((B, H, d), np.float64)
    for b in range(B):
        L = int(lengths[b])
        if L == 0:
            continue
        for h in range(H):
            g = h // (H // Hkv)
            K = kv4_dequant(kq[b, g, :L], ks[b, g, :L], kz[b, g, :L])
            V = kv4_dequant(vq[b, g, :L], vs[b, g, :L], vz[b, g, :L])
            sc = scale * (K @ q64[b, h])
            e = np.exp(sc - sc.max())
            out[b, h] = (e / e.sum()) @ V
    return fp16_rne(out)


# ------------------------------------------------- offline transforms (f4)

def hadamard_block_size(K):
    """Largest power of two dividing K: the block of the rotation."""
    K = int(K)
    if K < 1:
        raise ValueError("K must be positive")
    return K & -K


def hadamard_matrix(K):
    """Orthogonal rotation of the K input channels, in FP64.

    [PL §4, activation optimizations]: block inputs are rotated by a unitary
    matrix that is absorbed into the preceding weights.  The pages name no
    matrix; this is the normalized Walsh-Hadamard one (entries +-1/sqrt(b),
    the Sylvester construction), block-diagonal with b = the largest power of
    two dividing K when K is not a power of two (14336 = 7 * 2048).
    """
    b = hadamard_block_size(K)
    h = np.ones((1, 1))
    while h.shape[0] < b:
        h = np.block([[h, h], [h, -h]])
    h = h / np.sqrt(b)
    return np.kron(np.eye(K // b), h)


def rotate_rows(X, K=None):
    """fp16(X @ H) for FP16 rows X [.., K]: the rotated activations or weights
    (Y = X W^T = (X H)(W H)^T since H H^T = I)."""
    X64 = np.asarray(X, dtype=np.float16).astype(np.float64)
    K = X64.shape[-1] if K is None else K
    return fp16_rne(X64 @ hadamard_matrix(K))


def smoothing_factors(act_absmax, w_absmax, alpha):
    """Per-channel smoothing factors, lambda_j = a_j^alpha / w_j^(1 - alpha).

    [PL §4, activation optimizations]: output modules use per-channel
    smoothing factors; [PL §4, SmoothAttention]: keys are scaled down with
    alpha = 0.5 (there the weight side is absent: w = 1).  The form is the
    SmoothQuant one the pages build on.  A channel whose activation or weight
    maximum is 0 gets lambda = 1.  FP64, returned as FP32.
    """
    a = np.asarray(act_absmax, dtype=np.float64)
    w = np.asarray(w_absmax, dtype=np.float64)
    ok = (a > 0) & (w > 0)
    lam = np.ones(np.broadcast(a, w).shape)
    lam[ok] = a[ok] ** alpha / w[ok] ** (1.0 - alpha)
    return lam.astype(np.float32)


def scale_columns(X, factor, divide=False):
    """fp16(X * factor) (or X / factor) along the last axis, in FP64: weights
    take lambda, the activations (through the preceding layer) 1/lambda."""
    X64 = np.asarray(X, dtype=np.float16).astype(np.float64)
    f = np.asarray(factor, dtype=np.float32).astype(np.float64)
    return fp16_rne(X64 / f if divide else X64 * f)
