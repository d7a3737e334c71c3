// Offline accuracy transforms of the QoQ pipeline (host).
//
// "QServe: W4A8KV4 Quantization and System Co-design for Efficient LLM
// Serving" (paperlayer.ai summary), §4 activation optimizations: block inputs
// are rotated by a unitary matrix absorbed into the preceding weights, and
// the inputs of output modules are smoothed per channel; §4 SmoothAttention:
// outlier key channels are scaled down (alpha = 0.5) and the queries scaled
// up by the same factors.  All are exact identities of the product,
//   X W^T = (X H)(W H)^T = (X / lambda)(W * lambda)^T,
// applied offline to weights (and, through the preceding layer, to
// activations); the W4A8 path then quantizes the transformed tensors.
//
// Rotation: the normalized Walsh-Hadamard matrix, block-diagonal with blocks
// of b = the largest power of two dividing K, applied as a fast transform in
// FP64 and rounded once to FP16.  Smoothing factors:
//   lambda_j = a_j^alpha / w_j^(1 - alpha)  (1 where a_j or w_j is 0).

#include <cmath>
#include <cstring>
#include <vector>

#include "qoq_internal.h"

namespace qoq {
namespace {

double half_bits_to_double(uint16_t h) {
  const int sign = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 0) v = std::ldexp(double(m), -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = std::ldexp(double(1024 + m), e - 25);
  return sign ? -v : v;
}

// FP64 -> FP16, one rounding to nearest, ties to even; overflow to inf.
uint16_t double_to_half_rne(double d) {
  const uint16_t sign = std::signbit(d) ? 0x8000 : 0;
  const double x = std::fabs(d);
  if (std::isnan(x)) return uint16_t(sign | 0x7e00);
  if (x == 0.0) return sign;
  int e;
  std::frexp(x, &e);  // x = f * 2^e, f in [0.5, 1): leading bit 2^(e-1)
  const int lead = e - 1;
  if (lead < -14) {  // subnormal range: units of 2^-24, exact scaling then RNE
    const double q = std::nearbyint(std::ldexp(x, 24));
    return uint16_t(sign | uint16_t(q));  // q == 1024 encodes the smallest normal
  }
  double mant = std::nearbyint(std::ldexp(x, 10 - lead));  // in [1024, 2048]
  int ex = lead;
  if (mant == 2048.0) {
    mant = 1024.0;
    ++ex;
  }
  if (ex > 15) return uint16_t(sign | 0x7c00);
  return uint16_t(sign | uint16_t((ex + 15) << 10) | uint16_t(int(mant) - 1024));
}

}  // namespace
}  // namespace qoq

using namespace qoq;

extern "C" int qoq_hadamard_rotate(const uint16_t* in_fp16, int64_t rows, int64_t K, int64_t ld,
                                   uint16_t* out_fp16) {
  clear_error();
  if (!in_fp16 || !out_fp16) return fail(QOQ_ERR_INVALID_ARG, "qoq_hadamard_rotate: null pointer argument");
  if (rows < 1 || K < 1) return fail(QOQ_ERR_UNSUPPORTED_SHAPE, "qoq_hadamard_rotate: rows and K must be >= 1");
  if (ld < K) return fail(QOQ_ERR_INVALID_ARG, "qoq_hadamard_rotate: ld < K");
  const int64_t b = K & -K;
  const double norm = 1.0 / std::sqrt(double(b));
  std::vector<double> v(static_cast<size_t>(K));
  for (int64_t r = 0; r < rows; ++r) {
    const uint16_t* src = in_fp16 + r * ld;
    for (int64_t k = 0; k < K; ++k) v[size_t(k)] = half_bits_to_double(src[k]);
    for (int64_t blk = 0; blk < K; blk += b) {
      double* a = v.data() + blk;
      for (int64_t len = 1; len < b; len <<= 1)
        for (int64_t i = 0; i < b; i += 2 * len)
          for (int64_t j = i; j < i + len; ++j) {
            const double p = a[j], q = a[j + len];
            a[j] = p + q;
            a[j + len] = p - q;
          }
    }
    uint16_t* dst = out_fp16 + r * ld;
    for (int64_t k = 0; k < K; ++k) dst[k] = double_to_half_rne(v[size_t(k)] * norm);
  }
  return QOQ_OK;
}

extern "C" int qoq_smoothing_factors(const float* act_absmax, const float* w_absmax, int64_t K, float alpha,
                                     float* lambda) {
  clear_error();
  if (!act_absmax || !w_absmax || !lambda) return fail(QOQ_ERR_INVALID_ARG, "qoq_smoothing_factors: null pointer");
  if (K < 1) return fail(QOQ_ERR_UNSUPPORTED_SHAPE, "qoq_smoothing_factors: K must be >= 1");
  if (!(alpha >= 0.0f && alpha <= 1.0f)) return fail(QOQ_ERR_INVALID_ARG, "qoq_smoothing_factors: alpha not in [0, 1]");
  const double al = alpha;
  for (int64_t k = 0; k < K; ++k) {
    const double a = act_absmax[k], w = w_absmax[k];
    lambda[k] = (a > 0 && w > 0) ? float(std::pow(a, al) / std::pow(w, 1.0 - al)) : 1.0f;
  }
  return QOQ_OK;
}

extern "C" int qoq_scale_columns(const uint16_t* in_fp16, int64_t rows, int64_t K, int64_t ld, const float* factor,
                                 int32_t divide, uint16_t* out_fp16) {
  clear_error();
  if (!in_fp16 || !factor || !out_fp16) return fail(QOQ_ERR_INVALID_ARG, "qoq_scale_columns: null pointer argument");
  if (rows < 1 || K < 1) return fail(QOQ_ERR_UNSUPPORTED_SHAPE, "qoq_scale_columns: rows and K must be >= 1");
  if (ld < K) return fail(QOQ_ERR_INVALID_ARG, "qoq_scale_columns: ld < K");
  for (int64_t k = 0; k < K; ++k)
    if (!(factor[k] > 0.0f) || !std::isfinite(factor[k]))
      return fail(QOQ_ERR_INVALID_ARG, "qoq_scale_columns: factor %lld is not positive and finite", (long long)k);
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t k = 0; k < K; ++k) {
      const double x = half_bits_to_double(in_fp16[r * ld + k]);
      const double f = factor[k];
      out_fp16[r * ld + k] = double_to_half_rne(divide ? x / f : x * f);
    }
  return QOQ_OK;
}
