// Host-side exercise of libqoq's CPU code (weight packer, code packer,
// unpacker, layout query, offline transforms), built with AddressSanitizer
// and UndefinedBehaviorSanitizer by tests/test_host_sanitizers.py.  It checks
// round trips and error paths; any out-of-bounds access, use of
// uninitialized heap, overflow or misaligned access aborts the run under the
// sanitizers.  Prints "host_sanitize: ok" on success.

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "qoq.h"

namespace {

int g_failures = 0;

#define CHECK(cond)                                                     \
  do {                                                                  \
    if (!(cond)) {                                                      \
      std::printf("FAILED %s:%d: %s\n", __FILE__, __LINE__, #cond);     \
      ++g_failures;                                                     \
    }                                                                   \
  } while (0)

// Deterministic generator (64-bit LCG, high bits).
struct Lcg {
  uint64_t s;
  explicit Lcg(uint64_t seed) : s(seed * 2862933555777941757ull + 3037000493ull) {}
  uint32_t next() {
    s = s * 6364136223846793005ull + 1442695040888963407ull;
    return uint32_t(s >> 33);
  }
};

// FP16 bits of v = n / 1024 for |n| < 2048: exactly representable (at most
// 11 significant bits, and |v| >= 2^-10 lies in the normal range).
uint16_t half_of_ratio(int n) {
  if (n == 0) return 0;
  const uint16_t sign = n < 0 ? 0x8000 : 0;
  int a = n < 0 ? -n : n;
  int e = 0;
  while (a < 1024) {
    a <<= 1;
    --e;
  }
  // |v| = |n| / 1024 = (a / 1024) * 2^e with a / 1024 in [1, 2): biased exponent e + 15
  const int exp = e + 15;
  return uint16_t(sign | (uint16_t(exp) << 10) | uint16_t(a - 1024));
}

// Value of finite FP16 bits (normal or subnormal).
double half_value(uint16_t h) {
  const int e = (h >> 10) & 31, m = h & 1023;
  const double v = e ? std::ldexp(double(1024 + m), e - 25) : std::ldexp(double(m), -24);
  return (h & 0x8000) ? -v : v;
}

std::vector<uint16_t> random_weights(int64_t N, int64_t K, uint64_t seed) {
  Lcg r(seed);
  std::vector<uint16_t> w(size_t(N * K));
  for (auto& v : w) v = half_of_ratio(int(r.next() % 2047) - 1023);
  // a zero row and a constant row exercise the degenerate branches
  if (N > 2) {
    for (int64_t k = 0; k < K; ++k) w[size_t(1 * K + k)] = 0;
    for (int64_t k = 0; k < K; ++k) w[size_t(2 * K + k)] = half_of_ratio(300);
  }
  return w;
}

void pack_round_trip(int64_t N, int64_t K, int32_t gs, uint64_t seed) {
  qoq_weight_layout L;
  CHECK(qoq_weight_layout_query(N, K, gs, &L) == QOQ_OK);
  const auto w = random_weights(N, K, seed);
  std::vector<uint8_t> qw(L.qweight_bytes), meta(L.meta_bytes);
  std::vector<uint16_t> sc(L.scale_bytes / 2);
  CHECK(qoq_pack_weights(w.data(), N, K, gs, qw.data(), meta.data(), sc.data()) == QOQ_OK);

  const int64_t G = K / 128;
  const int64_t nm = gs ? N * G : N;
  std::vector<uint8_t> q4(static_cast<size_t>(N * K)), s1(static_cast<size_t>(gs ? nm : 1)), z(static_cast<size_t>(nm));
  std::vector<uint16_t> sc2(static_cast<size_t>(N));
  CHECK(qoq_unpack_weights(qw.data(), meta.data(), sc.data(), N, K, gs, q4.data(), gs ? s1.data() : nullptr,
                           z.data(), sc2.data()) == QOQ_OK);
  for (size_t i = 0; i < q4.size(); ++i) CHECK(q4[i] <= 15);
  if (gs)
    for (size_t i = 0; i < s1.size(); ++i) CHECK(s1[i] >= 1 && s1[i] <= 16 && z[i] <= 15);

  // packing the unpacked codes again gives the same bytes
  std::vector<uint8_t> qw2(L.qweight_bytes), meta2(L.meta_bytes);
  std::vector<uint16_t> sc3(L.scale_bytes / 2);
  CHECK(qoq_pack_codes(q4.data(), gs ? s1.data() : nullptr, z.data(), sc2.data(), N, K, gs, qw2.data(),
                       meta2.data(), sc3.data()) == QOQ_OK);
  CHECK(std::memcmp(qw.data(), qw2.data(), qw.size()) == 0);
  CHECK(std::memcmp(meta.data(), meta2.data(), meta.size()) == 0);
  CHECK(std::memcmp(sc.data(), sc3.data(), sc.size() * 2) == 0);

  // the INT8 comparator's packer on the same weights
  std::vector<uint8_t> q8(size_t(L.N_pad * K));
  std::vector<uint16_t> s8(size_t(L.N_pad));
  CHECK(qoq_pack_weights_w8(w.data(), N, K, q8.data(), s8.data()) == QOQ_OK);
}

void error_paths() {
  qoq_weight_layout L;
  CHECK(qoq_weight_layout_query(16, 100, 128, &L) == QOQ_ERR_UNSUPPORTED_SHAPE);
  CHECK(qoq_weight_layout_query(16, 128, 64, &L) != QOQ_OK);
  CHECK(qoq_weight_layout_query(0, 128, 128, &L) != QOQ_OK);
  CHECK(qoq_weight_layout_query(16, 128, 128, nullptr) == QOQ_ERR_INVALID_ARG);
  std::vector<uint16_t> w(16 * 128, 0);
  CHECK(qoq_pack_weights(w.data(), 16, 128, 128, nullptr, nullptr, nullptr) == QOQ_ERR_INVALID_ARG);
  CHECK(std::strlen(qoq_last_error()) > 0);
  // a non-finite weight is rejected
  CHECK(qoq_weight_layout_query(16, 128, 128, &L) == QOQ_OK);
  std::vector<uint8_t> qw(L.qweight_bytes), meta(L.meta_bytes);
  std::vector<uint16_t> sc(L.scale_bytes / 2);
  w[5] = 0x7c00;  // +inf
  CHECK(qoq_pack_weights(w.data(), 16, 128, 128, qw.data(), meta.data(), sc.data()) == QOQ_ERR_INVALID_ARG);
  // codes whose z * s1 exceeds 128 are rejected by the code packer
  std::vector<uint8_t> q4(16 * 128, 0), s1(16, 16), z(16, 15);
  std::vector<uint16_t> s0(16, 0x3c00);
  CHECK(qoq_pack_codes(q4.data(), s1.data(), z.data(), s0.data(), 16, 128, 128, qw.data(), meta.data(),
                       sc.data()) == QOQ_ERR_INVALID_ARG);
  for (int s = 0; s < 8; ++s) CHECK(qoq_status_string(s) != nullptr);
}

void transforms(uint64_t seed) {
  const int64_t rows = 5, K = 384, ld = 400;  // blocks of 128, padded rows
  Lcg r(seed);
  std::vector<uint16_t> x(size_t(rows * ld), 0), y(size_t(rows * ld), 0), z(size_t(rows * ld), 0);
  for (int64_t i = 0; i < rows; ++i)
    for (int64_t k = 0; k < K; ++k) x[size_t(i * ld + k)] = half_of_ratio(int(r.next() % 2047) - 1023);
  CHECK(qoq_hadamard_rotate(x.data(), rows, K, ld, y.data()) == QOQ_OK);
  CHECK(qoq_hadamard_rotate(y.data(), rows, K, ld, z.data()) == QOQ_OK);
  // H H = I: rotating twice returns the row up to the FP16 rounding of the
  // rotated row, spread over the row (bounded by 2^-8 of its RMS)
  for (int64_t i = 0; i < rows; ++i) {
    double ss = 0;
    for (int64_t k = 0; k < K; ++k) ss += half_value(x[size_t(i * ld + k)]) * half_value(x[size_t(i * ld + k)]);
    const double rms = std::sqrt(ss / double(K));
    for (int64_t k = 0; k < K; ++k)
      CHECK(std::fabs(half_value(x[size_t(i * ld + k)]) - half_value(z[size_t(i * ld + k)])) <= rms / 256.0);
  }
  CHECK(qoq_hadamard_rotate(x.data(), rows, K, K - 1, y.data()) == QOQ_ERR_INVALID_ARG);
  std::vector<float> a(static_cast<size_t>(K)), wm(static_cast<size_t>(K)), lam(static_cast<size_t>(K));
  for (int64_t k = 0; k < K; ++k) {
    a[size_t(k)] = float(r.next() % 100) / 10.0f;  // includes zeros
    wm[size_t(k)] = float(r.next() % 50 + 1) / 100.0f;
  }
  CHECK(qoq_smoothing_factors(a.data(), wm.data(), K, 0.5f, lam.data()) == QOQ_OK);
  for (int64_t k = 0; k < K; ++k) CHECK(lam[size_t(k)] > 0.0f && std::isfinite(lam[size_t(k)]));
  CHECK(qoq_smoothing_factors(a.data(), wm.data(), K, 1.5f, lam.data()) == QOQ_ERR_INVALID_ARG);
  CHECK(qoq_scale_columns(x.data(), rows, K, ld, lam.data(), 0, y.data()) == QOQ_OK);
  CHECK(qoq_scale_columns(y.data(), rows, K, ld, lam.data(), 1, z.data()) == QOQ_OK);
  lam[7] = 0.0f;
  CHECK(qoq_scale_columns(x.data(), rows, K, ld, lam.data(), 0, y.data()) == QOQ_ERR_INVALID_ARG);
}

}  // namespace

int main() {
  // shapes with ragged strips (N not a multiple of 16), a single group, and
  // a group count that is not a multiple of 4 (padded metadata runs); the
  // last one is large enough to take the threaded packer
  const int64_t shapes[][2] = {{1, 128}, {17, 384}, {33, 640}, {64, 1280}, {2048, 2048}};
  uint64_t seed = 1;
  for (const auto& s : shapes) {
    pack_round_trip(s[0], s[1], 128, seed++);
    pack_round_trip(s[0], s[1], 0, seed++);
  }
  error_paths();
  transforms(seed);
  if (g_failures) {
    std::printf("host_sanitize: %d failures\n", g_failures);
    return 1;
  }
  std::printf("host_sanitize: ok\n");
  return 0;
}
