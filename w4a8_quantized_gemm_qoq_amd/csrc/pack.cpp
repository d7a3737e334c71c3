// Host-side offline weight encode and packer of libqoq.so.
//
// Implements the progressive group quantization of
//   "QServe: W4A8KV4 Quantization and System Co-design for Efficient LLM
//   Serving" (paperlayer.ai abs/2405.04532v3 summary), §4 "QoQ Quantization",
//   progressive group quantization: per-output-channel INT8 with an FP16
//   scale inside the protective range [-119, 119], then per-group (128 along
//   K) UINT4 with an integer group scale and a UINT4 zero point;
// and the per-channel W4 variant of §6 (experimental setup).  The packed
// order follows §5 (compute-aware weight reordering: weights stored in the
// order the GEMM consumes them), laid out for the gfx950 INT8 MFMA operand
// fragments: see the layout comment in qoq.h.
//
// Arithmetic mirrors the definitions exactly: FP32 IEEE division, FP16
// round-half-to-even for stored scales, rintf (round half to even under the
// default rounding mode) for codes, exact integer arithmetic for level 1.
// Build without -ffast-math.

#include <algorithm>
#include <cmath>
#include <cstring>
#include <thread>
#include <vector>

#include "qoq_internal.h"

namespace qoq {
namespace {

inline float bits_to_float(uint32_t u) {
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}
inline uint32_t float_to_bits(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return u;
}

// IEEE binary16 -> binary32 (exact).
float half_to_float(uint16_t h) {
  const uint32_t sign = uint32_t(h & 0x8000u) << 16;
  const uint32_t e = (h >> 10) & 0x1fu;
  const uint32_t m = h & 0x3ffu;
  if (e == 0) {
    const float f = float(m) * 5.9604644775390625e-08f;  // m * 2^-24, exact
    return sign ? -f : f;
  }
  if (e == 31) return bits_to_float(sign | 0x7f800000u | (m << 13));
  return bits_to_float(sign | ((e + 112u) << 23) | (m << 13));
}

// IEEE binary32 -> binary16, round to nearest, ties to even; overflow to inf.
uint16_t float_to_half_rne(float f) {
  const uint32_t x = float_to_bits(f);
  const uint16_t sign = uint16_t((x >> 16) & 0x8000u);
  const uint32_t ax = x & 0x7fffffffu;
  if (ax >= 0x7f800000u) return uint16_t(sign | 0x7c00u | (ax > 0x7f800000u ? 0x200u : 0u));
  if (ax >= 0x477ff000u) return uint16_t(sign | 0x7c00u);  // >= 65520 rounds to inf
  if (ax >= 0x38800000u) {                                 // normal binary16 result
    const uint32_t e = (ax >> 23) - 112u;
    const uint32_t m = ax & 0x7fffffu;
    uint32_t h = (e << 10) | (m >> 13);
    const uint32_t rem = m & 0x1fffu;
    if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) ++h;  // carry may bump the exponent
    return uint16_t(sign | h);
  }
  // subnormal binary16 (or zero): result counts units of 2^-24
  const uint32_t e = ax >> 23;
  if (e == 0) return sign;                   // binary32 subnormal: far below 2^-25
  const uint32_t M = (ax & 0x7fffffu) | 0x800000u;  // value = M * 2^(e-150)
  const uint32_t shift = 126u - e;           // value / 2^-24 = M >> shift
  if (shift >= 25) return sign;              // below 2^-25: rounds to zero
  uint32_t q = M >> shift;
  const uint32_t rem = M & ((1u << shift) - 1u);
  const uint32_t half = 1u << (shift - 1u);
  if (rem > half || (rem == half && (q & 1u))) ++q;
  return uint16_t(sign | q);
}

// Integer a / s (s > 0) rounded to nearest, ties to even.
inline int rne_div(int a, int s) {
  int q = a / s, r = a % s;
  if (r < 0) { q -= 1; r += s; }
  if (2 * r > s || (2 * r == s && (q & 1))) q += 1;
  return q;
}

inline int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

struct Dims {
  int64_t N, K, N_pad, G, G4;
  int group_size;
};

Dims dims_of(int64_t N, int64_t K, int32_t group_size) {
  Dims d;
  d.N = N;
  d.K = K;
  d.N_pad = round_up(N, kStrip);
  d.G = K / kGroup;
  d.G4 = round_up(d.G, 4);
  d.group_size = group_size;
  return d;
}

inline size_t meta_index(const Dims& d, int64_t n, int64_t g) {
  const int64_t strip = n / kStrip, c = n % kStrip;
  return size_t(((strip * (d.G4 / 4) + g / 4) * kStrip + c) * 4 + (g % 4));
}

// Scatter one channel's UINT4 codes into the packed blocks.
void scatter_row(const Dims& d, int64_t n, const uint8_t* q4row, uint8_t* qw) {
  const int64_t strip = n / kStrip;
  const int c = int(n % kStrip);
  for (int64_t g = 0; g < d.G; ++g) {
    uint8_t* blk = qw + size_t(strip * d.G + g) * kBlockBytes;
    const uint8_t* src = q4row + g * kGroup;
    for (int kl = 0; kl < kGroup; ++kl) {
      int off, high;
      code_position(c, kl, &off, &high);
      if (high)
        blk[off] = uint8_t((blk[off] & 0x0f) | (src[kl] << 4));
      else
        blk[off] = uint8_t((blk[off] & 0xf0) | (src[kl] & 0x0f));
    }
  }
}

void gather_row(const Dims& d, int64_t n, const uint8_t* qw, uint8_t* q4row) {
  const int64_t strip = n / kStrip;
  const int c = int(n % kStrip);
  for (int64_t g = 0; g < d.G; ++g) {
    const uint8_t* blk = qw + size_t(strip * d.G + g) * kBlockBytes;
    for (int kl = 0; kl < kGroup; ++kl) {
      int off, high;
      code_position(c, kl, &off, &high);
      q4row[g * kGroup + kl] = high ? uint8_t(blk[off] >> 4) : uint8_t(blk[off] & 0x0f);
    }
  }
}

// Run fn(n0, n1) over [0, N) on up to hardware_concurrency threads.  Rows are
// independent; each 16-channel strip is written by exactly one thread.
template <class F>
void parallel_rows(int64_t N, F fn) {
  unsigned hw = std::thread::hardware_concurrency();
  if (hw == 0) hw = 1;
  const int64_t strips = (N + kStrip - 1) / kStrip;
  const int64_t nthreads = std::min<int64_t>(std::min<int64_t>(hw, 64), std::max<int64_t>(1, strips / 8));
  if (nthreads <= 1) {
    fn(int64_t(0), N);
    return;
  }
  std::vector<std::thread> th;
  const int64_t per = (strips + nthreads - 1) / nthreads;
  for (int64_t t = 0; t < nthreads; ++t) {
    const int64_t n0 = std::min(N, t * per * kStrip);
    const int64_t n1 = std::min(N, (t + 1) * per * kStrip);
    if (n0 >= n1) break;
    th.emplace_back([=] { fn(n0, n1); });
  }
  for (auto& x : th) x.join();
}

// Level 0 + level 1 of one channel (g128).  Returns false on non-finite input.
bool encode_row_g128(const uint16_t* w, int64_t K, uint8_t* q4, uint8_t* s1, uint8_t* z,
                     uint16_t* s0_out, std::vector<int>& q8) {
  float b = 0.0f;
  for (int64_t k = 0; k < K; ++k) {
    const float v = half_to_float(w[k]);
    if (!std::isfinite(v)) return false;
    b = std::max(b, std::fabs(v));
  }
  const uint16_t s0h = float_to_half_rne(b / 119.0f);
  const float s0 = half_to_float(s0h);
  *s0_out = s0h;
  for (int64_t k = 0; k < K; ++k) {
    if (s0 == 0.0f) {
      q8[k] = 0;
    } else {
      const float q = std::rint(half_to_float(w[k]) / s0);
      q8[k] = clampi(int(q), -119, 119);
    }
  }
  const int64_t G = K / kGroup;
  for (int64_t g = 0; g < G; ++g) {
    const int* q = q8.data() + g * kGroup;
    int lo = q[0], hi = q[0];
    for (int i = 1; i < kGroup; ++i) {
      lo = std::min(lo, q[i]);
      hi = std::max(hi, q[i]);
    }
    const int sc = std::max(1, (hi - lo + 7) / 15);  // hi - lo >= 0: truncation == floor
    const int zz = clampi(rne_div(-lo, sc), 0, 15);
    s1[g] = uint8_t(sc);
    z[g] = uint8_t(zz);
    for (int i = 0; i < kGroup; ++i) q4[g * kGroup + i] = uint8_t(clampi(rne_div(q[i], sc) + zz, 0, 15));
  }
  return true;
}

// Per-channel W4 of one channel.  Returns false on non-finite input.
bool encode_row_per_channel(const uint16_t* w, int64_t K, uint8_t* q4, uint8_t* z, uint16_t* s_out) {
  float hi = -INFINITY, lo = INFINITY;
  for (int64_t k = 0; k < K; ++k) {
    const float v = half_to_float(w[k]);
    if (!std::isfinite(v)) return false;
    hi = std::max(hi, v);
    lo = std::min(lo, v);
  }
  const uint16_t sh = float_to_half_rne((hi - lo) / 15.0f);
  const float s = half_to_float(sh);
  *s_out = sh;
  if (s == 0.0f) {
    *z = 0;
    std::memset(q4, 0, size_t(K));
    return true;
  }
  const float zf = std::min(15.0f, std::max(0.0f, std::rint(-lo / s)));
  *z = uint8_t(zf);
  for (int64_t k = 0; k < K; ++k) {
    const float q = std::rint(half_to_float(w[k]) / s) + zf;
    q4[k] = uint8_t(std::min(15.0f, std::max(0.0f, q)));
  }
  return true;
}

// Per-channel symmetric INT8 of one channel (the W8A8 comparator's weights):
// s = fp16(max_k |W| / 127), q = clamp(round(W / s), -127, 127); a zero scale
// gives a zero row.  Returns false on non-finite input.
bool encode_row_w8(const uint16_t* w, int64_t K, int8_t* q, uint16_t* s_out) {
  float b = 0.0f;
  for (int64_t k = 0; k < K; ++k) {
    const float v = half_to_float(w[k]);
    if (!std::isfinite(v)) return false;
    b = std::max(b, std::fabs(v));
  }
  const uint16_t sh = float_to_half_rne(b / 127.0f);
  const float s = half_to_float(sh);
  *s_out = sh;
  for (int64_t k = 0; k < K; ++k)
    q[k] = s == 0.0f ? int8_t(0) : int8_t(clampi(int(std::rint(half_to_float(w[k]) / s)), -127, 127));
  return true;
}

// INT8 block of (strip, group): 128 slots of 16 bytes, slot c + 16j + 64h
// holding input channels 128g + 64h + 16j + [0, 16) of channel c.
void scatter_row_w8(const Dims& d, int64_t n, const int8_t* qrow, uint8_t* qw) {
  const int64_t strip = n / kStrip;
  const int c = int(n % kStrip);
  for (int64_t g = 0; g < d.G; ++g) {
    uint8_t* blk = qw + size_t(strip * d.G + g) * kBlockBytesW8;
    for (int kl = 0; kl < kGroup; ++kl) {
      const int slot = c + 16 * ((kl >> 4) & 3) + 64 * (kl >> 6);
      blk[slot * 16 + (kl & 15)] = uint8_t(qrow[g * kGroup + kl]);
    }
  }
}

void write_meta_g128(const Dims& d, int64_t n, const uint8_t* s1, const uint8_t* z, uint8_t* meta) {
  for (int64_t g = 0; g < d.G; ++g) meta[meta_index(d, n, g)] = uint8_t((s1[g] - 1) | (z[g] << 4));
}

int check_ptrs(const char* fn, std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (!p) return fail(QOQ_ERR_INVALID_ARG, "%s: null pointer argument", fn);
  return QOQ_OK;
}

}  // namespace

int check_weight_shape(int64_t N, int64_t K, int32_t group_size) {
  if (group_size != 0 && group_size != kGroup)
    return fail(QOQ_ERR_INVALID_ARG, "group_size must be 128 or 0 (per-channel), got %d", group_size);
  if (N < 1) return fail(QOQ_ERR_UNSUPPORTED_SHAPE, "N must be >= 1, got %lld", (long long)N);
  if (K < kGroup || K % kGroup)
    return fail(QOQ_ERR_UNSUPPORTED_SHAPE, "K must be a positive multiple of 128, got %lld", (long long)K);
  if (K > kMaxK)
    return fail(QOQ_ERR_UNSUPPORTED_SHAPE, "K=%lld exceeds %lld (INT32 accumulator bound)", (long long)K,
                (long long)kMaxK);
  if (N > (int64_t(1) << 31) - 16)
    return fail(QOQ_ERR_UNSUPPORTED_SHAPE, "N=%lld too large", (long long)N);
  return QOQ_OK;
}

}  // namespace qoq

using namespace qoq;

extern "C" int qoq_weight_layout_query(int64_t N, int64_t K, int32_t group_size, qoq_weight_layout* out) {
  clear_error();
  if (!out) return fail(QOQ_ERR_INVALID_ARG, "qoq_weight_layout_query: null out");
  if (int st = check_weight_shape(N, K, group_size)) return st;
  const Dims d = dims_of(N, K, group_size);
  out->layout_id = QOQ_LAYOUT_ID;
  out->group_size = group_size;
  out->N = N;
  out->K = K;
  out->N_pad = d.N_pad;
  out->n_groups = d.G;
  out->qweight_bytes = size_t(d.N_pad) * size_t(K) / 2;
  out->meta_bytes = group_size ? size_t(d.N_pad / kStrip) * size_t(d.G4) * kStrip : size_t(d.N_pad);
  out->scale_bytes = size_t(d.N_pad) * 2;
  return QOQ_OK;
}

extern "C" int qoq_pack_weights(const uint16_t* w_fp16, int64_t N, int64_t K, int32_t group_size,
                                void* qweight, void* meta, uint16_t* scale_fp16) {
  clear_error();
  if (int st = check_ptrs("qoq_pack_weights", {w_fp16, qweight, meta, scale_fp16})) return st;
  qoq_weight_layout L;
  if (int st = qoq_weight_layout_query(N, K, group_size, &L)) return st;
  const Dims d = dims_of(N, K, group_size);
  uint8_t* qw = static_cast<uint8_t*>(qweight);
  uint8_t* mt = static_cast<uint8_t*>(meta);
  std::memset(qw, 0, L.qweight_bytes);
  std::memset(mt, 0, L.meta_bytes);
  std::memset(scale_fp16, 0, L.scale_bytes);
  std::vector<char> bad(size_t(N), 0);
  parallel_rows(N, [&](int64_t n0, int64_t n1) {
    std::vector<uint8_t> q4(static_cast<size_t>(K)), s1(static_cast<size_t>(d.G)), z(static_cast<size_t>(d.G));
    std::vector<int> q8(static_cast<size_t>(K));
    for (int64_t n = n0; n < n1; ++n) {
      const uint16_t* w = w_fp16 + size_t(n) * size_t(K);
      bool ok;
      if (group_size) {
        ok = encode_row_g128(w, K, q4.data(), s1.data(), z.data(), &scale_fp16[n], q8);
        if (ok) write_meta_g128(d, n, s1.data(), z.data(), mt);
      } else {
        ok = encode_row_per_channel(w, K, q4.data(), &mt[n], &scale_fp16[n]);
      }
      if (!ok) {
        bad[size_t(n)] = 1;
        continue;
      }
      scatter_row(d, n, q4.data(), qw);
    }
  });
  for (int64_t n = 0; n < N; ++n)
    if (bad[size_t(n)]) return fail(QOQ_ERR_INVALID_ARG, "qoq_pack_weights: non-finite weight in row %lld", (long long)n);
  return QOQ_OK;
}

extern "C" int qoq_pack_weights_w8(const uint16_t* w_fp16, int64_t N, int64_t K, void* qweight8,
                                   uint16_t* scale_fp16) {
  clear_error();
  if (int st = check_ptrs("qoq_pack_weights_w8", {w_fp16, qweight8, scale_fp16})) return st;
  if (int st = check_weight_shape(N, K, kGroup)) return st;
  const Dims d = dims_of(N, K, kGroup);
  uint8_t* qw = static_cast<uint8_t*>(qweight8);
  std::memset(qw, 0, size_t(d.N_pad) * size_t(K));
  std::memset(scale_fp16, 0, size_t(d.N_pad) * 2);
  std::vector<char> bad(size_t(N), 0);
  parallel_rows(N, [&](int64_t n0, int64_t n1) {
    std::vector<int8_t> q(static_cast<size_t>(K));
    for (int64_t n = n0; n < n1; ++n) {
      if (!encode_row_w8(w_fp16 + size_t(n) * size_t(K), K, q.data(), &scale_fp16[n])) {
        bad[size_t(n)] = 1;
        continue;
      }
      scatter_row_w8(d, n, q.data(), qw);
    }
  });
  for (int64_t n = 0; n < N; ++n)
    if (bad[size_t(n)])
      return fail(QOQ_ERR_INVALID_ARG, "qoq_pack_weights_w8: non-finite weight in row %lld", (long long)n);
  return QOQ_OK;
}

extern "C" int qoq_pack_codes(const uint8_t* q4, const uint8_t* s1, const uint8_t* z, const uint16_t* scale_fp16,
                              int64_t N, int64_t K, int32_t group_size, void* qweight, void* meta,
                              uint16_t* scale_out) {
  clear_error();
  if (int st = check_ptrs("qoq_pack_codes", {q4, z, scale_fp16, qweight, meta, scale_out})) return st;
  if (group_size && !s1) return fail(QOQ_ERR_INVALID_ARG, "qoq_pack_codes: s1 is required for g128");
  qoq_weight_layout L;
  if (int st = qoq_weight_layout_query(N, K, group_size, &L)) return st;
  const Dims d = dims_of(N, K, group_size);
  // validate first so nothing is written on failure
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t g = 0; g < d.G; ++g) {
      const int sc = group_size ? s1[n * d.G + g] : 1;
      const int zz = group_size ? z[n * d.G + g] : z[n];
      if (sc < 1 || sc > 16 || zz > 15)
        return fail(QOQ_ERR_INVALID_ARG, "qoq_pack_codes: s1/z out of range at channel %lld group %lld",
                    (long long)n, (long long)g);
      if (zz * sc > 128)
        return fail(QOQ_ERR_INVALID_ARG, "qoq_pack_codes: z*s1=%d > 128 at channel %lld group %lld", zz * sc,
                    (long long)n, (long long)g);
      const uint8_t* q = q4 + n * K + g * kGroup;
      for (int i = 0; i < kGroup; ++i) {
        const int w8 = (int(q[i]) - zz) * sc;
        if (q[i] > 15 || w8 < -128 || w8 > 127)
          return fail(QOQ_ERR_INVALID_ARG,
                      "qoq_pack_codes: code %d gives w8=%d outside INT8 at channel %lld k %lld", int(q[i]), w8,
                      (long long)n, (long long)(g * kGroup + i));
      }
    }
  }
  uint8_t* qw = static_cast<uint8_t*>(qweight);
  uint8_t* mt = static_cast<uint8_t*>(meta);
  std::memset(qw, 0, L.qweight_bytes);
  std::memset(mt, 0, L.meta_bytes);
  std::memset(scale_out, 0, L.scale_bytes);
  for (int64_t n = 0; n < N; ++n) {
    scale_out[n] = scale_fp16[n];
    if (group_size)
      write_meta_g128(d, n, s1 + n * d.G, z + n * d.G, mt);
    else
      mt[n] = z[n];
    scatter_row(d, n, q4 + n * K, qw);
  }
  return QOQ_OK;
}

extern "C" int qoq_unpack_weights(const void* qweight, const void* meta, const uint16_t* scale_in, int64_t N,
                                  int64_t K, int32_t group_size, uint8_t* q4, uint8_t* s1, uint8_t* z,
                                  uint16_t* scale_fp16) {
  clear_error();
  if (int st = check_ptrs("qoq_unpack_weights", {qweight, meta, scale_in, q4, z, scale_fp16})) return st;
  if (group_size && !s1) return fail(QOQ_ERR_INVALID_ARG, "qoq_unpack_weights: s1 is required for g128");
  if (int st = check_weight_shape(N, K, group_size)) return st;
  const Dims d = dims_of(N, K, group_size);
  const uint8_t* qw = static_cast<const uint8_t*>(qweight);
  const uint8_t* mt = static_cast<const uint8_t*>(meta);
  for (int64_t n = 0; n < N; ++n) {
    scale_fp16[n] = scale_in[n];
    gather_row(d, n, qw, q4 + n * K);
    if (group_size) {
      for (int64_t g = 0; g < d.G; ++g) {
        const uint8_t m = mt[meta_index(d, n, g)];
        s1[n * d.G + g] = uint8_t((m & 15) + 1);
        z[n * d.G + g] = uint8_t(m >> 4);
      }
    } else {
      z[n] = mt[n];
    }
  }
  return QOQ_OK;
}
