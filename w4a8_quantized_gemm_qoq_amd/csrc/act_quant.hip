// Per-token symmetric INT8 activation quantizer for gfx950.
//
// Follows "QServe: W4A8KV4 Quantization and System Co-design for Efficient
// LLM Serving" (paperlayer.ai abs/2405.04532v3 summary): §6 (experimental
// setup) quantizes activations per token to INT8; §5 (runtime and precision
// mapping) feeds INT8 activations to the W4A8 GEMM.  Per row m:
//   s_x = fp16(max_k |x| / 127)      -- FP32 IEEE divide, round half to even
//   x8  = clamp(rint(x / s_x), -127, 127), zero row when s_x == 0.
//
// One 256-thread workgroup per token row.  The row is read once with 128-bit
// loads and kept in registers (up to 16384 channels), the max |x| is reduced
// exactly on the FP16 bit patterns (for non-negative finite halves the integer
// order is the numeric order), then every element is divided by the stored
// FP16 scale -- the correctly rounded FP32 quotient, from one IEEE reciprocal
// per row and two FMAs per element -- and rounded half-even.
// Build without fast-math: the division must stay IEEE.

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <cmath>

#include "qoq_internal.h"

namespace qoq {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t max_abs_bits8(uint4 v) {
  // max over 8 halves of (bits & 0x7fff), computed in two u16 lanes
  const uint32_t a = v.x & 0x7fff7fffu, b = v.y & 0x7fff7fffu;
  const uint32_t c = v.z & 0x7fff7fffu, d = v.w & 0x7fff7fffu;
  auto m2 = [](uint32_t p, uint32_t q) {
    const uint32_t lo = max(p & 0xffffu, q & 0xffffu);
    const uint32_t hi = max(p >> 16, q >> 16);
    return lo | (hi << 16);
  };
  const uint32_t r = m2(m2(a, b), m2(c, d));
  return max(r & 0xffffu, r >> 16);
}

// x / s rounded to nearest even, for an FP16 value x and a positive FP16
// scale s, given y = 1 / s correctly rounded (one IEEE division per row):
// q0 = x * y is within an ulp of x / s, r = x - q0 * s is exact (FMA), and
// q0 + r * y rounded once is the correctly rounded quotient (Markstein's
// theorem).  Checked exhaustively on every finite FP16 x and every positive
// finite FP16 s against the IEEE quotient: identical except for x = -0 (+0
// here), which yields the same integer code.
__device__ __forceinline__ float div_rn(float x, float s, float y) {
  const float q0 = x * y;
  return __builtin_fmaf(__builtin_fmaf(-q0, s, x), y, q0);
}

__device__ __forceinline__ int quant1(uint32_t hbits, float s, float y) {
  const float x = __half2float(__ushort_as_half(static_cast<unsigned short>(hbits)));
  float q = rintf(div_rn(x, s, y));
  q = fminf(127.0f, fmaxf(-127.0f, q));
  return static_cast<int>(q);
}

__device__ __forceinline__ uint32_t quant4(uint32_t h01, uint32_t h23, float s, float y) {
  const int q0 = quant1(h01 & 0xffffu, s, y), q1 = quant1(h01 >> 16, s, y);
  const int q2 = quant1(h23 & 0xffffu, s, y), q3 = quant1(h23 >> 16, s, y);
  return (uint32_t(q0) & 0xffu) | ((uint32_t(q1) & 0xffu) << 8) | ((uint32_t(q2) & 0xffu) << 16) |
         ((uint32_t(q3) & 0xffu) << 24);
}

// Wave-wide reductions of a uint32 (every lane active).  Inside each row of
// 16 lanes four DPP permutations (lane xor 1, lane xor 2, mirror within 8,
// mirror within 16) leave every lane holding its row's result; the four rows
// are then combined from one lane each, so the result is wave-uniform.
// DPP moves are plain VALU operations, far cheaper than cross-lane permutes
// through the LDS crossbar.
constexpr int kDppXor1 = 0xb1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4e;        // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141; // row_half_mirror
constexpr int kDppMirror = 0x140;     // row_mirror
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ uint32_t lane_u32(uint32_t v, int l) {
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), l));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp<kDppXor1>(v));
  v = max(v, dpp<kDppXor2>(v));
  v = max(v, dpp<kDppHalfMirror>(v));
  v = max(v, dpp<kDppMirror>(v));
  return max(max(lane_u32(v, 0), lane_u32(v, 16)), max(lane_u32(v, 32), lane_u32(v, 48)));
}
// Sum; the caller guarantees that the 64 addends sum below 2^32.
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  v += dpp<kDppXor1>(v);
  v += dpp<kDppXor2>(v);
  v += dpp<kDppHalfMirror>(v);
  v += dpp<kDppMirror>(v);
  return (lane_u32(v, 0) + lane_u32(v, 16)) + (lane_u32(v, 32) + lane_u32(v, 48));
}

// Block-wide max of a uint32 value; every thread gets the result.
__device__ __forceinline__ uint32_t block_max(uint32_t v, uint32_t* red) {
  v = wave_max_u32(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  uint32_t r = red[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) r = max(r, red[w]);
  return r;
}

__device__ __forceinline__ float scale_from_absmax(uint32_t amax_bits, unsigned short* s_bits) {
  const float a = __half2float(__ushort_as_half(static_cast<unsigned short>(amax_bits)));
  const __half sh = __float2half_rn(a / 127.0f);
  *s_bits = __half_as_ushort(sh);
  return __half2float(sh);
}

// Vector path, row held in registers: VPT vectors of 8 halves per thread.
template <int VPT>
__global__ __launch_bounds__(kThreads) void act_quant_reg_kernel(const uint4* __restrict__ x, int64_t ldx_vec,
                                                                  int k_vec, uint2* __restrict__ x8,
                                                                  unsigned short* __restrict__ sx) {
  __shared__ uint32_t red[kThreads / 64];
  const int64_t m = blockIdx.x;
  const uint4* row = x + m * ldx_vec;
  uint4 v[VPT];
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int idx = threadIdx.x + i * kThreads;
    v[i] = idx < k_vec ? row[idx] : make_uint4(0, 0, 0, 0);
    amax = max(amax, max_abs_bits8(v[i]));
  }
  amax = block_max(amax, red);
  unsigned short s_bits;
  const float s = scale_from_absmax(amax, &s_bits);
  const float y = s != 0.0f ? 1.0f / s : 0.0f;
  if (threadIdx.x == 0) sx[m] = s_bits;
  uint2* out = x8 + m * k_vec;
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int idx = threadIdx.x + i * kThreads;
    if (idx < k_vec) {
      uint2 q = make_uint2(0u, 0u);
      if (s != 0.0f) q = make_uint2(quant4(v[i].x, v[i].y, s, y), quant4(v[i].z, v[i].w, s, y));
      out[idx] = q;
    }
  }
}

// Vector path for long rows: two passes over the row (the second from cache).
__global__ __launch_bounds__(kThreads) void act_quant_stream_kernel(const uint4* __restrict__ x, int64_t ldx_vec,
                                                                     int k_vec, uint2* __restrict__ x8,
                                                                     unsigned short* __restrict__ sx) {
  __shared__ uint32_t red[kThreads / 64];
  const int64_t m = blockIdx.x;
  const uint4* row = x + m * ldx_vec;
  uint32_t amax = 0;
  for (int idx = threadIdx.x; idx < k_vec; idx += kThreads) amax = max(amax, max_abs_bits8(row[idx]));
  amax = block_max(amax, red);
  unsigned short s_bits;
  const float s = scale_from_absmax(amax, &s_bits);
  const float y = s != 0.0f ? 1.0f / s : 0.0f;
  if (threadIdx.x == 0) sx[m] = s_bits;
  uint2* out = x8 + m * k_vec;
  for (int idx = threadIdx.x; idx < k_vec; idx += kThreads) {
    const uint4 v = row[idx];
    uint2 q = make_uint2(0u, 0u);
    if (s != 0.0f) q = make_uint2(quant4(v.x, v.y, s, y), quant4(v.z, v.w, s, y));
    out[idx] = q;
  }
}

// Scalar path for any K / alignment.
__global__ __launch_bounds__(kThreads) void act_quant_scalar_kernel(const unsigned short* __restrict__ x,
                                                                     int64_t ldx, int64_t K,
                                                                     int8_t* __restrict__ x8,
                                                                     unsigned short* __restrict__ sx) {
  __shared__ uint32_t red[kThreads / 64];
  const int64_t m = blockIdx.x;
  const unsigned short* row = x + m * ldx;
  uint32_t amax = 0;
  for (int64_t k = threadIdx.x; k < K; k += kThreads) amax = max(amax, uint32_t(row[k] & 0x7fffu));
  amax = block_max(amax, red);
  unsigned short s_bits;
  const float s = scale_from_absmax(amax, &s_bits);
  const float y = s != 0.0f ? 1.0f / s : 0.0f;
  if (threadIdx.x == 0) sx[m] = s_bits;
  for (int64_t k = threadIdx.x; k < K; k += kThreads)
    x8[m * K + k] = s != 0.0f ? static_cast<int8_t>(quant1(row[k], s, y)) : int8_t(0);
}

// ---------------------------------------------------------------------------
// Fused producer: RMS normalization of each token row, then the per-token
// quantization above ("QServe: W4A8KV4 Quantization and System Co-design for
// Efficient LLM Serving", paperlayer.ai summary, §5 runtime and precision
// mapping: the quantizer runs inside the normalization kernel that produces
// the activations).  Per row:
//   S   = sum_k x_k^2, exactly: an FP16 value is an integer times 2^-24, so
//         its square is an integer times 2^-48 below 2^80, and a 128-bit
//         integer holds the sum of any row;
//   ms  = fp32(fp64(S) * 2^-48 / K),  r = 1 / sqrtf(ms + eps),
//   h_k = fp16((x_k * r) * gamma_k), then s_x and x8 from h as above.
// Every rounding is one IEEE operation on a value that does not depend on the
// order of the reduction, so the result is the same for every launch shape.

typedef unsigned __int128 u128;

// Exact sum of squares of one thread's FP16 values, in units of 2^-48.  A
// square is mant^2 * 2^sh with mant^2 < 2^22 and sh = 2e - 2 in [0, 58] (e
// the biased exponent, 1 for subnormals).  Squares with sh < 32 are added
// into `lo`, the others (in units of 2^32) into `hi`: each addend is below
// 2^54, so 64 of them fit 64-bit sums without carry; flush() moves the pair
// into the 128-bit total before that bound is reached.
struct SumSq {
  uint64_t lo = 0, hi = 0;
  u128 total = 0;
  __device__ __forceinline__ void add(uint32_t hbits) {
    const uint32_t e = (hbits >> 10) & 31u;
    const uint32_t mant = e ? ((hbits & 0x3ffu) | 0x400u) : (hbits & 0x3ffu);
    const uint32_t sh = e ? 2u * e - 2u : 0u;
    const bool big = sh >= 32u;
    const uint64_t v = uint64_t(mant * mant) << (big ? sh - 32u : sh);
    lo += big ? 0 : v;
    hi += big ? v : 0;
  }
  __device__ __forceinline__ void add8(uint4 q) {
    add(q.x & 0xffffu); add(q.x >> 16); add(q.y & 0xffffu); add(q.y >> 16);
    add(q.z & 0xffffu); add(q.z >> 16); add(q.w & 0xffffu); add(q.w >> 16);
  }
  __device__ __forceinline__ void flush() {
    total += (u128(hi) << 32) + u128(lo);
    lo = hi = 0;
  }
};

// Block-wide sum of a 128-bit integer below 2^96 (a thread's sum of squares
// holds at most K / 256 <= 2^10 squares below 2^80 each); every thread gets
// the result.  The value is cut into four 24-bit limbs: 256 limbs sum below
// 2^32, so each limb is reduced exactly in 32-bit lanes and the limbs are
// recombined in 128-bit arithmetic at the end.
__device__ __forceinline__ u128 block_sum_u128(u128 v, uint32_t (*red)[4]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t s[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) s[k] = wave_sum_u32(static_cast<uint32_t>(v >> (24 * k)) & 0xffffffu);
  if (lane == 0) {
#pragma unroll
    for (int k = 0; k < 4; ++k) red[wave][k] = s[k];
  }
  __syncthreads();
  u128 r = 0;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w)
#pragma unroll
    for (int k = 0; k < 4; ++k) r += u128(red[w][k]) << (24 * k);
  return r;
}

// Round-to-nearest-even conversion of a 128-bit integer to FP64: the top 64
// bits, with every bit below them folded into bit 0 as a sticky bit (the
// rounding position of a 64-bit value with its top bit set is bit 10).
__device__ __forceinline__ double u128_to_double_rn(u128 v) {
  const unsigned long long hi = static_cast<unsigned long long>(v >> 64);
  if (hi == 0) return static_cast<double>(static_cast<unsigned long long>(v));
  const int n = 64 - __clzll(static_cast<long long>(hi));  // 1..64
  const unsigned long long top =
      static_cast<unsigned long long>(v >> n) | static_cast<unsigned long long>((v << (128 - n)) != 0);
  return ldexp(static_cast<double>(top), n);
}

__device__ __forceinline__ float mean_square(u128 S, int64_t K) {
  return static_cast<float>(ldexp(u128_to_double_rn(S), -48) / static_cast<double>(K));
}
__device__ __forceinline__ float rms_factor(float ms, float eps) { return 1.0f / sqrtf(ms + eps); }

// Fast path for the mean square.  The square of an FP16 value is exact in
// FP32 (at most 22 significant bits, between 2^-48 and 2^32), so summing the
// squares in FP64 rounds only at the additions: with non-negative addends, a
// sum reached through at most n additions along any path is within n * 2^-53
// (relative) of the exact S.  A thread adds at most 64 squares and the block
// reduction adds 8 levels, so S' is within 2^-46 of S.  Every step from S to
// ms (FP64 rounding, division by K, FP32 rounding) is monotone, so when the
// ends of [S'(1 - 2^-44), S'(1 + 2^-44)] give the same FP32 value, so does S
// and that value is the exact path's result; otherwise (a row whose mean
// square lies within about 2^-44 of an FP32 rounding boundary) the caller
// takes the exact 128-bit sum.
__device__ __forceinline__ double sumsq8_f64(uint4 q, double acc) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = __half2float(__ushort_as_half(static_cast<unsigned short>(w[i] & 0xffffu)));
    const float b = __half2float(__ushort_as_half(static_cast<unsigned short>(w[i] >> 16)));
    acc += static_cast<double>(a * a);
    acc += static_cast<double>(b * b);
  }
  return acc;
}

// Block-wide FP64 sum (every thread gets the same value).
__device__ __forceinline__ double block_sum_f64(double v, double* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  double r = red[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) r += red[w];
  return r;
}

// The mean square from the FP64 sum when it is certain to equal the exact
// path's value; NaN otherwise.
__device__ __forceinline__ float mean_square_fast(double s, int64_t K) {
  const double k = static_cast<double>(K);
  const float lo = static_cast<float>(s * (1.0 - 0x1p-44) / k);
  const float hi = static_cast<float>(s * (1.0 + 0x1p-44) / k);
  return lo == hi ? lo : __builtin_nanf("");
}

__device__ __forceinline__ uint32_t norm1(uint32_t xbits, uint32_t gbits, float r) {
  const float x = __half2float(__ushort_as_half(static_cast<unsigned short>(xbits)));
  const float g = __half2float(__ushort_as_half(static_cast<unsigned short>(gbits)));
  return __half_as_ushort(__float2half_rn((x * r) * g));
}
__device__ __forceinline__ uint32_t norm2(uint32_t x2, uint32_t g2, float r) {
  return norm1(x2 & 0xffffu, g2 & 0xffffu, r) | (norm1(x2 >> 16, g2 >> 16, r) << 16);
}
__device__ __forceinline__ uint4 norm8(uint4 x, uint4 g, float r) {
  return make_uint4(norm2(x.x, g.x, r), norm2(x.y, g.y, r), norm2(x.z, g.z, r), norm2(x.w, g.w, r));
}

// Vector path, row held in registers: VPT vectors of 8 halves per thread.
template <int VPT>
__global__ __launch_bounds__(kThreads) void rmsnorm_quant_reg_kernel(const uint4* __restrict__ x, int64_t ldx_vec,
                                                                      int k_vec, const uint4* __restrict__ gamma,
                                                                      float eps, uint2* __restrict__ x8,
                                                                      unsigned short* __restrict__ sx) {
  __shared__ uint32_t red_sum[kThreads / 64][4];
  __shared__ double red_f64[kThreads / 64];
  __shared__ uint32_t red[kThreads / 64];
  const int64_t m = blockIdx.x;
  const uint4* row = x + m * ldx_vec;
  static_assert(VPT * 8 <= 64, "one flush per row, at most 64 FP64 additions per thread");
  // gamma is fetched together with the row, so that its latency overlaps the
  // row's and the sum of squares instead of following the reduction
  uint4 v[VPT], gv[VPT];
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int idx = threadIdx.x + i * kThreads;
    v[i] = idx < k_vec ? row[idx] : make_uint4(0, 0, 0, 0);
    gv[i] = idx < k_vec ? gamma[idx] : make_uint4(0, 0, 0, 0);
  }
  double s2 = 0.0;
#pragma unroll
  for (int i = 0; i < VPT; ++i) s2 = sumsq8_f64(v[i], s2);
  float ms = mean_square_fast(block_sum_f64(s2, red_f64), int64_t(k_vec) * 8);
  if (ms != ms) {  // block-uniform: every thread holds the same sum
    SumSq S;
#pragma unroll
    for (int i = 0; i < VPT; ++i) S.add8(v[i]);
    S.flush();
    ms = mean_square(block_sum_u128(S.total, red_sum), int64_t(k_vec) * 8);
  }
  const float r = rms_factor(ms, eps);
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int idx = threadIdx.x + i * kThreads;
    if (idx < k_vec) {
      v[i] = norm8(v[i], gv[i], r);
      amax = max(amax, max_abs_bits8(v[i]));
    }
  }
  amax = block_max(amax, red);
  unsigned short s_bits;
  const float s = scale_from_absmax(amax, &s_bits);
  const float y = s != 0.0f ? 1.0f / s : 0.0f;
  if (threadIdx.x == 0) sx[m] = s_bits;
  uint2* out = x8 + m * k_vec;
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int idx = threadIdx.x + i * kThreads;
    if (idx < k_vec) {
      uint2 q = make_uint2(0u, 0u);
      if (s != 0.0f) q = make_uint2(quant4(v[i].x, v[i].y, s, y), quant4(v[i].z, v[i].w, s, y));
      out[idx] = q;
    }
  }
}

// Vector path for long rows: three passes over the row (the later ones from
// cache); the normalized values are recomputed, not stored.
__global__ __launch_bounds__(kThreads) void rmsnorm_quant_stream_kernel(const uint4* __restrict__ x, int64_t ldx_vec,
                                                                         int k_vec, const uint4* __restrict__ gamma,
                                                                         float eps, uint2* __restrict__ x8,
                                                                         unsigned short* __restrict__ sx) {
  __shared__ uint32_t red_sum[kThreads / 64][4];
  __shared__ uint32_t red[kThreads / 64];
  const int64_t m = blockIdx.x;
  const uint4* row = x + m * ldx_vec;
  SumSq S;
  int n = 0;
  for (int idx = threadIdx.x; idx < k_vec; idx += kThreads) {
    S.add8(row[idx]);
    if (++n == 8) {  // 64 squares
      S.flush();
      n = 0;
    }
  }
  S.flush();
  const float r = rms_factor(mean_square(block_sum_u128(S.total, red_sum), int64_t(k_vec) * 8), eps);
  uint32_t amax = 0;
  for (int idx = threadIdx.x; idx < k_vec; idx += kThreads)
    amax = max(amax, max_abs_bits8(norm8(row[idx], gamma[idx], r)));
  amax = block_max(amax, red);
  unsigned short s_bits;
  const float s = scale_from_absmax(amax, &s_bits);
  const float y = s != 0.0f ? 1.0f / s : 0.0f;
  if (threadIdx.x == 0) sx[m] = s_bits;
  uint2* out = x8 + m * k_vec;
  for (int idx = threadIdx.x; idx < k_vec; idx += kThreads) {
    const uint4 h = norm8(row[idx], gamma[idx], r);
    uint2 q = make_uint2(0u, 0u);
    if (s != 0.0f) q = make_uint2(quant4(h.x, h.y, s, y), quant4(h.z, h.w, s, y));
    out[idx] = q;
  }
}

// Scalar path for any K / alignment.
__global__ __launch_bounds__(kThreads) void rmsnorm_quant_scalar_kernel(const unsigned short* __restrict__ x,
                                                                         int64_t ldx, int64_t K,
                                                                         const unsigned short* __restrict__ gamma,
                                                                         float eps, int8_t* __restrict__ x8,
                                                                         unsigned short* __restrict__ sx) {
  __shared__ uint32_t red_sum[kThreads / 64][4];
  __shared__ uint32_t red[kThreads / 64];
  const int64_t m = blockIdx.x;
  const unsigned short* row = x + m * ldx;
  SumSq S;
  int n = 0;
  for (int64_t k = threadIdx.x; k < K; k += kThreads) {
    S.add(row[k]);
    if (++n == 64) {
      S.flush();
      n = 0;
    }
  }
  S.flush();
  const float r = rms_factor(mean_square(block_sum_u128(S.total, red_sum), K), eps);
  uint32_t amax = 0;
  for (int64_t k = threadIdx.x; k < K; k += kThreads) amax = max(amax, norm1(row[k], gamma[k], r) & 0x7fffu);
  amax = block_max(amax, red);
  unsigned short s_bits;
  const float s = scale_from_absmax(amax, &s_bits);
  const float y = s != 0.0f ? 1.0f / s : 0.0f;
  if (threadIdx.x == 0) sx[m] = s_bits;
  for (int64_t k = threadIdx.x; k < K; k += kThreads)
    x8[m * K + k] = s != 0.0f ? static_cast<int8_t>(quant1(norm1(row[k], gamma[k], r), s, y)) : int8_t(0);
}

// ---------------------------------------------------------------------------
// Fused producer of the down projection's input: h = SiLU(gate) * up, then the
// per-token quantization above ("QServe: W4A8KV4 Quantization and System
// Co-design for Efficient LLM Serving", paperlayer.ai summary, §5 runtime and
// precision mapping: the quantizer also runs inside the activation-function
// kernel that produces a layer's input).  Per element, each step rounded once:
//   s = fp16(g / (1 + e^-g))   the correctly rounded FP16 SiLU
//   h = fp16(s * u)            the product of two halves is exact in FP32
// then s_x and x8 from the row of h as for the plain quantizer.  Inputs must
// be finite and their products must not overflow FP16.

// FP16 SiLU, correctly rounded.  Evaluated in FP32 (e^-g by the library's
// expf, one hardware reciprocal): over every finite FP16 input whose SiLU is
// at least the smallest FP16 subnormal, that value lies within 2.5 FP32 ulps
// of the exact SiLU.  Where it lies within 4 FP32 ulps of an FP16 rounding
// boundary -- for normal FP16 results, its 13 bits below the FP16 precision
// within 4 of one half (0.1% of inputs); for subnormal ones, within 4 of its
// ulps of an odd multiple of 2^-25 -- the side of the boundary is decided from
// an FP64 evaluation instead, far more accurate than the 4.8e-12 (relative)
// that separates every finite FP16 input's exact SiLU from the nearest
// boundary.  The GPU tests check the result on every finite FP16 input.
// silu(g) has the sign of g.
__device__ __forceinline__ float half_bits_to_float(uint32_t b) {
  return __half2float(__ushort_as_half(static_cast<unsigned short>(b)));
}
constexpr uint32_t kSiluWindow = 4;  // FP32 ulps
__device__ __forceinline__ uint32_t silu_half(uint32_t gbits) {
  const float g = half_bits_to_float(gbits);
  const float a = fabsf(g * __builtin_amdgcn_rcpf(1.0f + expf(-g)));
  const uint32_t ab = __float_as_uint(a);
  const uint32_t c = __half_as_ushort(__float2half_rn(a));  // |s| candidate (RNE)
  bool near;
  if (ab >= 0x38800000u) {  // a normal FP16 result
    near = (ab & 0x1fffu) - (0x1000u - kSiluWindow) <= 2u * kSiluWindow;
  } else {
    // FP16 subnormals are multiples of 2^-24: the distance of a * 2^24 (exact)
    // to the nearest half-integer, against the FP32 ulps of a * 2^24
    const float r = a * 0x1p24f;
    const float d = fabsf(r - (floorf(r) + 0.5f));
    const float u = __uint_as_float((__float_as_uint(r) & 0x7f800000u) | 1u) - __uint_as_float(__float_as_uint(r) & 0x7f800000u);
    near = r >= 0x1p-30f && !(d > static_cast<float>(kSiluWindow) * u);
  }
  uint32_t r = c;
  if (near) {
    // midpoints to the neighbouring halves (exact in FP32), against FP64
    const float fc = half_bits_to_float(c);
    const float lo = c > 0 ? 0.5f * (fc + half_bits_to_float(c - 1)) : -1.0f;
    const float hi = c < 0x7bffu ? 0.5f * (fc + half_bits_to_float(c + 1)) : INFINITY;
    const double gd = static_cast<double>(g);
    const double ad = fabs(gd / (1.0 + exp(-gd)));
    r = ad > static_cast<double>(hi) ? c + 1 : (ad < static_cast<double>(lo) ? c - 1 : c);
  }
  return r | (gbits & 0x8000u);
}
__device__ __forceinline__ uint32_t swiglu1(uint32_t gbits, uint32_t ubits) {
  const float sv = half_bits_to_float(silu_half(gbits));
  return __half_as_ushort(__float2half_rn(sv * half_bits_to_float(ubits)));
}
__device__ __forceinline__ uint32_t swiglu2(uint32_t g2, uint32_t u2) {
  return swiglu1(g2 & 0xffffu, u2 & 0xffffu) | (swiglu1(g2 >> 16, u2 >> 16) << 16);
}
__device__ __forceinline__ uint4 swiglu8(uint4 g, uint4 u) {
  return make_uint4(swiglu2(g.x, u.x), swiglu2(g.y, u.y), swiglu2(g.z, u.z), swiglu2(g.w, u.w));
}

// Vector path: the row of h is computed once, in a loop of 8-element vectors
// (the SiLU with its rare FP64 branch is too long to unroll over a whole
// row), and kept in LDS until the scale is known.  h (optional) receives the
// FP16 activations.  Dynamic LDS: 16 bytes per vector of the row.
constexpr int kSwigluLdsMaxVec = 4000;  // 62.5 KB (within the 64 KB default): rows up to 32000 channels
__global__ __launch_bounds__(kThreads) void swiglu_quant_lds_kernel(const uint4* __restrict__ gate, int64_t ldg_vec,
                                                                     const uint4* __restrict__ up, int64_t ldu_vec,
                                                                     int k_vec, uint2* __restrict__ x8,
                                                                     unsigned short* __restrict__ sx,
                                                                     uint4* __restrict__ h, int64_t ldh_vec) {
  extern __shared__ uint4 hrow[];
  __shared__ uint32_t red[kThreads / 64];
  const int64_t m = blockIdx.x;
  uint32_t amax = 0;
  for (int idx = threadIdx.x; idx < k_vec; idx += kThreads) {
    const uint4 v = swiglu8(gate[m * ldg_vec + idx], up[m * ldu_vec + idx]);
    hrow[idx] = v;
    amax = max(amax, max_abs_bits8(v));
    if (h) h[m * ldh_vec + idx] = v;
  }
  amax = block_max(amax, red);  // each thread rereads only the entries it wrote
  unsigned short s_bits;
  const float s = scale_from_absmax(amax, &s_bits);
  const float y = s != 0.0f ? 1.0f / s : 0.0f;
  if (threadIdx.x == 0) sx[m] = s_bits;
  uint2* out = x8 + m * k_vec;
  for (int idx = threadIdx.x; idx < k_vec; idx += kThreads) {
    const uint4 v = hrow[idx];
    uint2 q = make_uint2(0u, 0u);
    if (s != 0.0f) q = make_uint2(quant4(v.x, v.y, s, y), quant4(v.z, v.w, s, y));
    out[idx] = q;
  }
}

// Vector path for long rows: two passes, the second recomputing h from the
// inputs (read again, from cache).
__global__ __launch_bounds__(kThreads) void swiglu_quant_stream_kernel(const uint4* __restrict__ gate, int64_t ldg_vec,
                                                                        const uint4* __restrict__ up, int64_t ldu_vec,
                                                                        int k_vec, uint2* __restrict__ x8,
                                                                        unsigned short* __restrict__ sx,
                                                                        uint4* __restrict__ h, int64_t ldh_vec) {
  __shared__ uint32_t red[kThreads / 64];
  const int64_t m = blockIdx.x;
  uint32_t amax = 0;
  for (int idx = threadIdx.x; idx < k_vec; idx += kThreads)
    amax = max(amax, max_abs_bits8(swiglu8(gate[m * ldg_vec + idx], up[m * ldu_vec + idx])));
  amax = block_max(amax, red);
  unsigned short s_bits;
  const float s = scale_from_absmax(amax, &s_bits);
  const float y = s != 0.0f ? 1.0f / s : 0.0f;
  if (threadIdx.x == 0) sx[m] = s_bits;
  uint2* out = x8 + m * k_vec;
  for (int idx = threadIdx.x; idx < k_vec; idx += kThreads) {
    const uint4 v = swiglu8(gate[m * ldg_vec + idx], up[m * ldu_vec + idx]);
    uint2 q = make_uint2(0u, 0u);
    if (s != 0.0f) q = make_uint2(quant4(v.x, v.y, s, y), quant4(v.z, v.w, s, y));
    out[idx] = q;
    if (h) h[m * ldh_vec + idx] = v;
  }
}

// Scalar path for any K / alignment.
__global__ __launch_bounds__(kThreads) void swiglu_quant_scalar_kernel(const unsigned short* __restrict__ gate,
                                                                        int64_t ldg,
                                                                        const unsigned short* __restrict__ up,
                                                                        int64_t ldu, int64_t K,
                                                                        int8_t* __restrict__ x8,
                                                                        unsigned short* __restrict__ sx,
                                                                        unsigned short* __restrict__ h, int64_t ldh) {
  __shared__ uint32_t red[kThreads / 64];
  const int64_t m = blockIdx.x;
  uint32_t amax = 0;
  for (int64_t k = threadIdx.x; k < K; k += kThreads)
    amax = max(amax, swiglu1(gate[m * ldg + k], up[m * ldu + k]) & 0x7fffu);
  amax = block_max(amax, red);
  unsigned short s_bits;
  const float s = scale_from_absmax(amax, &s_bits);
  const float y = s != 0.0f ? 1.0f / s : 0.0f;
  if (threadIdx.x == 0) sx[m] = s_bits;
  for (int64_t k = threadIdx.x; k < K; k += kThreads) {
    const uint32_t v = swiglu1(gate[m * ldg + k], up[m * ldu + k]);
    x8[m * K + k] = s != 0.0f ? static_cast<int8_t>(quant1(v, s, y)) : int8_t(0);
    if (h) h[m * ldh + k] = static_cast<unsigned short>(v);
  }
}

}  // namespace
}  // namespace qoq

using namespace qoq;

extern "C" int qoq_rmsnorm_quant_per_token(const void* x_fp16, const void* gamma_fp16, float eps, int64_t M,
                                           int64_t K, int64_t ldx, int8_t* x8, void* sx_fp16, void* stream) {
  clear_error();
  if (!x_fp16 || !gamma_fp16 || !x8 || !sx_fp16)
    return fail(QOQ_ERR_INVALID_ARG, "qoq_rmsnorm_quant_per_token: null pointer argument");
  if (!(eps > 0.0f) || !(eps < INFINITY))
    return fail(QOQ_ERR_INVALID_ARG, "qoq_rmsnorm_quant_per_token: eps must be positive and finite");
  if (M < 1 || K < 1) return fail(QOQ_ERR_UNSUPPORTED_SHAPE, "qoq_rmsnorm_quant_per_token: M and K must be >= 1");
  if (ldx < K) return fail(QOQ_ERR_INVALID_ARG, "qoq_rmsnorm_quant_per_token: ldx < K");
  if (M > 0x7fffffff || K > 0x7fffffff)
    return fail(QOQ_ERR_UNSUPPORTED_SHAPE, "qoq_rmsnorm_quant_per_token: M or K too large");
  const auto al = [](const void* p, uintptr_t n) { return reinterpret_cast<uintptr_t>(p) % n == 0; };
  if (!al(x_fp16, 2) || !al(gamma_fp16, 2) || !al(sx_fp16, 2))
    return fail(QOQ_ERR_ALIGNMENT, "qoq_rmsnorm_quant_per_token: FP16 pointers must be 2-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid(static_cast<unsigned>(M)), block(kThreads);
  const bool vec = K % 8 == 0 && ldx % 8 == 0 && al(x_fp16, 16) && al(gamma_fp16, 16) && al(x8, 8);
  auto* sx = static_cast<unsigned short*>(sx_fp16);
  if (vec) {
    const auto* xv = static_cast<const uint4*>(x_fp16);
    const auto* gv = static_cast<const uint4*>(gamma_fp16);
    auto* qv = reinterpret_cast<uint2*>(x8);
    const int k_vec = static_cast<int>(K / 8);
    const int64_t ldv = ldx / 8;
    if (k_vec <= kThreads)
      hipLaunchKernelGGL(rmsnorm_quant_reg_kernel<1>, grid, block, 0, st, xv, ldv, k_vec, gv, eps, qv, sx);
    else if (k_vec <= 2 * kThreads)
      hipLaunchKernelGGL(rmsnorm_quant_reg_kernel<2>, grid, block, 0, st, xv, ldv, k_vec, gv, eps, qv, sx);
    else if (k_vec <= 4 * kThreads)
      hipLaunchKernelGGL(rmsnorm_quant_reg_kernel<4>, grid, block, 0, st, xv, ldv, k_vec, gv, eps, qv, sx);
    else if (k_vec <= 8 * kThreads)
      hipLaunchKernelGGL(rmsnorm_quant_reg_kernel<8>, grid, block, 0, st, xv, ldv, k_vec, gv, eps, qv, sx);
    else
      hipLaunchKernelGGL(rmsnorm_quant_stream_kernel, grid, block, 0, st, xv, ldv, k_vec, gv, eps, qv, sx);
  } else {
    hipLaunchKernelGGL(rmsnorm_quant_scalar_kernel, grid, block, 0, st, static_cast<const unsigned short*>(x_fp16),
                       ldx, K, static_cast<const unsigned short*>(gamma_fp16), eps, x8, sx);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(QOQ_ERR_HIP, "qoq_rmsnorm_quant_per_token: launch failed: %s", hipGetErrorString(e));
  return QOQ_OK;
}

extern "C" int qoq_quant_act_per_token(const void* x_fp16, int64_t M, int64_t K, int64_t ldx, int8_t* x8,
                                       void* sx_fp16, void* stream) {
  clear_error();
  if (!x_fp16 || !x8 || !sx_fp16) return fail(QOQ_ERR_INVALID_ARG, "qoq_quant_act_per_token: null pointer argument");
  if (M < 1 || K < 1) return fail(QOQ_ERR_UNSUPPORTED_SHAPE, "qoq_quant_act_per_token: M and K must be >= 1");
  if (ldx < K) return fail(QOQ_ERR_INVALID_ARG, "qoq_quant_act_per_token: ldx < K");
  if (M > 0x7fffffff) return fail(QOQ_ERR_UNSUPPORTED_SHAPE, "qoq_quant_act_per_token: M too large");
  if (reinterpret_cast<uintptr_t>(x_fp16) % 2 || reinterpret_cast<uintptr_t>(sx_fp16) % 2)
    return fail(QOQ_ERR_ALIGNMENT, "qoq_quant_act_per_token: FP16 pointers must be 2-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid(static_cast<unsigned>(M)), block(kThreads);
  const bool vec = K % 8 == 0 && ldx % 8 == 0 && reinterpret_cast<uintptr_t>(x_fp16) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(x8) % 8 == 0 && K / 8 <= 0x7fffffff;
  auto* sx = static_cast<unsigned short*>(sx_fp16);
  if (vec) {
    const auto* xv = static_cast<const uint4*>(x_fp16);
    auto* qv = reinterpret_cast<uint2*>(x8);
    const int k_vec = static_cast<int>(K / 8);
    const int64_t ldv = ldx / 8;
    if (k_vec <= kThreads)
      hipLaunchKernelGGL(act_quant_reg_kernel<1>, grid, block, 0, st, xv, ldv, k_vec, qv, sx);
    else if (k_vec <= 2 * kThreads)
      hipLaunchKernelGGL(act_quant_reg_kernel<2>, grid, block, 0, st, xv, ldv, k_vec, qv, sx);
    else if (k_vec <= 4 * kThreads)
      hipLaunchKernelGGL(act_quant_reg_kernel<4>, grid, block, 0, st, xv, ldv, k_vec, qv, sx);
    else if (k_vec <= 8 * kThreads)
      hipLaunchKernelGGL(act_quant_reg_kernel<8>, grid, block, 0, st, xv, ldv, k_vec, qv, sx);
    else
      hipLaunchKernelGGL(act_quant_stream_kernel, grid, block, 0, st, xv, ldv, k_vec, qv, sx);
  } else {
    hipLaunchKernelGGL(act_quant_scalar_kernel, grid, block, 0, st, static_cast<const unsigned short*>(x_fp16), ldx,
                       K, x8, sx);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(QOQ_ERR_HIP, "qoq_quant_act_per_token: launch failed: %s", hipGetErrorString(e));
  return QOQ_OK;
}

extern "C" int qoq_swiglu_quant_per_token(const void* gate_fp16, const void* up_fp16, int64_t M, int64_t K,
                                          int64_t ldg, int64_t ldu, int8_t* x8, void* sx_fp16, void* h_fp16,
                                          int64_t ldh, void* stream) {
  clear_error();
  if (!gate_fp16 || !up_fp16 || !x8 || !sx_fp16)
    return fail(QOQ_ERR_INVALID_ARG, "qoq_swiglu_quant_per_token: null pointer argument");
  if (M < 1 || K < 1) return fail(QOQ_ERR_UNSUPPORTED_SHAPE, "qoq_swiglu_quant_per_token: M and K must be >= 1");
  if (ldg < K || ldu < K || (h_fp16 && ldh < K))
    return fail(QOQ_ERR_INVALID_ARG, "qoq_swiglu_quant_per_token: a leading dimension is below K");
  if (M > 0x7fffffff || K > 0x7fffffff)
    return fail(QOQ_ERR_UNSUPPORTED_SHAPE, "qoq_swiglu_quant_per_token: M or K too large");
  const auto al = [](const void* p, uintptr_t n) { return reinterpret_cast<uintptr_t>(p) % n == 0; };
  if (!al(gate_fp16, 2) || !al(up_fp16, 2) || !al(sx_fp16, 2) || (h_fp16 && !al(h_fp16, 2)))
    return fail(QOQ_ERR_ALIGNMENT, "qoq_swiglu_quant_per_token: FP16 pointers must be 2-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid(static_cast<unsigned>(M)), block(kThreads);
  const bool vec = K % 8 == 0 && ldg % 8 == 0 && ldu % 8 == 0 && al(gate_fp16, 16) && al(up_fp16, 16) &&
                   al(x8, 8) && (!h_fp16 || (ldh % 8 == 0 && al(h_fp16, 16)));
  auto* sx = static_cast<unsigned short*>(sx_fp16);
  if (vec) {
    const auto* gv = static_cast<const uint4*>(gate_fp16);
    const auto* uv = static_cast<const uint4*>(up_fp16);
    auto* qv = reinterpret_cast<uint2*>(x8);
    auto* hv = static_cast<uint4*>(h_fp16);
    const int k_vec = static_cast<int>(K / 8);
    const int64_t lg = ldg / 8, lu = ldu / 8, lh = h_fp16 ? ldh / 8 : 0;
    if (k_vec <= kSwigluLdsMaxVec) {
      const size_t lds = size_t(k_vec) * sizeof(uint4);
      hipLaunchKernelGGL(swiglu_quant_lds_kernel, grid, block, lds, st, gv, lg, uv, lu, k_vec, qv, sx, hv, lh);
    } else {
      hipLaunchKernelGGL(swiglu_quant_stream_kernel, grid, block, 0, st, gv, lg, uv, lu, k_vec, qv, sx, hv, lh);
    }
  } else {
    hipLaunchKernelGGL(swiglu_quant_scalar_kernel, grid, block, 0, st, static_cast<const unsigned short*>(gate_fp16),
                       ldg, static_cast<const unsigned short*>(up_fp16), ldu, K, x8, sx,
                       static_cast<unsigned short*>(h_fp16), ldh);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(QOQ_ERR_HIP, "qoq_swiglu_quant_per_token: launch failed: %s", hipGetErrorString(e));
  return QOQ_OK;
}
