// KV4: per-head dynamic asymmetric INT4 quantization of the KV cache and the
// decode attention that reads it, for gfx950.
//
// Follows "QServe: W4A8KV4 Quantization and System Co-design for Efficient
// LLM Serving" (paperlayer.ai abs/2405.04532v3 summary): §6 (experimental
// setup) keeps the KV cache as per-head asymmetric INT4; §5 (KV4 attention)
// computes the per-head scaling factors and zero points at run time and runs
// the attention in floating point on the vector units, as a memory-bound
// kernel; §4 (SmoothAttention) leaves the queries unquantized; §3 (roofline)
// motivates KV4 by its halved memory traffic against KV8.
//
// Cache layout (head_dim 128): codes [rows][64 bytes], byte j = code of dim
// 2j | code of dim 2j+1 << 4; scale FP16 [rows]; zero UINT4 in a byte [rows].
// For attention the rows are ordered [B][Hkv][T_max] (a head's tokens are
// consecutive).
//
// Quantization of one row x (128 FP16 values), exactly the per-channel W4 map:
//   s = fp16((max - min) / 15)  (FP32 subtract and divide, RNE),
//   z = clamp(rint(-min / s), 0, 15),  q = clamp(rint(x / s) + z, 0, 15);
//   s == 0 gives z = 0 and zero codes.
//
// Decode attention of one query head h of sequence b (kv head g = h/(H/Hkv),
// L = lengths[b] tokens): score_t = scale * <q, (c_t - z_t) s_t>, evaluated as
// s_t * (<q', c_t> - z_t * sum(q')) with q' = scale * q in FP32; then
// softmax and o = sum_t a_t v_t in FP32, written as FP16.  The scores of a
// head are kept in LDS (T_max <= 32768).  One 256-thread block per (b, h):
// four lanes share a token (32 dims, one 16-byte load each), so a wave reads
// 16 consecutive tokens = 1 KB per load instruction.

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <algorithm>
#include <cmath>

#include "qoq_internal.h"

namespace qoq {
namespace {

constexpr int kHeadDim = 128;
constexpr int kRowBytes = kHeadDim / 2;
constexpr int kAttnThreads = 256;
constexpr int kMaxCacheLen = 32768;
typedef int i32x4 __attribute__((ext_vector_type(4)));

// DPP lane permutations (VALU operations, no trip through the LDS crossbar):
// row_ror:4 / row_ror:8 rotate each row of 16 lanes, keeping lane % 4.
template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
constexpr int kDppRor4 = 0x124;
constexpr int kDppRor8 = 0x128;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// 16 lanes per row (8 values each, one 16-byte load), 16 rows per block.
constexpr int kQuantRowsPerBlock = 16;

__device__ __forceinline__ float half_lo(unsigned w) {
  return __half2float(__ushort_as_half(static_cast<unsigned short>(w & 0xffffu)));
}
__device__ __forceinline__ float half_hi(unsigned w) {
  return __half2float(__ushort_as_half(static_cast<unsigned short>(w >> 16)));
}
// max / min over the 16 lanes of a row group
__device__ __forceinline__ float group16_max(float v) {
#pragma unroll
  for (int off = 8; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}
__device__ __forceinline__ float group16_min(float v) {
#pragma unroll
  for (int off = 8; off > 0; off >>= 1) v = fminf(v, __shfl_xor(v, off, 64));
  return v;
}

__global__ __launch_bounds__(256) void kv4_quant_kernel(const uint4* __restrict__ x, int64_t ldx_vec,
                                                        int64_t n_rows, unsigned* __restrict__ codes,
                                                        unsigned short* __restrict__ scale,
                                                        uint8_t* __restrict__ zero) {
  const int sub = threadIdx.x & 15;  // which 8 dims of the row
  const int64_t row = int64_t(blockIdx.x) * kQuantRowsPerBlock + (threadIdx.x >> 4);
  // rows past the end read the last row; their results are not stored
  const uint4 u = x[min(row, n_rows - 1) * ldx_vec + sub];
  float v[8] = {half_lo(u.x), half_hi(u.x), half_lo(u.y), half_hi(u.y),
                half_lo(u.z), half_hi(u.z), half_lo(u.w), half_hi(u.w)};
  float hi = v[0], lo = v[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) {
    hi = fmaxf(hi, v[i]);
    lo = fminf(lo, v[i]);
  }
  hi = group16_max(hi);
  lo = group16_min(lo);
  const __half sh = __float2half_rn((hi - lo) / 15.0f);
  const float s = __half2float(sh);
  unsigned q = 0, zz = 0;
  if (s != 0.0f) {
    // correctly rounded quotients from one reciprocal (Markstein): q0 = x*y,
    // x/s = fma(fma(-q0, s, x), y, q0); exact for FP16 x and FP16 s
    const float y = 1.0f / s;
    auto div_rn = [&](float x) {
      const float q0 = x * y;
      return __builtin_fmaf(__builtin_fmaf(-q0, s, x), y, q0);
    };
    const float z = fminf(15.0f, fmaxf(0.0f, rintf(div_rn(-lo))));
#pragma unroll
    for (int i = 0; i < 8; ++i) q |= unsigned(fminf(15.0f, fmaxf(0.0f, rintf(div_rn(v[i])) + z))) << (4 * i);
    zz = unsigned(z);
  }
  if (row < n_rows) {
    codes[row * (kRowBytes / 4) + sub] = q;
    if (sub == 0) {
      scale[row] = __half_as_ushort(sh);
      zero[row] = static_cast<uint8_t>(zz);
    }
  }
}

// acc += w * (FP16 value in the low / high half of x), the conversion done
// inside the FMA (v_fma_mix_f32).  A code c enters as the FP16 subnormal
// c * 2^-24 (bit pattern c; exact, the kernel runs with FP16 denormals on),
// so the caller scales w by 2^24.
__device__ __forceinline__ float fma_mix_lo(float w, unsigned x, float acc) {
  asm("v_fma_mix_f32 %0, %1, %2, %0 op_sel_hi:[0,1,0]" : "+v"(acc) : "v"(w), "v"(x));
  return acc;
}
__device__ __forceinline__ float fma_mix_hi(float w, unsigned x, float acc) {
  asm("v_fma_mix_f32 %0, %1, %2, %0 op_sel:[0,1,0] op_sel_hi:[0,1,0]" : "+v"(acc) : "v"(w), "v"(x));
  return acc;
}

// byte k of v as a float (one v_cvt_f32_ubyte{k})
template <int k>
__device__ __forceinline__ float ubyte(unsigned v) {
  return static_cast<float>((v >> (8 * k)) & 0xffu);
}

// Weights of the V pass carry a factor kVScale(R): 2^24 where the codes enter
// the FMAs as FP16 subnormals (up to 2 heads a block), 1 where they are
// converted once and shared by 4 heads' FMAs (there the FMAs dominate and
// the mixed-precision form measured slower).
template <int R>
constexpr float kVScale = R <= 2 ? 16777216.0f : 1.0f;

// acc[r][d] += w[r] / kVScale * code[d] over the 8 NW dims of one lane's
// load (dword i holds dims 8i..8i+7, dim 8i+k in nibble k).
template <int R, int NW>
__device__ __forceinline__ void axpy_codes(float (&acc)[R][8 * NW], const float (&w)[R], const unsigned (&v)[NW]) {
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    if constexpr (R <= 2) {
      // a masked shift puts the codes of dims 8i+j and 8i+j+4 in the two
      // halves of one register, which the heads' FMAs read directly
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const unsigned x = (v[i] >> (4 * j)) & 0x000f000fu;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          acc[r][8 * i + j] = fma_mix_lo(w[r], x, acc[r][8 * i + j]);
          acc[r][8 * i + j + 4] = fma_mix_hi(w[r], x, acc[r][8 * i + j + 4]);
        }
      }
    } else {
      unsigned lo = v[i] & 0x0f0f0f0fu, hi = (v[i] >> 4) & 0x0f0f0f0fu;
      // Opaque to the optimizer, so that it cannot fold the masks into a
      // 4-bit field extract per code: each byte then converts with one
      // v_cvt_f32_ubyte{0..3}.
      asm volatile("" : "+v"(lo), "+v"(hi));
      const float x[8] = {ubyte<0>(lo), ubyte<0>(hi), ubyte<1>(lo), ubyte<1>(hi),
                          ubyte<2>(lo), ubyte<2>(hi), ubyte<3>(lo), ubyte<3>(hi)};
      // x[e]: the code of dim 8i + e
#pragma unroll
      for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r][8 * i + e] = fmaf(w[r], x[e], acc[r][8 * i + e]);
    }
  }
}

struct AttnArgs {
  const unsigned short* q;
  const uint8_t *kc, *vc;
  const unsigned short *ks, *vs;
  const uint8_t *kz, *vz;
  const int* lengths;
  unsigned short* o;
  int H, Hkv, T;
  float scale;
  int Tc;     // tokens per chunk when the tokens are split over blocks
  float* ws;  // per-chunk partials: o [nc][B][H][128], max [nc][B][H], sum [nc][B][H]
};

// Tokens in flight per wave and pass: U loads of 16 tokens each.
constexpr int kUnroll = 4;
// Query heads per block, at most.  The heads of one kv group in a block
// share its cache reads and code conversions; their scores sit side by side
// in LDS ([R][rows] floats, at most kAttnScoreLds bytes).  The launch plan
// picks 4 or 2, or 1 when neither divides the group or fits.
constexpr int kMaxHeadsPerBlock = 4;
constexpr size_t kAttnScoreLds = size_t(kMaxCacheLen) * sizeof(float);

// SPLIT: block (x, y, z) takes only tokens [z Tc, (z + 1) Tc) of its
// sequence and writes that chunk's softmax partials (running max m, sum of
// exp(s - m), unnormalized output) to the workspace; a second kernel combines
// the chunks.  Used when (sequence, head group) pairs alone would leave most
// CUs idle (small batches, long caches).
template <int R, bool SPLIT>
__global__ __launch_bounds__(kAttnThreads) void kv4_decode_attention_kernel(AttnArgs a) {
  extern __shared__ float sc[];  // [R][Ts] scores, then weights
  __shared__ float red[R][kAttnThreads / 64];
  __shared__ float part[kAttnThreads / 64][R][kHeadDim + 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // Block -> (b, R consecutive query heads of one kv head).  Workgroups are
  // dealt round-robin to the 8 XCDs, each with its own L2; when a kv head
  // has several blocks, they are given consecutive slots on one XCD, so that
  // the cache rows they all read come from that L2 after the first.  (Plain
  // order when the grid does not tile.)
  const int rep = a.H / a.Hkv;     // query heads per kv head
  const int bpg = rep / R;         // blocks per kv head
  int hb = blockIdx.x, b = blockIdx.y;
  {
    const int nb = gridDim.x * gridDim.y;
    const int d = blockIdx.y * gridDim.x + blockIdx.x;
    if (bpg > 1 && nb % (8 * bpg) == 0) {
      const int xcd = d % 8, slot = d / 8;
      const int pair = (slot / bpg) * 8 + xcd;  // (b, kv head) index
      b = pair / a.Hkv;
      hb = (pair % a.Hkv) * bpg + slot % bpg;
    }
  }
  const int h0 = hb * R;           // first query head of the block
  const int g = h0 / rep;
  const int L = min(max(a.lengths[b], 0), a.T);
  const int64_t row0 = (int64_t(b) * a.Hkv + g) * a.T;  // first cache row of this kv head
  // this block's tokens [t0, t1), and the stride of a score row in LDS
  const int t0 = SPLIT ? int(blockIdx.z) * a.Tc : 0;
  const int t1 = SPLIT ? min(L, t0 + a.Tc) : L;
  const int Ts = SPLIT ? a.Tc : a.T;

  // Pass 1, the scores, on the matrix cores in exact integer arithmetic.
  // Each query row q' = scale * q is split into three signed-byte pieces,
  //   q' ~= S0 b0 + S1 b1 + S2 b2,  S0 = max|q'| / 127,  S1 = S0 / 254,  S2 = S1 / 254,
  // each piece the rounded remainder left by the ones before (the sum is
  // within about 2^-23 max|q'| of q'), so that
  //   <q', c_t - z_t> = sum_p S_p (<b_p, c_t> - z_t sum(b_p))
  // takes only exact INT8 products.  One v_mfma_i32_16x16x64_i8 multiplies
  // 16 rows (M: 4 heads x (3 pieces + an empty row)) by 16 tokens (N); the
  // 128 dims are two K steps.  Lane (l16 = lane % 16, jq = lane / 16) holds,
  // for K step h, the 16 K values of quarter jq: dims 32 jq + 16 h + o(k),
  // o = 0,2,4,6, 1,3,5,7, 8,10,12,14, 9,11,13,15 -- the order in which a
  // 16-byte load of codes (dims 32 jq .. 32 jq + 31) comes out of the
  // nibble split below.  The A operand (row l16 = 4 r + p) is piece p of
  // head r; the B operand (column l16) is a token's codes; the result lane
  // (token l16, jq) holds the three piece products of head jq in elements
  // 0..2.
  const int l16 = lane & 15, jq = lane >> 4;
  i32x4 qa[2];
  float spc;  // step S_p of this lane's row
  int bsum;   // sum of its piece over the 128 dims
  {
    const int r = l16 >> 2, pc = l16 & 3;
    const bool on = r < R && pc < 3;
    const uint4* qv = reinterpret_cast<const uint4*>(a.q + (int64_t(b) * a.H + h0 + min(r, R - 1)) * kHeadDim + 32 * jq);
    float x[32];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 u = qv[i];
      const unsigned w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[8 * i + 2 * e] = a.scale * half_lo(w[e]);
        x[8 * i + 2 * e + 1] = a.scale * half_hi(w[e]);
      }
    }
    float amax = 0.0f;
#pragma unroll
    for (int d = 0; d < 32; ++d) amax = fmaxf(amax, fabsf(x[d]));
    amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
    const float s0 = amax / 127.0f, s1 = s0 / 254.0f, s2 = s1 / 254.0f;
    const float i0 = amax > 0.0f ? 127.0f / amax : 0.0f, i1 = 254.0f * i0, i2 = 254.0f * i1;
    const auto clamp127 = [](float v) { return fminf(127.0f, fmaxf(-127.0f, v)); };
    int bp[32];
    int sum = 0;
#pragma unroll
    for (int d = 0; d < 32; ++d) {
      const float b0 = clamp127(rintf(x[d] * i0));
      const float r1 = fmaf(-b0, s0, x[d]);
      const float b1 = clamp127(rintf(r1 * i1));
      const float r2 = fmaf(-b1, s1, r1);
      const float b2 = clamp127(rintf(r2 * i2));
      bp[d] = on ? int(pc == 0 ? b0 : pc == 1 ? b1 : b2) : 0;
      sum += bp[d];
    }
    sum += __shfl_xor(sum, 16, 64);
    sum += __shfl_xor(sum, 32, 64);
    bsum = sum;
    spc = pc == 0 ? s0 : pc == 1 ? s1 : s2;
    // byte 4 w + e of K step h: dim 16 h + 8 (w / 2) + 2 e + w % 2
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        unsigned v = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) v |= (unsigned(bp[16 * h + 8 * (w >> 1) + 2 * e + (w & 1)]) & 0xffu) << (8 * e);
        qa[h][w] = int(v);
      }
  }
  // steps and piece sums of head jq (rows 4 jq + p), for the lanes that
  // combine its scores
  float sp[3], bs[3];
#pragma unroll
  for (int pc = 0; pc < 3; ++pc) {
    sp[pc] = __shfl(spc, 4 * jq + pc, 64);
    bs[pc] = float(__shfl(bsum, 4 * jq + pc, 64));
  }

  // Both passes load the next round's cache rows before working on the
  // current one, so each wave has a round of loads in flight while it computes.
  constexpr int kStride = kAttnThreads / 4 * kUnroll;  // tokens per block round
  const int first = t0 + wave * 16 * kUnroll;          // this wave's first token
  float mown = -INFINITY;  // largest score of head jq seen by this lane
  // this kv head's rows: block-uniform bases, 32-bit token offsets
  const uint4* kc = reinterpret_cast<const uint4*>(a.kc + row0 * kRowBytes);
  const unsigned short* ksb = a.ks + row0;
  const uint8_t* kzb = a.kz + row0;
  uint4 kn[kUnroll];
  unsigned short sn[kUnroll];
  int zn[kUnroll];
  auto kload = [&](int base) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int t = min(base + 16 * u + l16, t1 - 1);  // past t1: a valid token, result dropped
      kn[u] = kc[unsigned(t * 4 + jq)];
      sn[u] = ksb[unsigned(t)];
      zn[u] = kzb[unsigned(t)];
    }
  };
  if (first < t1) kload(first);
  for (int base = first; base < t1; base += kStride) {
    uint4 c[kUnroll];
    float s[kUnroll];
    int z[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      c[u] = kn[u];
      s[u] = __half2float(__ushort_as_half(sn[u]));
      z[u] = zn[u];
    }
    if (base + kStride < t1) kload(base + kStride);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const unsigned w[4] = {c[u].x, c[u].y, c[u].z, c[u].w};
      i32x4 d = {0, 0, 0, 0};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const i32x4 cb = {int(w[2 * h] & 0x0f0f0f0fu), int((w[2 * h] >> 4) & 0x0f0f0f0fu),
                          int(w[2 * h + 1] & 0x0f0f0f0fu), int((w[2 * h + 1] >> 4) & 0x0f0f0f0fu)};
        d = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[h], cb, d, 0, 0, 0);
      }
      const int t = base + 16 * u + l16;
      // <b_p, c_t> - z_t sum(b_p): integers below 2^24 in magnitude, so the
      // FMA is exact
      const float zf = float(z[u]);
      const float v = s[u] * (sp[0] * fmaf(-zf, bs[0], float(d[0])) + sp[1] * fmaf(-zf, bs[1], float(d[1])) +
                              sp[2] * fmaf(-zf, bs[2], float(d[2])));
      if (jq < R && t < t1) {
        mown = fmaxf(mown, v);
        sc[jq * Ts + (t - t0)] = v;
      }
    }
  }
  float mx[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    mx[r] = wave_max(jq == r ? mown : -INFINITY);
    if (lane == 0) red[r][wave] = mx[r];
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < R; ++r) mx[r] = fmaxf(fmaxf(red[r][0], red[r][1]), fmaxf(red[r][2], red[r][3]));
  __syncthreads();

  // weights and their sums
  float lsum[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    lsum[r] = 0.0f;
    for (int t = threadIdx.x; t < t1 - t0; t += kAttnThreads) {
      const float e = __expf(sc[r * Ts + t] - mx[r]);
      sc[r * Ts + t] = e;
      lsum[r] += e;
    }
    lsum[r] = wave_sum(lsum[r]);
    if (lane == 0) red[r][wave] = lsum[r];
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < R; ++r) lsum[r] = red[r][0] + red[r][1] + red[r][2] + red[r][3];

  // pass 2: o = sum_t a_t s_t (c_t - z_t), accumulated as
  // sum (a_t s_t) c_t - sum (a_t s_t z_t); the weights carry kVScale<R>,
  // taken off the second sum at the end (exact).  LPT lanes share a token,
  // DPT dims each: 4 x 32 for up to 2 heads, 8 x 16 for 4 heads, whose
  // R x DPT accumulators would otherwise leave room for only 2 waves per SIMD.
  constexpr int LPT = R >= 4 ? 8 : 4;
  constexpr int DPT = kHeadDim / LPT;
  constexpr int NW = DPT / 8;     // code dwords per lane and token
  constexpr int SLOTS = 64 / LPT; // tokens per wave-wide load
  constexpr int U = LPT;          // loads per round: 64 tokens a wave
  static_assert(SLOTS * U == 16 * kUnroll, "both passes take the same tokens per round");
  const int vp = lane % LPT;      // which DPT dims of the head
  const int vt = lane / LPT;      // token slot within the wave's SLOTS
  float acc[R][DPT], zacc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    zacc[r] = 0.0f;
#pragma unroll
    for (int i = 0; i < DPT; ++i) acc[r][i] = 0.0f;
  }
  const uint8_t* vrow = a.vc + row0 * kRowBytes;
  const unsigned short* vsb = a.vs + row0;
  const uint8_t* vzb = a.vz + row0;
  unsigned vn[U][NW];
  unsigned short vsn[U];
  int vzn[U];
  auto vload = [&](int base) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int tc = min(base + SLOTS * u + vt, t1 - 1);
      if constexpr (NW == 4) {
        const uint4 q = reinterpret_cast<const uint4*>(vrow)[unsigned(tc * 4 + vp)];
        vn[u][0] = q.x;
        vn[u][1] = q.y;
        vn[u][2] = q.z;
        vn[u][3] = q.w;
      } else {
        const uint2 q = reinterpret_cast<const uint2*>(vrow)[unsigned(tc * 8 + vp)];
        vn[u][0] = q.x;
        vn[u][1] = q.y;
      }
      vsn[u] = vsb[unsigned(tc)];
      vzn[u] = vzb[unsigned(tc)];
    }
  };
  if (first < t1) vload(first);
  for (int base = first; base < t1; base += kStride) {
    unsigned c[U][NW];
    float w[U][R];
    int z[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = base + SLOTS * u + vt;
      const int tc = min(t, t1 - 1);
#pragma unroll
      for (int i = 0; i < NW; ++i) c[u][i] = vn[u][i];
      const float vs = __half2float(__ushort_as_half(vsn[u])) * kVScale<R>;  // exact
#pragma unroll
      for (int r = 0; r < R; ++r) w[u][r] = t < t1 ? sc[r * Ts + (tc - t0)] * vs : 0.0f;
      z[u] = vzn[u];
    }
    if (base + kStride < t1) vload(base + kStride);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      axpy_codes<R, NW>(acc, w[u], c[u]);
#pragma unroll
      for (int r = 0; r < R; ++r) zacc[r] = fmaf(w[u][r], float(z[u]), zacc[r]);
    }
  }
  // sum over the token slots of the wave (lanes with equal vp): the slots
  // of a row of 16 lanes by rotations (by 4 and 8, or by 8), then the rows
#pragma unroll
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int i = 0; i < DPT; ++i) {
      if constexpr (LPT == 4) acc[r][i] += dppf<kDppRor4>(acc[r][i]);
      acc[r][i] += dppf<kDppRor8>(acc[r][i]);
    }
    if constexpr (LPT == 4) zacc[r] += dppf<kDppRor4>(zacc[r]);
    zacc[r] += dppf<kDppRor8>(zacc[r]);
#pragma unroll
    for (int off = 16; off < 64; off <<= 1) {
#pragma unroll
      for (int i = 0; i < DPT; ++i) acc[r][i] += __shfl_xor(acc[r][i], off, 64);
      zacc[r] += __shfl_xor(zacc[r], off, 64);
    }
    if (vt == 0) {
#pragma unroll
      for (int i = 0; i < DPT; ++i) part[wave][r][DPT * vp + i] = acc[r][i] - zacc[r] * (1.0f / kVScale<R>);
    }
  }
  __syncthreads();
  const int64_t BH = int64_t(gridDim.y) * a.H;  // (sequence, query head) pairs
  for (int idx = threadIdx.x; idx < R * kHeadDim; idx += kAttnThreads) {
    const int r = idx / kHeadDim, d = idx % kHeadDim;
    const float v = part[0][r][d] + part[1][r][d] + part[2][r][d] + part[3][r][d];
    float ls = lsum[0], m = mx[0];
#pragma unroll
    for (int k = 1; k < R; ++k) {
      ls = r == k ? lsum[k] : ls;
      m = r == k ? mx[k] : m;
    }
    const int64_t bh = int64_t(b) * a.H + h0 + r;
    if constexpr (SPLIT) {
      const int64_t cbh = int64_t(blockIdx.z) * BH + bh;
      a.ws[cbh * kHeadDim + d] = v;
      if (d == 0) {
        a.ws[int64_t(gridDim.z) * BH * kHeadDim + cbh] = t1 > t0 ? m : -INFINITY;
        a.ws[int64_t(gridDim.z) * BH * (kHeadDim + 1) + cbh] = ls;
      }
    } else {
      const float o = L > 0 ? v / ls : 0.0f;
      a.o[bh * kHeadDim + d] = __half_as_ushort(__float2half_rn(o));
    }
  }
}

// Combines the nc chunk partials of every (sequence, head): with M the
// largest chunk max, o = sum_c o_c e^(m_c - M) / sum_c l_c e^(m_c - M).
// Empty chunks carry m = -inf and contribute nothing; a sequence with no
// tokens gets zeros.  One block per (head, sequence): a thread per chunk
// finds M and the weights, then 8 groups of 32 threads each sum every 8th
// chunk's output, 4 dims a thread, so that the chunk loads are independent.
constexpr int kCombineThreads = 256;
constexpr int kMaxChunks = kMaxCacheLen / kAttnThreads;  // a chunk is at least one 256-token pass
static_assert(kMaxChunks <= kCombineThreads, "one thread per chunk");

__global__ __launch_bounds__(kCombineThreads) void kv4_attention_combine_kernel(const float* __restrict__ ws, int nc,
                                                                               int64_t BH, int H,
                                                                               unsigned short* __restrict__ o) {
  __shared__ float wgt[kMaxChunks];
  __shared__ float red[2][kCombineThreads / 64];
  __shared__ float4 part[kCombineThreads / 32][kHeadDim / 4];
  const int64_t bh = int64_t(blockIdx.y) * H + blockIdx.x;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const float* wm = ws + int64_t(nc) * BH * kHeadDim;
  const float* wl = wm + int64_t(nc) * BH;
  const float m = t < nc ? wm[t * BH + bh] : -INFINITY;
  const float l = t < nc ? wl[t * BH + bh] : 0.0f;
  float M = wave_max(m);
  if (lane == 0) red[0][wave] = M;
  __syncthreads();
  M = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
  const float e = t < nc && M > -INFINITY ? __expf(m - M) : 0.0f;  // m = -inf: 0
  if (t < nc) wgt[t] = e;
  float L = wave_sum(l * e);
  if (lane == 0) red[1][wave] = L;
  __syncthreads();
  L = red[1][0] + red[1][1] + red[1][2] + red[1][3];
  const int d4 = t & 31, cg = t >> 5;
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll 4
  for (int c = cg; c < nc; c += kCombineThreads / 32) {
    const float4 v = *reinterpret_cast<const float4*>(ws + (c * BH + bh) * kHeadDim + 4 * d4);
    const float w = wgt[c];
    acc.x = fmaf(v.x, w, acc.x);
    acc.y = fmaf(v.y, w, acc.y);
    acc.z = fmaf(v.z, w, acc.z);
    acc.w = fmaf(v.w, w, acc.w);
  }
  part[cg][d4] = acc;
  __syncthreads();
  if (t < kHeadDim) {
    const float* pf = reinterpret_cast<const float*>(&part[0][0]);
    float v = 0.0f;
#pragma unroll
    for (int g = 0; g < kCombineThreads / 32; ++g) v += pf[g * kHeadDim + t];
    o[bh * kHeadDim + t] = __half_as_ushort(__float2half_rn(L > 0.0f ? v / L : 0.0f));
  }
}

}  // namespace
}  // namespace qoq

using namespace qoq;

extern "C" int qoq_kv4_quant(const void* x_fp16, int64_t n_rows, int32_t head_dim, int64_t ldx, uint8_t* codes,
                             void* scale_fp16, uint8_t* zero, void* stream) {
  clear_error();
  if (!x_fp16 || !codes || !scale_fp16 || !zero) return fail(QOQ_ERR_INVALID_ARG, "qoq_kv4_quant: null pointer argument");
  if (head_dim != kHeadDim) return fail(QOQ_ERR_UNSUPPORTED_SHAPE, "qoq_kv4_quant: head_dim must be 128, got %d", head_dim);
  if (n_rows < 1 || n_rows > (int64_t(1) << 40)) return fail(QOQ_ERR_UNSUPPORTED_SHAPE, "qoq_kv4_quant: n_rows out of range");
  if (ldx < head_dim || ldx % 8)
    return fail(QOQ_ERR_INVALID_ARG, "qoq_kv4_quant: ldx must be a multiple of 8 and >= head_dim");
  if (reinterpret_cast<uintptr_t>(x_fp16) % 16 || reinterpret_cast<uintptr_t>(codes) % 4 ||
      reinterpret_cast<uintptr_t>(scale_fp16) % 2)
    return fail(QOQ_ERR_ALIGNMENT, "qoq_kv4_quant: x needs 16-byte, codes 4-byte, scale 2-byte alignment");
  const int64_t blocks = (n_rows + kQuantRowsPerBlock - 1) / kQuantRowsPerBlock;
  if (blocks > 0x7fffffff) return fail(QOQ_ERR_UNSUPPORTED_SHAPE, "qoq_kv4_quant: too many rows");
  hipLaunchKernelGGL(kv4_quant_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(x_fp16), ldx / 8, n_rows,
                     reinterpret_cast<unsigned*>(codes), static_cast<unsigned short*>(scale_fp16), zero);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(QOQ_ERR_HIP, "qoq_kv4_quant: launch failed: %s", hipGetErrorString(e));
  return QOQ_OK;
}

namespace {

// Launch plan of the decode attention: R query heads per block; with
// nc > 1 the tokens are cut into nc chunks of Tc whose partials are combined
// afterwards.
struct AttnPlan {
  int R = 1, Tc = 0, nc = 1;
};

// Tokens are split only while (sequence, head group) workgroups alone number
// fewer than kSplitBelowBlocks (one per CU).  A chunk is 1024 tokens, four
// passes of the block's token loop, which amortizes the block's fixed work
// (query load, cross-lane reductions, partial write); it is halved, down to
// one pass, while there would be fewer than kSplitTargetBlocks workgroups
// (two per CU: a lone 4-wave block per CU leaves each SIMD one wave and
// nothing to hide its load latency behind).
constexpr int64_t kSplitBelowBlocks = 256;
constexpr int64_t kSplitTargetBlocks = 512;
constexpr int kSplitChunkMax = 1024;
constexpr int kSplitChunkMin = kAttnThreads;  // 16 tokens x kUnroll per wave, 4 waves
static_assert(kSplitChunkMin == kAttnThreads / 64 * 16 * kUnroll, "one pass of the token loop");
static_assert(kMaxHeadsPerBlock * kSplitChunkMax <= kMaxCacheLen, "chunk scores fit the LDS budget");

// Chunks for R heads per block (nc = 1: the whole cache in one block).
AttnPlan plan_with(int B, int H, int T_max, int R, bool allow_split) {
  AttnPlan p;
  p.R = R;
  const int64_t blocks = int64_t(B) * H / R;
  if (!allow_split || blocks >= kSplitBelowBlocks || T_max < 2 * kSplitChunkMin) return p;
  int64_t Tc = kSplitChunkMax;
  while (Tc > kSplitChunkMin && blocks * ((T_max + Tc - 1) / Tc) < kSplitTargetBlocks) Tc /= 2;
  const int64_t nc = (T_max + Tc - 1) / Tc;
  if (nc < 2) return p;
  p.Tc = int(Tc);
  p.nc = int(nc);
  return p;
}

// Heads per block: 4, 2 or 1 of a kv group (with token chunks, 1 only when
// neither 4 nor 2 divides the group or fits the LDS budget: there the chunks
// supply the blocks).  More heads per block share each code's conversion
// among more FMAs, fewer heads give more blocks: among the plans that reach
// kSplitTargetBlocks blocks the one with the longest chunks wins (then the
// most heads); if none does, the one with the most blocks.
AttnPlan attn_plan(int B, int H, int Hkv, int T_max, bool allow_split) {
  const int rep = H / Hkv;
  AttnPlan best;
  bool have = false;
  int64_t best_blocks = 0, best_tc = 0;
  for (int r = kMaxHeadsPerBlock; r >= 1; r >>= 1) {
    if (rep % r) continue;
    if (r == 1 && have && allow_split) break;
    const AttnPlan p = plan_with(B, H, T_max, r, allow_split);
    const int64_t rows = p.nc > 1 ? p.Tc : T_max;  // score row length in LDS
    if (size_t(r) * size_t(rows) * sizeof(float) > kAttnScoreLds) continue;
    const int64_t blocks = int64_t(B) * H / r * p.nc;
    const int64_t tc = p.nc > 1 ? p.Tc : int64_t(1) << 40;
    const bool full = blocks >= kSplitTargetBlocks, best_full = best_blocks >= kSplitTargetBlocks;
    const bool better = !have || (full != best_full ? full : full ? tc > best_tc : blocks > best_blocks);
    if (better) {
      best = p;
      best_blocks = blocks;
      best_tc = tc;
      have = true;
    }
  }
  return best;
}

size_t attn_workspace_bytes(const AttnPlan& p, int B, int H) {
  return p.nc > 1 ? size_t(p.nc) * size_t(B) * size_t(H) * (kHeadDim + 2) * sizeof(float) : 0;
}

int check_attn_args(const char* fn, const void* q_fp16, const uint8_t* k_codes, const void* k_scale_fp16,
                    const uint8_t* k_zero, const uint8_t* v_codes, const void* v_scale_fp16, const uint8_t* v_zero,
                    const int32_t* lengths, int32_t B, int32_t H, int32_t Hkv, int32_t T_max, int32_t head_dim,
                    float softmax_scale, void* o_fp16) {
  if (!q_fp16 || !k_codes || !k_scale_fp16 || !k_zero || !v_codes || !v_scale_fp16 || !v_zero || !lengths || !o_fp16)
    return fail(QOQ_ERR_INVALID_ARG, "%s: null pointer argument", fn);
  if (head_dim != kHeadDim) return fail(QOQ_ERR_UNSUPPORTED_SHAPE, "%s: head_dim must be 128, got %d", fn, head_dim);
  if (B < 1 || H < 1 || Hkv < 1 || H % Hkv || B > 65535 || H > 65535)
    return fail(QOQ_ERR_UNSUPPORTED_SHAPE, "%s: need B, H, Hkv >= 1 and H a multiple of Hkv", fn);
  if (T_max < 1 || T_max > kMaxCacheLen)
    return fail(QOQ_ERR_UNSUPPORTED_SHAPE, "%s: T_max must be in [1, %d]", fn, kMaxCacheLen);
  if (!std::isfinite(softmax_scale)) return fail(QOQ_ERR_INVALID_ARG, "%s: scale not finite", fn);
  const auto al = [](const void* p, uintptr_t n) { return reinterpret_cast<uintptr_t>(p) % n == 0; };
  if (!al(q_fp16, 16) || !al(k_codes, 16) || !al(v_codes, 16) || !al(k_scale_fp16, 2) || !al(v_scale_fp16, 2) ||
      !al(lengths, 4) || !al(o_fp16, 2))
    return fail(QOQ_ERR_ALIGNMENT, "%s: q and codes need 16-byte alignment", fn);
  return QOQ_OK;
}

template <bool SPLIT>
int launch_attention(const char* fn, const AttnArgs& a, const AttnPlan& p, int B, int64_t lds, hipStream_t stream) {
  using Kernel = void (*)(AttnArgs);
  const Kernel k = p.R == 4   ? kv4_decode_attention_kernel<4, SPLIT>
                   : p.R == 2 ? kv4_decode_attention_kernel<2, SPLIT>
                              : kv4_decode_attention_kernel<1, SPLIT>;
  if (lds > 48 * 1024) {
    const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                                hipFuncAttributeMaxDynamicSharedMemorySize, int(kAttnScoreLds));
    if (attr != hipSuccess) return fail(QOQ_ERR_HIP, "%s: LDS attribute: %s", fn, hipGetErrorString(attr));
  }
  const dim3 grid(static_cast<unsigned>(a.H / p.R), static_cast<unsigned>(B), static_cast<unsigned>(p.nc));
  hipLaunchKernelGGL(k, grid, dim3(kAttnThreads), size_t(lds), stream, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(QOQ_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return QOQ_OK;
}

int run_attention(const char* fn, bool allow_split, const void* q_fp16, const uint8_t* k_codes,
                  const void* k_scale_fp16, const uint8_t* k_zero, const uint8_t* v_codes, const void* v_scale_fp16,
                  const uint8_t* v_zero, const int32_t* lengths, int32_t B, int32_t H, int32_t Hkv, int32_t T_max,
                  int32_t head_dim, float softmax_scale, void* o_fp16, void* workspace, size_t workspace_bytes,
                  void* stream) {
  clear_error();
  const int st = check_attn_args(fn, q_fp16, k_codes, k_scale_fp16, k_zero, v_codes, v_scale_fp16, v_zero, lengths,
                                 B, H, Hkv, T_max, head_dim, softmax_scale, o_fp16);
  if (st != QOQ_OK) return st;
  const AttnPlan p = attn_plan(B, H, Hkv, T_max, allow_split);
  const size_t need = attn_workspace_bytes(p, B, H);
  if (need) {
    if (!workspace || workspace_bytes < need)
      return fail(QOQ_ERR_INVALID_ARG, "%s: workspace of %zu bytes required (got %zu); see the workspace-size query", fn, need,
                  workspace ? workspace_bytes : size_t(0));
    if (reinterpret_cast<uintptr_t>(workspace) % 16)
      return fail(QOQ_ERR_ALIGNMENT, "%s: workspace needs 16-byte alignment", fn);
  }
  AttnArgs a;
  a.q = static_cast<const unsigned short*>(q_fp16);
  a.kc = k_codes;
  a.vc = v_codes;
  a.ks = static_cast<const unsigned short*>(k_scale_fp16);
  a.vs = static_cast<const unsigned short*>(v_scale_fp16);
  a.kz = k_zero;
  a.vz = v_zero;
  a.lengths = lengths;
  a.o = static_cast<unsigned short*>(o_fp16);
  a.H = H;
  a.Hkv = Hkv;
  a.T = T_max;
  a.scale = softmax_scale;
  a.Tc = p.Tc;
  a.ws = static_cast<float*>(workspace);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.nc == 1) return launch_attention<false>(fn, a, p, B, int64_t(p.R) * T_max * int64_t(sizeof(float)), s);
  const int st2 = launch_attention<true>(fn, a, p, B, int64_t(p.R) * p.Tc * int64_t(sizeof(float)), s);
  if (st2 != QOQ_OK) return st2;
  hipLaunchKernelGGL(kv4_attention_combine_kernel, dim3(static_cast<unsigned>(H), static_cast<unsigned>(B)),
                     dim3(kCombineThreads), 0, s, static_cast<const float*>(workspace), p.nc, int64_t(B) * H, int(H),
                     static_cast<unsigned short*>(o_fp16));
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(QOQ_ERR_HIP, "%s: combine launch failed: %s", fn, hipGetErrorString(e));
  return QOQ_OK;
}

}  // namespace

extern "C" int qoq_kv4_decode_attention(const void* q_fp16, const uint8_t* k_codes, const void* k_scale_fp16,
                                        const uint8_t* k_zero, const uint8_t* v_codes, const void* v_scale_fp16,
                                        const uint8_t* v_zero, const int32_t* lengths, int32_t B, int32_t H,
                                        int32_t Hkv, int32_t T_max, int32_t head_dim, float softmax_scale,
                                        void* o_fp16, void* stream) {
  return run_attention("qoq_kv4_decode_attention", false, q_fp16, k_codes, k_scale_fp16, k_zero, v_codes,
                       v_scale_fp16, v_zero, lengths, B, H, Hkv, T_max, head_dim, softmax_scale, o_fp16, nullptr, 0,
                       stream);
}

extern "C" size_t qoq_kv4_decode_attention_workspace_size(int32_t B, int32_t H, int32_t Hkv, int32_t T_max) {
  if (B < 1 || H < 1 || Hkv < 1 || H % Hkv || B > 65535 || H > 65535 || T_max < 1 || T_max > kMaxCacheLen) return 0;
  return attn_workspace_bytes(attn_plan(B, H, Hkv, T_max, true), B, H);
}

extern "C" int qoq_kv4_decode_attention_plan(int32_t B, int32_t H, int32_t Hkv, int32_t T_max, int32_t split,
                                             int32_t* heads_per_block, int32_t* token_chunks) {
  clear_error();
  if (!heads_per_block || !token_chunks)
    return fail(QOQ_ERR_INVALID_ARG, "qoq_kv4_decode_attention_plan: null pointer argument");
  if (B < 1 || H < 1 || Hkv < 1 || H % Hkv || B > 65535 || H > 65535 || T_max < 1 || T_max > kMaxCacheLen)
    return fail(QOQ_ERR_UNSUPPORTED_SHAPE, "qoq_kv4_decode_attention_plan: shape out of range");
  const AttnPlan p = attn_plan(B, H, Hkv, T_max, split != 0);
  *heads_per_block = p.R;
  *token_chunks = p.nc;
  return QOQ_OK;
}

extern "C" int qoq_kv4_decode_attention_split(const void* q_fp16, const uint8_t* k_codes, const void* k_scale_fp16,
                                              const uint8_t* k_zero, const uint8_t* v_codes,
                                              const void* v_scale_fp16, const uint8_t* v_zero,
                                              const int32_t* lengths, int32_t B, int32_t H, int32_t Hkv,
                                              int32_t T_max, int32_t head_dim, float softmax_scale, void* o_fp16,
                                              void* workspace, size_t workspace_bytes, void* stream) {
  return run_attention("qoq_kv4_decode_attention_split", true, q_fp16, k_codes, k_scale_fp16, k_zero, v_codes,
                       v_scale_fp16, v_zero, lengths, B, H, Hkv, T_max, head_dim, softmax_scale, o_fp16, workspace,
                       workspace_bytes, stream);
}
