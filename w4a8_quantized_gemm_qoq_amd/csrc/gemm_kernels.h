#pragma once
// Kernels of the W4A8 GEMM for gfx950 (MI355X), shared by the entry points
// of gemm_w4.hip, gemm_w8.hip and gemm_sat.hip: UINT4 weights dequantized to
// INT8 in registers, INT8 MFMA with INT32 accumulation, fused FP32 scale epilogue.
//
// Follows "QServe: W4A8KV4 Quantization and System Co-design for Efficient
// LLM Serving" (paperlayer.ai abs/2405.04532v3 summary):
//   §3 / §4: weights (not partial sums) are dequantized inside the main loop,
//     so one INT32 accumulator spans all of K and the matrix units stay on
//     INT8; four weights are decoded per 32-bit register operation;
//   §4: the protective level-0 range [-119, 119] keeps the dequantized
//     intermediates inside INT8, so no saturating arithmetic is needed;
//   §5: subtraction after multiplication, w8 = q4*s1 - z*s1; weights stored in
//     computation order and read with 128-bit loads; per-channel scale fused
//     into the epilogue; FP16 output.
//
// In-register dequantization (per 32-bit word of 8 packed UINT4 codes):
//   lo = v & 0x0f0f0f0f, hi = (v >> 4) & 0x0f0f0f0f   (four codes per word)
//   u  = v_pk_mad_u16(lo, s1|s1<<16, c*0x01010101) with c = 128 - z*s1
//   w8 = u ^ 0x80808080
// Each byte of u is q4*s1 + 128 - z*s1 = w8 + 128, which lies in [7, 249]
// because |w8| <= 121 (exhaustively true for the [-119, 119] level-0 range),
// so neither the 16-bit multiply-add nor the byte lanes carry, and XOR 0x80
// turns the biased byte into the two's-complement INT8 w8.  For the
// per-channel variant s1 = 1 and c = 128 - z.
//
// Weight formats (template parameter WF of every kernel):
//   kWfG128:       progressive g128 UINT4 (the path above);
//   kWfPerChannel: per-channel UINT4, w8 = q4 - z;
//   kWfW8:         per-channel INT8 weights used as they are (the W8A8
//                  comparator: same kernels, twice the weight bytes, no
//                  dequantization);
//   kWfG128Sat:    g128 with a saturating dequantization (ablation of the
//                  protective range): each value goes through a 16-bit lane,
//                  clamp(q4*s1 + 128 - z*s1, 0, 255) ^ 0x80.
//
// Three kernels share the packed layout (see qoq.h):
//   strip:  v_mfma_i32_16x16x64_i8, up to 16 rows; one contiguous weight
//           strip per wave, activations copied into LDS once (decode).
//   skinny: v_mfma_i32_16x16x64_i8, 16-row M tiles, K split across the
//           waves of a block; up to 64 rows (decode, memory-bound), and up
//           to 256 rows when one round of blocks covers the problem.
//   large:  v_mfma_i32_32x32x32_i8, 128x128 or 256x256 block tiles, K
//           optionally split across blocks; above 64 rows (prefill).
// Weights always go global -> VGPR directly and are dequantized in
// registers.  Both MFMA operands use the same K order per (lane group, byte),
// so the contraction is exact whatever order the matrix unit walks K in.

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <algorithm>

#include "qoq_internal.h"

// Large-M tile: WM x WN waves, each TM x TN tiles of 32x32.
#ifndef QOQ_LWM
#define QOQ_LWM 2
#define QOQ_LWN 4
#define QOQ_LTM 4
#define QOQ_LTN 2
#endif
// Register-ring depth (groups of weights / activations in flight) of the big
// and of the 128x128 large-M tile.
#ifndef QOQ_LD
#define QOQ_LD 2
#endif
#ifndef QOQ_SD
#define QOQ_SD 4
#endif
#ifndef QOQ_LDA
#define QOQ_LDA 2
#endif
#ifndef QOQ_AF_PIN
#define QOQ_AF_PIN 0
#endif
#ifndef QOQ_SDA
#define QOQ_SDA 2
#endif
// 128x128 tile: WM x WN waves, each TM x TN tiles of 32x32
#ifndef QOQ_SWM
#define QOQ_SWM 2
#endif
#ifndef QOQ_SWN
#define QOQ_SWN 4
#endif
#ifndef QOQ_STM
#define QOQ_STM 2
#endif
#ifndef QOQ_STN
#define QOQ_STN 1
#endif
static_assert(QOQ_SWM * QOQ_STM * 32 == 128 && QOQ_SWN * QOQ_STN * 32 == 128, "the small large-M tile is 128x128");

namespace qoq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
// 128-bit payloads are native vectors (HIP's u32x4 is a struct whose copies
// lower to memcpy through scratch).
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Raw buffer access.  A buffer descriptor bounds every load by its byte
// count: a load whose offset lies past it returns zeros without a memory
// access.  Prefetch rounds use that to stay straight-line at the end of a K
// range: a load of a group past the range is issued with an offset beyond the
// descriptor and costs no HBM traffic.
constexpr int kBufDword3 = 0x00020000;    // raw 32-bit access, gfx9 family
constexpr int kDeadOffset = 0x40000000;   // past any descriptor built here
constexpr int kCacheStream = 2;           // nt: streamed once, do not keep in cache

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), bytes, kBufDword3);
}

template <int AUX>
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX);
}
// Same, with a wave-uniform part of the offset in an SGPR (soffset).  Callers
// keep every byte that the descriptor's bound must catch in the per-lane
// offset and only offsets known to stay inside the buffer in soffset.
template <int AUX>
__device__ __forceinline__ u32x4 buf_load16s(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, AUX);
}
__device__ __forceinline__ uint32_t buf_load4s(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}

// Packed 16-bit lanes, written as vector arithmetic (selected as v_pk_mad_u16
// and friends) so that the scheduler sees ordinary VALU instructions.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pk_mad_u16(uint32_t a, uint32_t b, uint32_t c) {
  const u16x2 r = __builtin_bit_cast(u16x2, a) * __builtin_bit_cast(u16x2, b) + __builtin_bit_cast(u16x2, c);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ uint32_t pk_mad_i16(uint32_t a, uint32_t b, uint32_t c) {
  const i16x2 r = __builtin_bit_cast(i16x2, a) * __builtin_bit_cast(i16x2, b) + __builtin_bit_cast(i16x2, c);
  return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ uint32_t pk_max_i16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(i16x2, a), __builtin_bit_cast(i16x2, b)));
}
__device__ __forceinline__ uint32_t pk_min_i16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(i16x2, a), __builtin_bit_cast(i16x2, b)));
}

// Two packed words (16 codes) -> one 16-byte INT8 MFMA operand.
__device__ __forceinline__ v4i dequant16(uint32_t v0, uint32_t v1, uint32_t S, uint32_t C) {
  v4i r;
  r[0] = int(pk_mad_u16(v0 & 0x0f0f0f0fu, S, C) ^ 0x80808080u);
  r[1] = int(pk_mad_u16((v0 >> 4) & 0x0f0f0f0fu, S, C) ^ 0x80808080u);
  r[2] = int(pk_mad_u16(v1 & 0x0f0f0f0fu, S, C) ^ 0x80808080u);
  r[3] = int(pk_mad_u16((v1 >> 4) & 0x0f0f0f0fu, S, C) ^ 0x80808080u);
  return r;
}

// Saturating form of dequant16 (ablation): every code gets a 16-bit lane,
// t = q4*s1 + (128 - z*s1) is clamped to [0, 255] and the bytes are packed
// back, XOR 0x80 giving clamp((q4 - z)*s1, -128, 127).  C holds the signed
// 16-bit 128 - z*s1 in both lanes, so no bound on z*s1 is assumed.  Same
// output bytes as dequant16 wherever that one is exact.
__device__ __forceinline__ uint32_t sat_lanes(uint32_t e, uint32_t S, uint32_t C) {
  return pk_min_i16(pk_max_i16(pk_mad_i16(e, S, C), 0u), 0x00ff00ffu);
}
__device__ __forceinline__ void dequant_word_sat(uint32_t v, uint32_t S, uint32_t C, int& even, int& odd) {
  // 16-bit lanes of codes (0,4) and (2,6) give the bytes of codes 0,2,4,6;
  // lanes (1,5) and (3,7) those of 1,3,5,7 -- the byte order of dequant16
  even = int((sat_lanes(v & 0x000f000fu, S, C) | (sat_lanes((v >> 8) & 0x000f000fu, S, C) << 8)) ^ 0x80808080u);
  odd = int((sat_lanes((v >> 4) & 0x000f000fu, S, C) | (sat_lanes((v >> 12) & 0x000f000fu, S, C) << 8)) ^ 0x80808080u);
}
__device__ __forceinline__ v4i dequant16_sat(uint32_t v0, uint32_t v1, uint32_t S, uint32_t C) {
  int e0, o0, e1, o1;
  dequant_word_sat(v0, S, C, e0, o0);
  dequant_word_sat(v1, S, C, e1, o1);
  return v4i{e0, o0, e1, o1};
}

// Weight formats the kernels are instantiated for.
constexpr int kWfG128 = 0;
constexpr int kWfPerChannel = 1;
constexpr int kWfW8 = 2;
constexpr int kWfG128Sat = 3;
// formats with a metadata byte per (channel, group)
constexpr bool wf_group_meta(int wf) { return wf == kWfG128 || wf == kWfG128Sat; }
// bytes of one (16-channel strip, 128-wide group) block, and 16-byte loads
// per lane of a wave reading one such block
constexpr int wf_block_bytes(int wf) { return wf == kWfW8 ? 2048 : 1024; }
constexpr int wf_vec(int wf) { return wf == kWfW8 ? 2 : 1; }

// Metadata byte -> (S, C) operands of the dequantization.
template <int WF>
__device__ __forceinline__ void meta_g128(uint32_t mbyte, uint32_t& S, uint32_t& C) {
  const uint32_t s1 = (mbyte & 15u) + 1u;
  const uint32_t z = mbyte >> 4;
  const uint32_t c = 128u - z * s1;
  S = s1 * 0x00010001u;
  // Packed metadata keeps c = u(q4 = 0) within [7, 249] (the protective
  // range), so replicating its low byte (one v_perm_b32) equals
  // c * 0x01010101 without the quarter-rate 32-bit multiply.
  C = WF == kWfG128Sat ? (c & 0xffffu) * 0x00010001u : __builtin_amdgcn_perm(0u, c, 0u);
}
__device__ __forceinline__ void meta_perchannel(uint32_t z, uint32_t& S, uint32_t& C) {
  S = 0x00010001u;
  C = (128u - z) * 0x01010101u;
}

// 16x16x64 B operand h (K 0-63 or 64-127 of the group) of one lane, from
// that lane's loads of one (strip, group) block.
template <int WF>
__device__ __forceinline__ v4i b_op16(const u32x4 (&q)[wf_vec(WF)], int h, uint32_t S, uint32_t C) {
  if constexpr (WF == kWfW8) {
    return __builtin_bit_cast(v4i, q[h]);
  } else if constexpr (WF == kWfG128Sat) {
    return dequant16_sat(h ? q[0][2] : q[0][0], h ? q[0][3] : q[0][1], S, C);
  } else {
    return dequant16(h ? q[0][2] : q[0][0], h ? q[0][3] : q[0][1], S, C);
  }
}

// LDS tile of BM rows x 128 bytes; 16-byte chunk kc of row r lives at chunk
// kc ^ ((r >> 1) & 7).  A 128-byte row spans half of the 64 four-byte banks,
// so rows of equal parity share a bank half; XOR-ing with r >> 1 spreads 16
// consecutive rows reading the same K chunk over all 64 banks.
__device__ __forceinline__ int lds_off(int row, int kc) { return row * 128 + ((kc ^ ((row >> 1) & 7)) << 4); }

// Keeps prefetch loads where they are written: the empty asm with a memory
// clobber stops IR passes from sinking loads toward their uses, and the
// scheduling barrier stops the machine scheduler from doing the same.
#define QOQ_COMPILER_FENCE()          \
  do {                                \
    asm volatile("" ::: "memory");    \
    __builtin_amdgcn_sched_barrier(0); \
  } while (0)

struct GemmArgs {
  const int8_t* x8;
  const unsigned short* sx;
  const u32x4* qw;
  const uint32_t* meta;  // g128: dwords; per-channel: bytes read through meta8
  const uint8_t* meta8;
  const unsigned short* scale;
  void* out;
  int M, N, G, G4q;  // G4q = G4 / 4 (meta dwords per strip per channel)
  int n_strips;
  int64_t ldo;
  int ksplit;        // K splits (grid.z); > 1 writes INT32 partials
  int64_t zstride;   // element offset between the partials of two splits
};

// Epilogue scales.  Every scale an epilogue needs is loaded before its first
// store: the output may alias the scale arrays as far as the compiler knows,
// so a scale loaded between stores would wait for each of them in turn.
__device__ __forceinline__ float col_scale(const GemmArgs& a, int col) {
  return col < a.N ? __half2float(__ushort_as_half(a.scale[col])) : 0.0f;
}
__device__ __forceinline__ float row_scale(const GemmArgs& a, int row) {
  return row < a.M ? __half2float(__ushort_as_half(a.sx[row])) : 0.0f;
}

template <bool I32OUT>
__device__ __forceinline__ void store_out(const GemmArgs& a, int row, int col, int acc, float sxr, float sc) {
  if (row < a.M && col < a.N) {
    if constexpr (I32OUT) {
      static_cast<int*>(a.out)[int64_t(blockIdx.z) * a.zstride + int64_t(row) * a.ldo + col] = acc;
    } else {
      const float y = static_cast<float>(acc) * sxr * sc;
      static_cast<__half*>(a.out)[int64_t(row) * a.ldo + col] = __float2half_rn(y);
    }
  }
}

// ---------------------------------------------------------------------------
// skinny: M <= 64 (decode), and up to 256 rows when one round of blocks
// covers the problem.  A block is KS waves that split the K groups of the
// same TN strips between them, so every wave streams different weight bytes.
// Each wave passes its activations (whole 128-byte rows, shared by all blocks
// and mostly served from L2) through a wave-private LDS buffer into the MFMA
// operand layout, and streams its weights through a PF-deep register ring of
// 128-bit loads so that enough bytes are in flight to cover HBM latency.  The
// KS partial INT32 accumulators are summed exactly through LDS at the end.
template <int TM, int TN, int KS, int PF, int AD, int WF, bool I32OUT>
__global__ __launch_bounds__(64 * KS) void gemm_skinny_kernel(GemmArgs a) {
  static_assert(PF % AD == 0 && PF % 2 == 0, "the activation ring and the LDS ping-pong must tile the weight ring");
  // LDS: while multiplying, each wave stages its own activations in two
  // buffers of TM*16 rows x 128 B; afterwards the same memory holds the
  // partial sums of every wave, [KS][TN][TM][64 lanes] records of 4 INT32.
  constexpr int kStageBytes = 2 * TM * 16 * 128;
  constexpr int kRedBytes = KS > 1 ? KS * TN * TM * 4 * 64 * 4 : 0;
  constexpr int kSmemBytes = KS * kStageBytes > kRedBytes ? KS * kStageBytes : kRedBytes;
  __shared__ __align__(16) int8_t smem[kSmemBytes];
  // wave-uniform by construction; readfirstlane lets the compiler keep
  // everything derived from it (K range, group indices) in SGPRs
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // (S, C) dequantization operands of every metadata byte, filled once per
  // block: one LDS lookup replaces the per-(strip, group) decode arithmetic
  __shared__ uint2 mtab[wf_group_meta(WF) ? 256 : 1];
  if constexpr (wf_group_meta(WF)) {
    for (int e = threadIdx.x; e < 256; e += 64 * KS) {
      uint32_t s0, c0;
      meta_g128<WF>(uint32_t(e), s0, c0);
      mtab[e] = make_uint2(s0, c0);
    }
    __syncthreads();
  }
  int8_t* stage = smem + wave * kStageBytes;
  const int c16 = lane & 15, j = lane >> 4;
  const int sbase = blockIdx.x * TN;
  const int m0 = blockIdx.y * TM * 16;
  const int64_t K = int64_t(a.G) * 128;
  const int g0 = (a.G * wave) / KS, g1 = (a.G * (wave + 1)) / KS;

  int strip[TN];
#pragma unroll
  for (int t = 0; t < TN; ++t) strip[t] = min(sbase + t, a.n_strips - 1);

  constexpr int kVec = wf_vec(WF);
  uint32_t S[TN] = {}, C[TN] = {};
  if constexpr (WF == kWfPerChannel) {
#pragma unroll
    for (int t = 0; t < TN; ++t) meta_perchannel(a.meta8[strip[t] * 16 + c16], S[t], C[t]);
  }

  v4i acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int t = 0; t < TN; ++t) acc[i][t] = v4i{0, 0, 0, 0};

  u32x4 bq[PF][TN][kVec];
  uint32_t mq[PF][TN];
  u32x4 aq[AD][TM][2];

  // The block's strips are contiguous in the packed weights.  Every load's
  // per-lane offset is the same loop-invariant lane * 16; the group moves the
  // descriptor's base and the strip is a wave-uniform soffset, so a round of
  // loads costs no vector ALU work.  The strip index in soffset is clamped to
  // the last valid strip (a ragged last block re-reads it; its columns are
  // never stored), and a group past this wave's K range gets a descriptor of
  // size zero: its loads return zeros without touching memory.
  constexpr int kBlk = wf_block_bytes(WF);
  const int strip_bytes = a.G * kBlk;
  const int nvalid = min(TN, a.n_strips - sbase);
  const int8_t* wbase = reinterpret_cast<const int8_t*>(a.qw) + int64_t(sbase) * strip_bytes;
  auto load_b = [&](int g, u32x4 (&b)[TN][kVec], uint32_t (&m)[TN]) {
    const bool live = g < g1;
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(wbase + (live ? g : 0) * kBlk, live ? nvalid * strip_bytes : 0);
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      // weights are streamed once per call: non-temporal loads
#pragma unroll
      for (int v = 0; v < kVec; ++v)
        b[t][v] = buf_load16s<kCacheStream>(wr, lane * 16 + v * 1024, min(t, nvalid - 1) * strip_bytes);
    }
    if constexpr (wf_group_meta(WF)) {
      // metadata dword of the group's 4-group run (clamped into the range)
      const int gm = min(g, g1 - 1);
      const int8_t* mbase = reinterpret_cast<const int8_t*>(a.meta) + (int64_t(sbase) * a.G4q + (gm >> 2)) * 64;
      const __amdgpu_buffer_rsrc_t mr = make_rsrc(mbase, nvalid * a.G4q * 64);
#pragma unroll
      for (int t = 0; t < TN; ++t) m[t] = buf_load4s(mr, c16 * 4, min(t, nvalid - 1) * a.G4q * 64);
    }
  };
  // Activations are read in whole 128-byte rows: one load covers 8 rows x one
  // group (lane l: row l/8, chunk l%8), so every cache line it touches is
  // used in full (loads in the MFMA operand layout would touch 16 half-used
  // lines each).  The descriptor covers the block's valid rows; rows past M
  // and groups past this wave's range read zeros without touching memory.
  // As for the weights, the group moves the descriptor's base (a group past
  // the range gets an empty descriptor); rows past M have a per-lane offset
  // beyond the descriptor.
  const int ar8 = lane >> 3, aq8 = lane & 7;
  const int8_t* xbase = a.x8 + int64_t(m0) * K;
  const int xbytes = int(min(TM * 16, a.M - m0) * K);
  int arow[TM][2];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int rl = 16 * i + 8 * hh + ar8;
      arow[i][hh] = m0 + rl < a.M ? int(rl * K) + 16 * aq8 : kDeadOffset;
    }
  auto load_a = [&](int g, u32x4 (&ar)[TM][2]) {
    const bool live = g < g1;
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(xbase + (live ? g : 0) * 128, live ? xbytes : 0);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) ar[i][hh] = buf_load16<0>(xr, arow[i][hh]);
  };
  // Into this wave's LDS buffer (chunk-XOR swizzled, conflict-free both
  // ways), to be read back in the MFMA A layout: lane (c16, j) takes row c16
  // of tile i, K chunk j (+4 for the second 64-wide step).  A wave reads only
  // what it wrote, and LDS operations of one wave complete in order, so no
  // barrier is involved.
  auto stage_a = [&](const u32x4 (&ar)[TM][2], int buf) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        *reinterpret_cast<u32x4*>(stage + buf * (TM * 16 * 128) + lds_off(16 * i + 8 * hh + ar8, aq8)) = ar[i][hh];
  };

  // Multiply group g: its activations come out of LDS buffer (g - g0) % 2,
  // read here so that the fragments are live only while they are used.
  auto compute = [&](int g, const u32x4 (&bc)[TN][kVec], const uint32_t (&mc)[TN]) {
    v4i af[TM][2];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        af[i][h] = *reinterpret_cast<const v4i*>(stage + ((g - g0) & 1) * (TM * 16 * 128) + lds_off(16 * i + c16, j + 4 * h));
    if constexpr (wf_group_meta(WF)) {
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        const uint2 e = mtab[(mc[t] >> (8 * (g & 3))) & 0xffu];
        S[t] = e.x;
        C[t] = e.y;
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        const v4i bf = b_op16<WF>(bc[t], h, S[t], C[t]);
#pragma unroll
        for (int i = 0; i < TM; ++i) acc[i][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[i][h], bf, acc[i][t], 0, 0, 0);
      }
    }
  };

  // Epilogue scales, loaded once the prologue's loads are in flight so that
  // their latency hides behind the main loop (global loads retire in order,
  // so no wait of the loop is held up by them): row scales of the lane's
  // rows and column scales of the strips this wave stores.
  // The raw FP16 bits are kept (addresses clamped into range, so there is no
  // select on the loaded values) and converted only in the epilogue.
  constexpr int kScN = KS > 1 ? (TN + KS - 1) / KS : TN;
  unsigned short sxh[TM][4] = {}, sch[kScN] = {};
  auto load_scales = [&]() {
    if constexpr (!I32OUT) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) sxh[i][r] = a.sx[min(m0 + i * 16 + 4 * j + r, a.M - 1)];
#pragma unroll
      for (int u = 0; u < kScN; ++u) {
        const int t = min(KS > 1 ? wave + u * KS : u, TN - 1);
        sch[u] = a.scale[min((sbase + t) * 16 + c16, a.N - 1)];
      }
    }
  };
  auto fp16 = [](unsigned short h) { return __half2float(__ushort_as_half(h)); };

  const int ng = g1 - g0;
  if (ng <= 0) load_scales();
  if (ng > 0) {
    // prologue: activations of the first AD groups, then weights of the first
    // PF (loads retire in order: the first multiply waits only for what was
    // issued before its operands); group g0 goes into LDS right away.
#pragma unroll
    for (int p = 0; p < AD; ++p) load_a(g0 + p, aq[p]);
#pragma unroll
    for (int p = 0; p < PF; ++p) load_b(g0 + p, bq[p], mq[p]);
    stage_a(aq[0], 0);
    load_a(g0 + AD, aq[0]);
    QOQ_COMPILER_FENCE();
    load_scales();

    // full rounds of PF groups.  Loads are unconditional (past the range they
    // read zeros for free) so a round is straight-line code.  Step l: multiply
    // group g0+l (weights from ring slot l % PF, activations already in
    // registers from LDS buffer l % 2); then pass group l+1 through the other
    // LDS buffer and refill both rings, the weights PF groups ahead and the
    // activations AD + 1 ahead.  Loads retire in issue order, so the
    // activation lookahead also bounds how far ahead the weights effectively
    // run.
    int it = 0;
    for (; it + PF <= ng; it += PF) {
#pragma unroll
      for (int u = 0; u < PF; ++u) {
        const int g = g0 + it + u;
        compute(g, bq[u], mq[u]);
        QOQ_COMPILER_FENCE();
        stage_a(aq[(u + 1) % AD], (u + 1) & 1);
        load_b(g + PF, bq[u], mq[u]);
        load_a(g + 1 + AD, aq[(u + 1) % AD]);
        QOQ_COMPILER_FENCE();
      }
    }
    // remaining ng % PF groups: weights are in bq[0 .. rem), the activations
    // of the next ones in the activation ring
    const int rem = ng - it;
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      if (u < rem) {
        const int g = g0 + it + u;
        compute(g, bq[u], mq[u]);
        if (u + 1 < rem) {
          stage_a(aq[(u + 1) % AD], (u + 1) & 1);
          if (u + 1 + AD < rem) load_a(g + 1 + AD, aq[(u + 1) % AD]);
        }
      }
    }
  }

  // Exact cross-wave reduction of the K-split partial sums, and the epilogue.
  // Once every wave is done with its activation buffers, every wave parks its
  // partials in the same LDS; after a second barrier wave w sums and stores
  // strips w, w+KS, ... (lane holds rows 4*(lane/16)+r of each 16x16
  // tile, column lane%16).  The scales were loaded before the main loop.
  if constexpr (KS > 1) {
    __syncthreads();  // every wave is done with its activation buffers
    // [wave][strip][row tile][lane] 16-byte records: one 128-bit LDS write
    // per accumulator tile and one 128-bit read per partial
    v4i* red4 = reinterpret_cast<v4i*>(smem);
#pragma unroll
    for (int t = 0; t < TN; ++t)
#pragma unroll
      for (int i = 0; i < TM; ++i) red4[((wave * TN + t) * TM + i) * 64 + lane] = acc[i][t];
    __syncthreads();
#pragma unroll
    for (int u = 0; u < (TN + KS - 1) / KS; ++u) {
      const int t = wave + u * KS;
      if (t < TN && sbase + t < a.n_strips) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          v4i v = red4[(t * TM + i) * 64 + lane];
#pragma unroll
          for (int w = 1; w < KS; ++w) v += red4[((w * TN + t) * TM + i) * 64 + lane];
#pragma unroll
          for (int r = 0; r < 4; ++r)
            store_out<I32OUT>(a, m0 + i * 16 + 4 * j + r, (sbase + t) * 16 + c16, v[r], fp16(sxh[i][r]), fp16(sch[u]));
        }
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int t = 0; t < TN; ++t)
          if (sbase + t < a.n_strips)
            store_out<I32OUT>(a, m0 + i * 16 + 4 * j + r, (sbase + t) * 16 + c16, acc[i][t][r], fp16(sxh[i][r]), fp16(sch[t]));
  }
}

// ---------------------------------------------------------------------------
// strip: up to 16 rows (decode, memory-bound).  Every wave streams one
// 16-channel strip over its K range -- the strip's packed bytes are one
// contiguous run, and HBM serves a few long runs far better than many short
// interleaved ones -- with PF groups of 128-bit loads in flight.  The INT8
// activations of the block's rows (at most 16 x K bytes) are copied into LDS
// once, with direct-to-LDS loads issued before the weight stream starts, and
// every wave reads its MFMA A operand from there.  The weights are then the
// only global loads of the main loop: global loads retire in issue order, so
// any other global load would hold the weight stream back.  A block is `spb`
// strips x `ks` K parts; the parts are summed exactly through LDS at the end.
//
// LDS activation layout: [group][row][128 B], 16-byte chunk q of LDS row
// L = g*R + r stored at chunk q ^ ((L >> 1) & 7) (16 rows reading the same
// chunk hit all 64 banks).
__device__ __forceinline__ int round_up_lds(int bytes) { return (bytes + 1023) & ~1023; }
__device__ __forceinline__ int strip_lds_off(int lrow, int q) { return lrow * 128 + ((q ^ ((lrow >> 1) & 7)) << 4); }

// s_waitcnt immediates (gfx9 encoding): wait until at most n vector-memory
// operations of this wave are outstanding, leaving the other counters free.
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

template <int PF, int WF, bool I32OUT>
__global__ __launch_bounds__(512) void gemm_strip_kernel(GemmArgs a, int spb, int ks) {
  extern __shared__ __align__(16) int8_t smem[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int nwaves = blockDim.x >> 6;
  const int ws = wave / ks, wk = wave - ws * ks;
  const int sb = blockIdx.x * spb;
  const int strip = sb + ws;
  const bool live = strip < a.n_strips;
  const int cstrip = min(strip, a.n_strips - 1);
  const int c16 = lane & 15, j = lane >> 4;
  const int64_t K = int64_t(a.G) * 128;
  const int R = min(a.M, 16);
  const int g0 = (a.G * wk) / ks, g1 = (a.G * (wk + 1)) / ks, ng = g1 - g0;

  constexpr int kVec = wf_vec(WF);
  uint32_t S = 0, C = 0;
  if constexpr (WF == kWfPerChannel) meta_perchannel(a.meta8[cstrip * 16 + c16], S, C);

  // activations -> LDS.  Lane l of a wave-wide copy fills LDS chunk base + l;
  // lanes past the end fetch a valid chunk into the allocation's padding.
  const int n_chunks = a.G * R * 8;
  for (int base = wave * 64; base < n_chunks; base += nwaves * 64) {
    const int pc = min(base + lane, n_chunks - 1);
    const int lrow = pc >> 3;
    const int q = (pc & 7) ^ ((lrow >> 1) & 7);
    const int g = lrow / R, r = lrow - g * R;
    __builtin_amdgcn_global_load_lds(static_cast<const void*>(a.x8 + int64_t(r) * K + int64_t(g) * 128 + q * 16),
                                     (__attribute__((address_space(3))) void*)(smem + base * 16), 16, 0, 0);
  }
  // group metadata of the block's strips -> LDS, after the activations (the
  // strips' metadata is one contiguous run of G4q * 64 bytes per strip)
  const int act_bytes = round_up_lds(n_chunks * 16);
  if constexpr (wf_group_meta(WF)) {
    const int m_chunks = min(spb, a.n_strips - sb) * a.G4q * 4;
    const int8_t* msrc = reinterpret_cast<const int8_t*>(a.meta) + int64_t(sb) * a.G4q * 64;
    for (int base = wave * 64; base < m_chunks; base += nwaves * 64) {
      const int pc = min(base + lane, m_chunks - 1);
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(msrc + pc * 16),
                                       (__attribute__((address_space(3))) void*)(smem + act_bytes + base * 16), 16, 0, 0);
    }
  }
  const uint32_t* lmeta = reinterpret_cast<const uint32_t*>(smem + act_bytes) + ws * a.G4q * 16 + c16;

  // weights: one descriptor over this wave's strip (empty past N), PF groups
  // in flight from here on
  constexpr int kBlk = wf_block_bytes(WF);
  const int strip_bytes = a.G * kBlk;
  const __amdgpu_buffer_rsrc_t wrs =
      make_rsrc(reinterpret_cast<const int8_t*>(a.qw) + int64_t(cstrip) * strip_bytes, live ? strip_bytes : 0);
  u32x4 bq[PF][kVec];
  auto load_b = [&](int g, u32x4 (&b)[kVec]) {
#pragma unroll
    for (int v = 0; v < kVec; ++v) b[v] = buf_load16<kCacheStream>(wrs, lane * 16 + v * 1024 + (g < g1 ? g * kBlk : kDeadOffset));
  };
  // Wait for this wave's direct-to-LDS copies only (they were issued before
  // the weight loads, and loads retire in order), then meet the other waves.
  // A plain __syncthreads would also wait for the PF weight loads and drain
  // the HBM stream once before the first multiply.  The prologue is
  // unconditional (a wave with an empty K range loads zeros for free) so the
  // main loop is entered on a single path.
#pragma unroll
  for (int p = 0; p < PF; ++p) load_b(g0 + p, bq[p]);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(PF * kVec));
  __builtin_amdgcn_s_barrier();
  QOQ_COMPILER_FENCE();

  const int ra = c16 < R ? c16 : 0;  // rows past M reuse row 0; they are never stored
  v4i acc = {0, 0, 0, 0};
  auto compute = [&](int g, const u32x4 (&bc)[kVec]) {
    if constexpr (wf_group_meta(WF)) meta_g128<WF>((lmeta[(g >> 2) * 16] >> (8 * (g & 3))) & 0xffu, S, C);
    const int lrow = g * R + ra;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const v4i af = *reinterpret_cast<const v4i*>(smem + strip_lds_off(lrow, j + 4 * h));
      const v4i bf = b_op16<WF>(bc, h, S, C);
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(af, bf, acc, 0, 0, 0);
    }
  };
  auto round = [&](int it) {
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const int g = g0 + it + u;
      compute(g, bq[u]);
      QOQ_COMPILER_FENCE();
      load_b(g + PF, bq[u]);
      QOQ_COMPILER_FENCE();
    }
  };
  // The first round is peeled: the loop is then entered in the same state as
  // its back edge (PF weight loads in flight, nothing else), which lets the
  // compiler wait for one group at a time instead of draining every round.
  int it = 0;
  if (ng >= PF) {
    round(0);
    for (it = PF; it + PF <= ng; it += PF) round(it);
  }
  const int rem = ng - it;
#pragma unroll
  for (int u = 0; u < PF; ++u) {
    if (u < rem) compute(g0 + it + u, bq[u]);
  }

  // exact sum of the K parts (the activations in LDS are no longer needed)
  if (ks > 1) {
    __syncthreads();
    int* red = reinterpret_cast<int*>(smem);
    if (wk > 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) red[((ws * (ks - 1) + wk - 1) * 4 + r) * 64 + lane] = acc[r];
    }
    __syncthreads();
    if (wk == 0) {
      for (int w = 1; w < ks; ++w)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] += red[((ws * (ks - 1) + w - 1) * 4 + r) * 64 + lane];
    }
  }
  if (wk != 0 || !live) return;

  // epilogue: lane holds rows 4*(lane/16)+r, column lane%16 of the strip
  const float sc = I32OUT ? 0.0f : col_scale(a, strip * 16 + c16);
  float sxv[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) sxv[r] = I32OUT ? 0.0f : row_scale(a, 4 * j + r);
#pragma unroll
  for (int r = 0; r < 4; ++r) store_out<I32OUT>(a, 4 * j + r, strip * 16 + c16, acc[r], sxv[r], sc);
}

// ---------------------------------------------------------------------------
// gemm_large: M > 64 (prefill, compute-bound).  Block = WM x WN waves, wave
// tile = TM*32 rows x TN*32 columns of v_mfma_i32_32x32x32_i8.  The K loop is
// unrolled by two with explicit ping-pong register buffers: while group g is
// multiplied from LDS buffer g&1 and weight registers set g&1, the activation
// chunks and packed weights of group g+1 are already in flight into the other
// set, and are written to the other LDS buffer after the MFMAs.  There are no
// loop-carried register copies, so every wait is for data that is actually
// needed next.
template <int BM, int THREADS>
struct ATile {
  static constexpr int kChunks = BM * 8;
  static constexpr int kPer = kChunks / THREADS;
  static_assert(kChunks % THREADS == 0, "A tile must split evenly over the block");
};

template <int NA, int THREADS>
__device__ __forceinline__ void a_store(const u32x4 (&r)[NA], int8_t* lds) {
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int ch = threadIdx.x + i * THREADS;
    *reinterpret_cast<u32x4*>(lds + lds_off(ch >> 3, ch & 7)) = r[i];
  }
}

// 16-byte weight loads per lane, per 32-column tile and group: UINT4 slots
// (c16, hh) and (c16, 2+hh) hold K steps {0, 2} and {1, 3}; INT8 slots hold
// one K step each.
constexpr int wf_large_vec(int wf) { return wf == kWfW8 ? 4 : 2; }

// 32x32x32 B operand of K step s from one lane's loads of a group.
template <int WF>
__device__ __forceinline__ v4i b_op32(const u32x4 (&b)[wf_large_vec(WF)], int s, uint32_t S, uint32_t C) {
  if constexpr (WF == kWfW8) {
    return __builtin_bit_cast(v4i, b[s]);
  } else {
    const u32x4& q = b[s & 1];
    if constexpr (WF == kWfG128Sat) return dequant16_sat((s >> 1) ? q[2] : q[0], (s >> 1) ? q[3] : q[1], S, C);
    else return dequant16((s >> 1) ? q[2] : q[0], (s >> 1) ? q[3] : q[1], S, C);
  }
}

// Multiply one 128-wide K group: 4 K steps of 32.  Weight slot 0 of a column
// tile holds K steps 0 and 2 (low / high half), slot 1 holds steps 1 and 3.
template <int TM, int TN, int WF>
__device__ __forceinline__ void large_group(v16i (&acc)[TM][TN], const int8_t* lds,
                                            const u32x4 (&b)[TN][wf_large_vec(WF)], const uint32_t (&m)[TN],
                                            uint32_t (&S)[TN], uint32_t (&C)[TN], int g, int row0, int c32, int hh) {
  if constexpr (wf_group_meta(WF)) {
#pragma unroll
    for (int t = 0; t < TN; ++t) meta_g128<WF>((m[t] >> (8 * (g & 3))) & 0xffu, S[t], C[t]);
  }
  // A fragments are double-buffered across the 4 K steps: the reads of step
  // s+1 are issued before the multiplies of step s, so LDS latency hides
  // behind them.
  v4i af[2][TM];
#pragma unroll
  for (int i = 0; i < TM; ++i) af[0][i] = *reinterpret_cast<const v4i*>(lds + lds_off(row0 + i * 32 + c32, hh));
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    if (s + 1 < 4) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[(s + 1) & 1][i] = *reinterpret_cast<const v4i*>(lds + lds_off(row0 + i * 32 + c32, 2 * (s + 1) + hh));
    }
#if QOQ_AF_PIN
    __builtin_amdgcn_sched_barrier(0);
#endif
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      const v4i bf = b_op32<WF>(b[t], s, S[t], C[t]);
#pragma unroll
      for (int i = 0; i < TM; ++i) acc[i][t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[s & 1][i], bf, acc[i][t], 0, 0, 0);
    }
  }
}


template <int WM, int WN, int TM, int TN, int D, int DA, int WF, bool I32OUT>
__global__ __launch_bounds__(64 * WM * WN) void gemm_large_kernel(GemmArgs a) {
  static_assert(D % 2 == 0, "ring depth must be even (LDS ping-pong parity)");
  static_assert(D % DA == 0, "the activation ring must tile the weight ring");
  constexpr int THREADS = 64 * WM * WN;
  constexpr int BM = WM * TM * 32;
  constexpr int BN = WN * TN * 32;
  constexpr int NA = ATile<BM, THREADS>::kPer;
  __shared__ __align__(16) int8_t As0[BM * 128];
  __shared__ __align__(16) int8_t As1[BM * 128];

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WN, wn = wave % WN;
  // Tile order.  Workgroups are dispatched round-robin over the 8 XCDs, each
  // with its own L2.  Remap so that each XCD gets a contiguous run of tiles,
  // and walk that run in bands of up to 8 row tiles, column by column, so the
  // blocks resident on one XCD at a time cover a compact patch of the output
  // and share both their activation rows and their packed weight columns.
  const int ny = gridDim.y;
  const int nb = gridDim.x * ny;
  int d = blockIdx.y * gridDim.x + blockIdx.x;
  if (d < (nb / 8) * 8) d = (d % 8) * (nb / 8) + d / 8;
  constexpr int kBand = 8;
  const int band = d / (kBand * int(gridDim.x));
  const int band_rows = min(kBand, ny - band * kBand);
  const int in_band = d - band * kBand * int(gridDim.x);
  const int m0 = (band * kBand + in_band % band_rows) * BM;
  const int n0 = (in_band / band_rows) * BN + wn * TN * 32;  // first column of this wave
  const int64_t K = int64_t(a.G) * 128;
  const int c32 = lane & 31, hh = lane >> 5;
  const int c16 = c32 & 15;
  const int row0 = wm * TM * 32;
  // K range of this split (every split holds at least one group)
  const int gb = (a.G * int(blockIdx.z)) / a.ksplit;
  const int ge = (a.G * (int(blockIdx.z) + 1)) / a.ksplit;

  int strip[TN];
#pragma unroll
  for (int t = 0; t < TN; ++t) strip[t] = min((n0 + 32 * t + c32) >> 4, a.n_strips - 1);

  uint32_t S[TN] = {}, C[TN] = {};
  if constexpr (WF == kWfPerChannel) {
#pragma unroll
    for (int t = 0; t < TN; ++t) meta_perchannel(a.meta8[strip[t] * 16 + c16], S[t], C[t]);
  }

  v16i acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int t = 0; t < TN; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][t][e] = 0;

  // Register rings.  Weights: D slots, slot l % D holds the packed weights of
  // group gb+l, refilled right after use, D groups ahead.  Activations: DA
  // slots; at the start of step l the chunks of group gb+l+1 are written to
  // the LDS buffer not being read (every wave passed the previous barrier),
  // and the slot is refilled DA groups ahead.  LDS is double-buffered by
  // group parity.  Loads retire in issue order, so a step waits for the
  // activations loaded DA steps earlier: DA steps of work must cover the
  // load latency.
  u32x4 ra[DA][NA];
  u32x4 rb[D][TN][wf_large_vec(WF)];
  uint32_t rm[D][TN];
  const int n = ge - gb;
  auto gcl = [&](int l) { return gb + min(l, n - 1); };

  // Global loads go through buffer descriptors: the per-lane offsets below
  // are loop-invariant and the group is a wave-uniform soffset, so a round of
  // loads costs no vector ALU work.  Every offset is clamped into the
  // operands (rows past M read row M-1, strips past N the last strip, and
  // groups past the range the last group), so no load leaves its buffer.
  // Activations: chunk ch of the tile is row ch / 8, 16-byte chunk ch % 8.
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x8 + int64_t(m0) * K, int(min(BM, a.M - m0) * K));
  int aoff[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int ch = threadIdx.x + i * THREADS;
    aoff[i] = (min(m0 + (ch >> 3), a.M - 1) - m0) * int(K) + (ch & 7) * 16;
  }
  auto a_ld = [&](u32x4 (&r)[NA], int g) {
#pragma unroll
    for (int i = 0; i < NA; ++i) r[i] = buf_load16s<0>(xr, aoff[i], g * 128);
  };
  // Weights and group metadata: one descriptor over the (at most 2 TN)
  // strips of this wave's columns.  UINT4 blocks: lane (c32, hh) loads slots
  // c16 + 16 hh and c16 + 16 (2 + hh), K steps {0, 2} and {1, 3}; INT8 blocks:
  // K step st is K chunk 2 st + hh = 16 j + 64 h, slot c16 + 16 j + 64 h.
  constexpr int kBlk = wf_block_bytes(WF);
  constexpr int kVec = wf_large_vec(WF);
  const int sfirst = min(n0 >> 4, a.n_strips - 1);
  const int nws = min(2 * TN, a.n_strips - sfirst);
  const __amdgpu_buffer_rsrc_t wr =
      make_rsrc(reinterpret_cast<const int8_t*>(a.qw) + int64_t(sfirst) * a.G * kBlk, nws * a.G * kBlk);
  int woff[TN][kVec];
#pragma unroll
  for (int t = 0; t < TN; ++t) {
    const int sb = (strip[t] - sfirst) * a.G * kBlk;
#pragma unroll
    for (int v = 0; v < kVec; ++v) {
      const int slot = WF == kWfW8 ? c16 + 16 * ((2 * v + hh) & 3) + 64 * ((2 * v + hh) >> 2) : c16 + 16 * (2 * v + hh);
      woff[t][v] = sb + slot * 16;
    }
  }
  // (formats without group metadata get an empty descriptor that is never used)
  const __amdgpu_buffer_rsrc_t mr =
      wf_group_meta(WF)
          ? make_rsrc(reinterpret_cast<const int8_t*>(a.meta) + int64_t(sfirst) * a.G4q * 64, nws * a.G4q * 64)
          : make_rsrc(a.qw, 0);
  int moff[TN];
#pragma unroll
  for (int t = 0; t < TN; ++t) moff[t] = ((strip[t] - sfirst) * a.G4q * 16 + c16) * 4;
  auto b_ld = [&](u32x4 (&b)[TN][kVec], uint32_t (&m)[TN], int g) {
#pragma unroll
    for (int t = 0; t < TN; ++t) {
#pragma unroll
      for (int v = 0; v < kVec; ++v) b[t][v] = buf_load16s<0>(wr, woff[t][v], g * kBlk);
      if constexpr (wf_group_meta(WF)) m[t] = buf_load4s(mr, moff[t], (g >> 2) * 64);
    }
  };

  a_ld(ra[0], gb);
  a_store<NA, THREADS>(ra[0], As0);
#pragma unroll
  for (int d = 1; d <= DA; ++d) a_ld(ra[d % DA], gcl(d));
#pragma unroll
  for (int d = 0; d < D; ++d) b_ld(rb[d], rm[d], gcl(d));
  __syncthreads();

  int l0 = 0;
  for (; l0 + D <= n; l0 += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      const int l = l0 + u;
      a_store<NA, THREADS>(ra[(u + 1) % DA], (u & 1) ? As0 : As1);
      a_ld(ra[(u + 1) % DA], gcl(l + 1 + DA));
      QOQ_COMPILER_FENCE();
      large_group<TM, TN, WF>(acc, (u & 1) ? As1 : As0, rb[u], rm[u], S, C, gb + l, row0, c32, hh);
      __syncthreads();
      b_ld(rb[u], rm[u], gcl(l + D));
      QOQ_COMPILER_FENCE();
    }
  }
  // the last n % D groups are already in the rings
  const int rem = n - l0;
#pragma unroll
  for (int u = 0; u < D; ++u) {
    if (u < rem) {
      if (u + 1 < rem) a_store<NA, THREADS>(ra[(u + 1) % DA], (u & 1) ? As0 : As1);
      large_group<TM, TN, WF>(acc, (u & 1) ? As1 : As0, rb[u], rm[u], S, C, gb + l0 + u, row0, c32, hh);
      __syncthreads();
    }
  }

  // epilogue: lane holds column lane%32 and rows 8*(r/4) + 4*(lane/32) + r%4.
  // Every scale is fetched before the first store: stores count on the same
  // in-order counter as global loads, so a load issued after a store waits
  // for it.  The block's row scales go through LDS (free after the last
  // barrier of the K loop; LDS reads have a counter of their own).
  float sc[TN];
#pragma unroll
  for (int t = 0; t < TN; ++t) sc[t] = I32OUT ? 0.0f : col_scale(a, n0 + 32 * t + c32);
  float* sxs = reinterpret_cast<float*>(As0);
  if constexpr (!I32OUT) {
    for (int r = threadIdx.x; r < BM; r += THREADS) sxs[r] = row_scale(a, m0 + r);
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int lr = row0 + i * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
      const float sxr = I32OUT ? 0.0f : sxs[lr];
#pragma unroll
      for (int t = 0; t < TN; ++t) store_out<I32OUT>(a, m0 + lr, n0 + 32 * t + c32, acc[i][t][r], sxr, sc[t]);
    }
  }
}

// ---------------------------------------------------------------------------
// Split-K reduction: sums the INT32 partials of the K splits (exact, in a
// fixed order) and applies the epilogue.  Partials are [ksplit][M][ldw] with
// ldw a multiple of 16; each thread handles eight consecutive columns: two
// 16-byte loads per split, and one 16-byte FP16 store (or two INT32 ones)
// when the output rows are 16-byte aligned (`vec`).
template <bool I32OUT>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const int* __restrict__ ws, int ksplit, int M, int N,
                                                            int ldw, const unsigned short* __restrict__ sx,
                                                            const unsigned short* __restrict__ scale, void* out,
                                                            int64_t ldo, int vec) {
  const int per_row = ldw / 8;
  const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= int64_t(M) * per_row) return;
  const int row = int(idx / per_row);
  const int col = int(idx % per_row) * 8;
  const int64_t zs = int64_t(M) * ldw;
  const int* p = ws + int64_t(row) * ldw + col;
  v4i s0 = *reinterpret_cast<const v4i*>(p), s1 = *reinterpret_cast<const v4i*>(p + 4);
  for (int z = 1; z < ksplit; ++z) {
    s0 += *reinterpret_cast<const v4i*>(p + z * zs);
    s1 += *reinterpret_cast<const v4i*>(p + z * zs + 4);
  }
  int v[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
  if constexpr (I32OUT) {
    int* o = static_cast<int*>(out) + int64_t(row) * ldo + col;
    if (vec && col + 8 <= N) {
      *reinterpret_cast<v4i*>(o) = s0;
      *reinterpret_cast<v4i*>(o + 4) = s1;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (col + e < N) o[e] = v[e];
    }
  } else {
    // scales before any store: a load issued after a store waits for it
    const float sxr = __half2float(__ushort_as_half(sx[row]));
    float sc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) sc[e] = col + e < N ? __half2float(__ushort_as_half(scale[col + e])) : 0.0f;
    __half h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = __float2half_rn(static_cast<float>(v[e]) * sxr * sc[e]);
    __half* o = static_cast<__half*>(out) + int64_t(row) * ldo + col;
    if (vec && col + 8 <= N) {
      u32x4 pk;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        pk[e] = uint32_t(__half_as_ushort(h[2 * e])) | (uint32_t(__half_as_ushort(h[2 * e + 1])) << 16);
      *reinterpret_cast<u32x4*>(o) = pk;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (col + e < N) o[e] = h[e];
    }
  }
}

// ---------------------------------------------------------------------------
// Launch helpers.

// Skinny launch shapes.  HBM streams best as few long contiguous runs: for
// up to 16 rows every wave reads one 16-channel strip front to back (its
// packed bytes are contiguous), with PF groups in flight and the activations
// on a ring of the same depth.  K is split over the waves of a block only when
// there are too few strips to give every CU several waves.  For 32 or 64 rows
// the activation operand is larger than the weights it multiplies, so a wave
// covers TN strips with one activation load and the K range is split over 4
// waves.
#ifndef QOQ_S1PF
#define QOQ_S1PF 4
#endif
#ifndef QOQ_SKS4
#define QOQ_SKS4 4
#endif
#ifndef QOQ_SPF
#define QOQ_SPF 4
#endif
constexpr int kStripWavesTarget = 1024;  // 4 waves per CU

template <int TM, int TN, int KS, int PF, int AD, int WF, bool I32>
hipError_t launch_skinny(const GemmArgs& a, hipStream_t st) {
  const dim3 grid((a.n_strips + TN - 1) / TN, (a.M + TM * 16 - 1) / (TM * 16));
  hipLaunchKernelGGL((gemm_skinny_kernel<TM, TN, KS, PF, AD, WF, I32>), grid, dim3(64 * KS), 0, st, a);
  return hipGetLastError();
}

// Strips per skinny block: the fewest rounds of 256 blocks (one per CU) times
// strips per block, for `ny` row tiles and at most `hi` strips; ties go to more
// strips per block (less activation traffic).
inline int pick_skinny_tn(int n_strips, int ny, int hi) {
  int best = 1;
  long best_cost = -1;
  for (int tn = 1; tn <= hi; ++tn) {
    const long blocks = long((n_strips + tn - 1) / tn) * ny;
    const long cost = ((blocks + 255) / 256) * tn;
    if (best_cost < 0 || cost <= best_cost) {
      best = tn;
      best_cost = cost;
    }
  }
  return best;
}

// Strips per block of the skinny kernel with 64-row tiles.  Besides its tn
// weight strips every block reads a 64 x K activation slab (eight strips'
// worth of bytes per group, mostly from L2); a block takes about
// kActStrips + tn strip-times (fitted to K = 4096 runs of 1, 2 and 4 strips
// per block), so the fewest rounds of 256 blocks times that wins, ties going
// to more strips per block.
#ifndef QOQ_ACT_STRIPS
#define QOQ_ACT_STRIPS 4
#endif
inline int pick_skinny_tn_rows(int n_strips, int ny, int hi) {
  int best = 1;
  long best_cost = -1;
  for (int tn = 1; tn <= hi; ++tn) {
    const long blocks = long((n_strips + tn - 1) / tn) * ny;
    const long cost = ((blocks + 255) / 256) * (QOQ_ACT_STRIPS + tn);
    if (best_cost < 0 || cost <= best_cost) {
      best = tn;
      best_cost = cost;
    }
  }
  return best;
}

#ifndef QOQ_SAD
#define QOQ_SAD 2
#endif
// Most strips per skinny block: 8, or 7 with 64-row tiles (eight would not
// fit the register file beside four row tiles of accumulators).
constexpr int skinny_tn_max(int tm) { return tm >= 4 ? 7 : 8; }
// Weight-ring depth of the skinny kernel: the same bytes in flight for every
// format (INT8 blocks are twice as large, so half as many groups).
constexpr int skinny_pf(int wf) { return QOQ_SPF / wf_vec(wf); }

// launch_skinny with TN = tn, instantiated for 1 <= TN <= T only
template <int TM, int WF, bool I32, int T>
hipError_t launch_skinny_upto(int tn, const GemmArgs& a, hipStream_t st) {
  if constexpr (T > 1) {
    if (tn < T) return launch_skinny_upto<TM, WF, I32, T - 1>(tn, a, st);
  }
  return launch_skinny<TM, T, QOQ_SKS4, skinny_pf(WF), QOQ_SAD, WF, I32>(a, st);
}

template <int TM, int WF, bool I32>
hipError_t dispatch_skinny_tn(const GemmArgs& a, hipStream_t st) {
  constexpr int kHi = skinny_tn_max(TM);
  const int ny = (a.M + TM * 16 - 1) / (TM * 16);
  const int tn = TM == 4 ? pick_skinny_tn_rows(a.n_strips, ny, kHi) : pick_skinny_tn(a.n_strips, ny, kHi);
  return launch_skinny_upto<TM, WF, I32, kHi>(tn, a, st);
}

// Dynamic LDS of the strip kernel: the activations, or the K-part partial
// sums, whichever is larger.
inline size_t strip_lds_bytes(int G, int R, int spb, int ks, bool group_meta) {
  const size_t act = size_t(round_up(int64_t(G) * R * 8 * 16, 1024));
  const size_t meta = group_meta ? size_t(round_up(int64_t(spb) * round_up(G, 4) / 4 * 64, 1024)) : 0;
  const size_t red = size_t(spb) * size_t(ks - 1) * 1024;
  return act + meta > red ? act + meta : red;
}
constexpr size_t kStripMaxLds = 160 * 1024;

template <int WF, bool I32>
hipError_t launch_strip(const GemmArgs& a, int spb, int ks, size_t lds, hipStream_t st) {
  constexpr int PF = QOQ_S1PF;
  auto* fn = gemm_strip_kernel<PF, WF, I32>;
  if (lds > 64 * 1024) {
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(kStripMaxLds));
    if (attr != hipSuccess) return attr;
  }
  const dim3 grid((a.n_strips + spb - 1) / spb);
  hipLaunchKernelGGL(fn, grid, dim3(64 * spb * ks), lds, st, a, spb, ks);
  return hipGetLastError();
}

// Up to 16 rows: the strip kernel when the activations fit in LDS, else the
// K-split skinny kernel.  Strips per block as for the skinny kernel (rounds of
// 256 blocks); the K split fills a block up to 8 waves.
template <int WF, bool I32>
hipError_t dispatch_skinny_strip(const GemmArgs& a, hipStream_t st) {
  const int R = a.M < 16 ? a.M : 16;
  const int spb = pick_skinny_tn(a.n_strips, 1, 8);
  int ks = 8 / spb;
  if (ks < 1) ks = 1;
  const size_t lds = strip_lds_bytes(a.G, R, spb, ks, wf_group_meta(WF));
  if (lds <= kStripMaxLds) return launch_strip<WF, I32>(a, spb, ks, lds, st);
  return dispatch_skinny_tn<1, WF, I32>(a, st);
}


// Large-M plans.  Tile 0: 256x256 blocks of 8 waves (each 128 x 64).
// Tile 1: 128x128 blocks of 4 waves (each 64 x 64), for smaller problems.
struct LargePlan {
  int tile;    // 0 or 1
  int ksplit;  // K splits
};

inline int64_t tiles_of(int64_t M, int64_t N_pad, int bm, int bn) { return ((M + bm - 1) / bm) * ((N_pad + bn - 1) / bn); }

// Pick a tile, then the K split with the least estimated time: ceil(blocks /
// 256) rounds of blocks, each G / ksplit groups long, plus, for a split, the
// INT32 partials written and read again by the reduction (about 5 TB/s)
// and its launch.  Per-group block times are the ones measured with every CU
// busy: about 0.8 us for a 128x128 tile and 2.2 us for a 256x256 one.  Every
// split keeps at least 4 groups (512 channels).
inline LargePlan plan_large(int64_t M, int64_t N, int64_t K) {
  const int64_t N_pad = round_up(N, kStrip);
  const int64_t G = K / kGroup;
  LargePlan p{0, 1};
  const int64_t big = tiles_of(M, N_pad, 256, 256);
  if (big < 192) p.tile = 1;
  const int64_t tiles = p.tile ? tiles_of(M, N_pad, 128, 128) : big;
  const int64_t group_ns = p.tile ? 800 : 2200;
  auto cost_ns = [&](int64_t ks) {
    const int64_t run = ((tiles * ks + 255) / 256) * ((G + ks - 1) / ks) * group_ns;
    return ks > 1 ? run + ks * M * N_pad * 8 / 5000 + 2000 : run;
  };
  for (int64_t ks = 2; G / ks >= 4; ks *= 2)
    if (cost_ns(ks) < cost_ns(p.ksplit)) p.ksplit = int(ks);
  return p;
}

// Largest M served by the K-split skinny kernel (64-row tiles above 32 rows).
#ifndef QOQ_SKINNY_MAXM
#define QOQ_SKINNY_MAXM 64
#endif
constexpr int64_t kSkinnyMaxM = QOQ_SKINNY_MAXM;

// Up to 256 rows, the K-split skinny kernel (64-row tiles, partials summed in
// LDS) also serves when it covers the whole problem in one round of blocks:
// the large kernel would split K across blocks there, and its INT32 partials
// need a second pass through memory.
constexpr int64_t kSkinnyMidMaxM = 256;
inline bool skinny_mid(int64_t M, int64_t N) {
  if (M <= kSkinnyMaxM || M > kSkinnyMidMaxM) return false;
  const int n_strips = int(round_up(N, kStrip) / kStrip);
  const int ny = int((M + 63) / 64);
  const int tn = pick_skinny_tn_rows(n_strips, ny, skinny_tn_max(4));
  const int64_t blocks = int64_t((n_strips + tn - 1) / tn) * ny;
  return blocks <= 256;
}

inline size_t workspace_bytes_of(int64_t M, int64_t N, int64_t K) {
  if (M <= kSkinnyMaxM || skinny_mid(M, N)) return 0;
  const LargePlan p = plan_large(M, N, K);
  return p.ksplit > 1 ? size_t(p.ksplit) * size_t(M) * size_t(round_up(N, kStrip)) * sizeof(int) : 0;
}

template <int WM, int WN, int TM, int TN, int D, int DA, int WF, bool I32>
hipError_t launch_large(const GemmArgs& a, hipStream_t st) {
  constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
  const dim3 grid((a.n_strips * 16 + BN - 1) / BN, (a.M + BM - 1) / BM, a.ksplit);
  hipLaunchKernelGGL((gemm_large_kernel<WM, WN, TM, TN, D, DA, WF, I32>), grid, dim3(64 * WM * WN), 0, st, a);
  return hipGetLastError();
}

template <int WF, bool I32>
hipError_t launch_large_tile(int tile, const GemmArgs& a, hipStream_t st) {
  // On the 256x256 tile the INT8 weight ring and the 16-bit lanes of the
  // saturating dequantization leave room for one group of activations in
  // flight instead of two (two would spill).
  constexpr int kLDA = (WF == kWfW8 || WF == kWfG128Sat) ? 1 : QOQ_LDA;
  if (tile == 0) return launch_large<QOQ_LWM, QOQ_LWN, QOQ_LTM, QOQ_LTN, QOQ_LD, kLDA, WF, I32>(a, st);
  return launch_large<QOQ_SWM, QOQ_SWN, QOQ_STM, QOQ_STN, QOQ_SD, QOQ_SDA, WF, I32>(a, st);
}

template <int WF, bool I32>
hipError_t dispatch(const GemmArgs& a0, void* ws, hipStream_t st) {
  if (a0.M <= 16) return dispatch_skinny_strip<WF, I32>(a0, st);
  if (a0.M <= 32) return dispatch_skinny_tn<2, WF, I32>(a0, st);
  if (a0.M <= kSkinnyMaxM || skinny_mid(a0.M, a0.N)) return dispatch_skinny_tn<4, WF, I32>(a0, st);
  const LargePlan p = plan_large(a0.M, a0.N, int64_t(a0.G) * kGroup);
  if (p.ksplit == 1) return launch_large_tile<WF, I32>(p.tile, a0, st);
  // split K: INT32 partials into the workspace, then reduce + epilogue
  GemmArgs a = a0;
  a.ksplit = p.ksplit;
  a.out = ws;
  a.ldo = int64_t(a.n_strips) * kStrip;
  a.zstride = int64_t(a.M) * a.ldo;
  hipError_t e = launch_large_tile<WF, true>(p.tile, a, st);
  if (e != hipSuccess) return e;
  const int ldw = a.n_strips * kStrip;
  const int64_t threads = int64_t(a.M) * (ldw / 8);
  const dim3 grid(static_cast<unsigned>((threads + 255) / 256));
  // 16-byte row segments: aligned base, and a row stride that keeps them aligned
  const int esize = I32 ? 4 : 2;
  const int vec = reinterpret_cast<uintptr_t>(a0.out) % 16 == 0 && (a0.ldo * esize) % 16 == 0;
  hipLaunchKernelGGL((splitk_reduce_kernel<I32>), grid, dim3(256), 0, st, static_cast<const int*>(ws), a.ksplit, a.M,
                     a.N, ldw, a0.sx, a0.scale, a0.out, a0.ldo, vec);
  return hipGetLastError();
}

// Argument checks and launch of one weight format.  meta may be NULL for the
// INT8 weights; group_size is the one of the UINT4 formats (128 or 0).
template <int WF>
int run_gemm(const char* fn, const int8_t* x8, const void* sx, const void* qweight, const void* meta,
             const void* scale, void* out, int64_t M, int64_t N, int64_t K, int64_t ldo, int32_t group_size,
             void* workspace, size_t workspace_bytes, bool i32, hipStream_t st) {
  clear_error();
  const bool need_meta = WF != kWfW8;
  if (!x8 || !qweight || (need_meta && !meta) || !out || (!i32 && (!sx || !scale)))
    return fail(QOQ_ERR_INVALID_ARG, "%s: null pointer argument", fn);
  if (int stt = check_weight_shape(N, K, group_size)) return stt;
  if (M < 1 || M > 0x7fffffffLL - 4096) return fail(QOQ_ERR_UNSUPPORTED_SHAPE, "%s: M=%lld out of range", fn, (long long)M);
  if (ldo < N) return fail(QOQ_ERR_INVALID_ARG, "%s: leading dimension %lld < N=%lld", fn, (long long)ldo, (long long)N);
  const auto al = [](const void* p, uintptr_t n) { return reinterpret_cast<uintptr_t>(p) % n == 0; };
  if (!al(x8, 16) || !al(qweight, 16) || (need_meta && !al(meta, 4)) || !al(out, i32 ? 4 : 2) ||
      (!i32 && (!al(sx, 2) || !al(scale, 2))))
    return fail(QOQ_ERR_ALIGNMENT, "%s: x8/qweight need 16-byte, meta 4-byte, FP16 2-byte alignment", fn);
  GemmArgs a;
  a.x8 = x8;
  a.sx = static_cast<const unsigned short*>(sx);
  a.qw = static_cast<const u32x4*>(qweight);
  a.meta = static_cast<const uint32_t*>(meta);
  a.meta8 = static_cast<const uint8_t*>(meta);
  a.scale = static_cast<const unsigned short*>(scale);
  a.out = out;
  a.M = static_cast<int>(M);
  a.N = static_cast<int>(N);
  a.G = static_cast<int>(K / kGroup);
  a.G4q = static_cast<int>(round_up(a.G, 4) / 4);
  a.n_strips = static_cast<int>(round_up(N, kStrip) / kStrip);
  a.ldo = ldo;
  a.ksplit = 1;
  a.zstride = 0;
  const size_t need = workspace_bytes_of(M, N, K);
  if (need && (!workspace || workspace_bytes < need))
    return fail(QOQ_ERR_INVALID_ARG, "%s: workspace of %zu bytes required (got %zu); see the workspace-size query",
                fn, need, workspace ? workspace_bytes : size_t(0));
  if (need && reinterpret_cast<uintptr_t>(workspace) % 16)
    return fail(QOQ_ERR_ALIGNMENT, "%s: workspace must be 16-byte aligned", fn);
  const hipError_t e = i32 ? dispatch<WF, true>(a, workspace, st) : dispatch<WF, false>(a, workspace, st);
  if (e != hipSuccess) return fail(QOQ_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return QOQ_OK;
}

inline size_t workspace_size_query(int64_t M, int64_t N, int64_t K, int32_t group_size) {
  if (M < 1 || check_weight_shape(N, K, group_size) != QOQ_OK) {
    clear_error();
    return 0;
  }
  return workspace_bytes_of(M, N, K);
}

}  // namespace
}  // namespace qoq
