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
//   §5: subtraction after multiplication, w8 = q4*s1 - z*s1; the packed
//     weights laid out in the order the kernel consumes them, fetched 16 bytes
//     per lane; the per-channel scale applied in the epilogue; FP16 output.
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
//   large:  v_mfma_i32_32x32x32_i8, 128x512, 64x256 or 128x128 block tiles, K
//           optionally split across blocks (and, on the 128x128 tile,
//           inside the block); above 64 rows (prefill).
// Weights always go global -> VGPR directly and are dequantized in
// registers.  Both MFMA operands use the same K order per (lane group, byte),
// so the contraction is exact whatever order the matrix unit walks K in.

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <algorithm>
#include <type_traits>
#include <utility>

#include "qoq_internal.h"

// Large-M tiles: WM x WN waves, each TM x TN tiles of 32x32.  Both are one
// row of 8 waves side by side: every wave multiplies the block's whole row
// range by its own columns, so no two waves load or dequantize the same
// weights, and the block's activation tile (read from LDS by all 8 waves) is
// BM rows.  Big tile: 128 x 512 (waves of 128 x 64); small tile: 64 x 256
// (waves of 64 x 32), for problems with too few big tiles.  Both hold 65536
// outputs, so per-group block times are alike.
#ifndef QOQ_LWM
#define QOQ_LWM 1
#define QOQ_LWN 8
#define QOQ_LTM 4
#define QOQ_LTN 2
#endif
#ifndef QOQ_SWM
#define QOQ_SWM 1
#define QOQ_SWN 8
#define QOQ_STM 2
#define QOQ_STN 1
#endif
// K-set tile: the small tile's problems when each block has many groups to
// run: 128 x 128 blocks of two sets of 4 waves (waves of 128 x 32), the sets
// taking alternate groups.  A weight fragment then feeds 4 MFMAs instead of 2.
#ifndef QOQ_KWM
#define QOQ_KWM 1
#define QOQ_KWN 4
#define QOQ_KTM 4
#define QOQ_KTN 1
#define QOQ_KKI 2
#endif
// Fewest groups per block (after any K split) for the K-set tile.
#ifndef QOQ_KSET_MIN_GROUPS
#define QOQ_KSET_MIN_GROUPS 64
#endif
// Weight-ring depth (groups of weights in flight) of the big and of the
// small large-M tile.
#ifndef QOQ_LD
#define QOQ_LD 2
#endif
#ifndef QOQ_SD
#define QOQ_SD 4
#endif
static_assert(QOQ_LWM * QOQ_LWN == 8 && QOQ_SWM * QOQ_SWN == 8 && QOQ_KWM * QOQ_KWN * QOQ_KKI == 8,
              "large-M blocks are 8 waves");

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

// s_waitcnt immediates (gfx9 encoding): wait until at most n vector-memory
// operations of this wave are outstanding, leaving the other counters free.
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Barrier for LDS traffic only: this wave's LDS operations are complete
// (lgkmcnt 0) and every wave has arrived.  Global loads stay in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __builtin_amdgcn_s_barrier();
}

// Direct global -> LDS copy of 16 bytes per lane: lane i writes lds + 16 i.
// (Kept in a device function: the builtin is not meaningful to the host pass.)
__device__ __forceinline__ void buf_load_lds16(__amdgpu_buffer_rsrc_t r, int8_t* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
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

// f(std::integral_constant<int, i>) for i = 0 .. N-1, each i a compile-time
// constant (for immediates such as hand-counted waits in unrolled loops).
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

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
// same TN strips between them, so every wave streams different weight bytes
// (8 waves, two per SIMD, when every wave still gets at least 8 groups: one
// wave's dequantization then runs while the other's MFMAs do).  Each wave
// streams its weights through a PF-deep register ring of 128-bit loads and
// its activations (whole 128-byte rows, shared by all blocks and mostly
// served from L2) through a PF-deep ring of its own in LDS, filled by direct
// global -> LDS copies, so that enough bytes are in flight to cover HBM
// latency.  The KS partial INT32 accumulators are summed exactly through LDS
// at the end, and the FP16 results leave through an LDS tile in 16-byte row
// segments.

// The A fragments of one K half from a wave's activation ring: row tile i
// sits 2048 bytes after tile i-1 (the chunk swizzle depends only on the row
// within its 16-row tile).  Read in inline assembly: the compiler cannot tell
// which ring slot a direct-to-LDS copy fills and would otherwise wait for
// every copy in flight before each read.  The caller's hand-counted vmcnt
// wait covers the slot read here, and the block waits for its own reads, so
// no output register is left in flight.
// One dword from LDS, read the same way (for data that direct-to-LDS copies
// wrote before the last barrier, while other copies are in flight).
__device__ __forceinline__ uint32_t lds_read_u32(const uint32_t* p) {
  const auto* lp = (const __attribute__((address_space(3))) uint32_t*)p;
  uint32_t v;
  asm volatile("ds_read_b32 %0, %1\n s_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lp))));
  return v;
}

// Both K halves' A fragments of one group (row tile i of half h at p[h] +
// 2048 i) and, when `pm` is given, the metadata dword at pm, with a single
// wait: one LDS round trip per group.
template <int TM>
__device__ __forceinline__ void read_group_frags(v4i (&af)[2][TM], uint32_t& m, const int8_t* p0, const int8_t* p1,
                                                 const uint32_t* pm) {
  const auto ad = [](const void* q) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) int8_t*)q));
  };
  const uint32_t a0 = ad(p0), a1 = ad(p1), am = ad(pm);
  if constexpr (TM == 1) {
    asm volatile("ds_read_b128 %0, %3\n ds_read_b128 %1, %4\n ds_read_b32 %2, %5\n s_waitcnt lgkmcnt(0)"
                 : "=&v"(af[0][0]), "=&v"(af[1][0]), "=&v"(m)
                 : "v"(a0), "v"(a1), "v"(am));
  } else if constexpr (TM == 2) {
    asm volatile(
        "ds_read_b128 %0, %5\n ds_read_b128 %1, %5 offset:2048\n ds_read_b128 %2, %6\n"
        " ds_read_b128 %3, %6 offset:2048\n ds_read_b32 %4, %7\n s_waitcnt lgkmcnt(0)"
        : "=&v"(af[0][0]), "=&v"(af[0][1]), "=&v"(af[1][0]), "=&v"(af[1][1]), "=&v"(m)
        : "v"(a0), "v"(a1), "v"(am));
  } else {
    static_assert(TM == 4, "row tiles per ring block: 1, 2 or 4");
    asm volatile(
        "ds_read_b128 %0, %9\n ds_read_b128 %1, %9 offset:2048\n ds_read_b128 %2, %9 offset:4096\n"
        " ds_read_b128 %3, %9 offset:6144\n ds_read_b128 %4, %10\n ds_read_b128 %5, %10 offset:2048\n"
        " ds_read_b128 %6, %10 offset:4096\n ds_read_b128 %7, %10 offset:6144\n ds_read_b32 %8, %11\n"
        " s_waitcnt lgkmcnt(0)"
        : "=&v"(af[0][0]), "=&v"(af[0][1]), "=&v"(af[0][2]), "=&v"(af[0][3]), "=&v"(af[1][0]), "=&v"(af[1][1]),
          "=&v"(af[1][2]), "=&v"(af[1][3]), "=&v"(m)
        : "v"(a0), "v"(a1), "v"(am));
  }
}

template <int TM>
__device__ __forceinline__ void read_a_frags(v4i (&af)[TM], const int8_t* p) {
  const auto* lp = (const __attribute__((address_space(3))) int8_t*)p;
  const uint32_t ad = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lp));
  if constexpr (TM == 1) {
    asm volatile("ds_read_b128 %0, %1\n s_waitcnt lgkmcnt(0)" : "=&v"(af[0]) : "v"(ad));
  } else if constexpr (TM == 2) {
    asm volatile("ds_read_b128 %0, %2\n ds_read_b128 %1, %2 offset:2048\n s_waitcnt lgkmcnt(0)"
                 : "=&v"(af[0]), "=&v"(af[1])
                 : "v"(ad));
  } else {
    static_assert(TM == 4, "row tiles per skinny block: 1, 2 or 4");
    asm volatile(
        "ds_read_b128 %0, %4\n ds_read_b128 %1, %4 offset:2048\n ds_read_b128 %2, %4 offset:4096\n"
        " ds_read_b128 %3, %4 offset:6144\n s_waitcnt lgkmcnt(0)"
        : "=&v"(af[0]), "=&v"(af[1]), "=&v"(af[2]), "=&v"(af[3])
        : "v"(ad));
  }
}

template <int TM, int TN, int KS, int PF, int WF, bool I32OUT>
__global__ __launch_bounds__(64 * KS) void gemm_skinny_kernel(GemmArgs a) {
  static_assert(KS == 4 || KS == 8, "K parts per skinny block: 4 or 8");
  // LDS: while multiplying, wave w's activation ring (PF slots of TM*16 rows
  // x 128 B); afterwards the partial sums, [KS/2 or KS][TN][TM][64 lanes]
  // records of 4 INT32 (with 8 waves the upper four first hand theirs to the
  // lower four), followed by the FP16 output tile [TM*16][TN*16].
  constexpr int kSlot = TM * 16 * 128;
  constexpr int kRingBytes = KS * PF * kSlot;
  constexpr int kRedWaves = KS > 4 ? KS / 2 : KS;
  constexpr int kRedBytes = kRedWaves * TN * TM * 1024;
  constexpr int kTileCols = TN * 16;
  constexpr int kTileBytes = I32OUT ? 0 : TM * 16 * kTileCols * 2;
  constexpr int kSmemBytes = kRingBytes > kRedBytes + kTileBytes ? kRingBytes : kRedBytes + kTileBytes;
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
  int8_t* ring = smem + wave * (PF * kSlot);
  const int c16 = lane & 15, j = lane >> 4;
  const int sbase = blockIdx.x * TN;
  const int m0 = blockIdx.y * TM * 16;
  const int64_t K = int64_t(a.G) * 128;
  const int g0 = (a.G * wave) / KS, g1 = (a.G * (wave + 1)) / KS;

  constexpr int kVec = wf_vec(WF);
  uint32_t S[TN] = {}, C[TN] = {};
  if constexpr (WF == kWfPerChannel) {
#pragma unroll
    for (int t = 0; t < TN; ++t) meta_perchannel(a.meta8[min(sbase + t, a.n_strips - 1) * 16 + c16], S[t], C[t]);
  }

  v4i acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int t = 0; t < TN; ++t) acc[i][t] = v4i{0, 0, 0, 0};

  u32x4 bq[PF][TN][kVec];
  uint32_t mq[PF][TN];

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
  // Activations: copy (i, hh) of a group moves 8 whole 128-byte rows (every
  // cache line it touches is used in full), lane l filling LDS row r = 16 i +
  // 8 hh + l/8 at stored position l % 8, which holds the row's logical chunk
  // (l % 8) ^ ((r >> 1) & 7): the swizzle of lds_off, so the MFMA-layout
  // reads are conflict-free.  Rows past M read row M-1 (never stored); a
  // group past the range gets an empty descriptor and touches no memory.
  const int8_t* xbase = a.x8 + int64_t(m0) * K;
  const int xbytes = int(min(TM * 16, a.M - m0) * K);
  int aoff[TM][2];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int r = 16 * i + 8 * hh + (lane >> 3);
      const int kc = (lane & 7) ^ ((r >> 1) & 7);
      aoff[i][hh] = (min(m0 + r, a.M - 1) - m0) * int(K) + kc * 16;
    }
  auto load_a = [&](int g, int slot) {
    const bool live = g < g1;
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(xbase + (live ? g : 0) * 128, live ? xbytes : 0);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) buf_load_lds16(xr, ring + slot * kSlot + (2 * i + hh) * 1024, aoff[i][hh], 0);
  };
  // vector-memory operations of one group (weights, metadata, activation
  // copies); a wait down to kAhead outstanding leaves the last PF - 1 groups
  // in flight (at most 63 can be counted)
  constexpr int kLoads = TN * kVec + (wf_group_meta(WF) ? TN : 0) + 2 * TM;
  constexpr int kAhead = (PF - 1) * kLoads < 63 ? (PF - 1) * kLoads : 63;

  // Multiply group g from ring slot `slot`: per K half, the TM A fragments,
  // then per strip the dequantized B operand feeding TM MFMAs.
  auto compute = [&](int g, int slot, const u32x4 (&bc)[TN][kVec], const uint32_t (&mc)[TN]) {
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
      v4i af[TM];
      read_a_frags<TM>(af, ring + slot * kSlot + lds_off(c16, j + 4 * h));
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        const v4i bf = b_op16<WF>(bc[t], h, S[t], C[t]);
#pragma unroll
        for (int i = 0; i < TM; ++i) acc[i][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[i], bf, acc[i][t], 0, 0, 0);
      }
    }
  };

  const int ng = g1 - g0;
  if (ng > 0) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      load_b(g0 + p, bq[p], mq[p]);
      load_a(g0 + p, p);
    }
    // Rounds of PF groups; ring slot u holds group g0 + it + u.  Step u waits
    // until the operands of its group have landed (everything issued before
    // the last PF - 1 groups' loads), multiplies it, and refills the slot with
    // the group PF ahead.  Past the range the loads are empty and free.  The
    // refill follows the slot's last read: the fragments were consumed by the
    // MFMAs before the fence.
    for (int it = 0; it < ng; it += PF) {
#pragma unroll
      for (int u = 0; u < PF; ++u) {
        const int g = g0 + it + u;
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(kAhead));
        QOQ_COMPILER_FENCE();
        if (g < g1) compute(g, u, bq[u], mq[u]);
        QOQ_COMPILER_FENCE();
        load_b(g + PF, bq[u], mq[u]);
        load_a(g + PF, u);
        QOQ_COMPILER_FENCE();
      }
    }
  }
  // the trailing (empty) copies land before the LDS is reused
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));

  // Epilogue scales, fetched now so that their latency overlaps the
  // reduction (held through the loop they would cost registers): row scales
  // of the lane's rows and column scales of the strips this wave stores.
  // The raw FP16 bits are kept (addresses clamped into range) and converted
  // where they are used.
  constexpr int kScN = (TN + KS - 1) / KS;
  unsigned short sxh[TM][4] = {}, sch[kScN] = {};
  if constexpr (!I32OUT) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) sxh[i][r] = a.sx[min(m0 + i * 16 + 4 * j + r, a.M - 1)];
#pragma unroll
    for (int u = 0; u < kScN; ++u) sch[u] = a.scale[min((sbase + min(wave + u * KS, TN - 1)) * 16 + c16, a.N - 1)];
  }
  auto fp16 = [](unsigned short h) { return __half2float(__ushort_as_half(h)); };

  // Exact cross-wave reduction of the K-part sums ([wave][strip][row tile]
  // [lane] 16-byte records: one 128-bit LDS access per accumulator tile),
  // then wave w finishes strips w, w+KS, ... (lane holds rows 4*(lane/16)+r
  // of each 16x16 tile, column lane%16).
  __syncthreads();  // every wave is done with its ring
  v4i* red4 = reinterpret_cast<v4i*>(smem);
  if constexpr (KS > kRedWaves) {
    if (wave >= kRedWaves) {
#pragma unroll
      for (int t = 0; t < TN; ++t)
#pragma unroll
        for (int i = 0; i < TM; ++i) red4[(((wave - kRedWaves) * TN + t) * TM + i) * 64 + lane] = acc[i][t];
    }
    __syncthreads();
    if (wave < kRedWaves) {
#pragma unroll
      for (int t = 0; t < TN; ++t)
#pragma unroll
        for (int i = 0; i < TM; ++i) acc[i][t] += red4[((wave * TN + t) * TM + i) * 64 + lane];
    }
    __syncthreads();
  }
  if (wave < kRedWaves) {
#pragma unroll
    for (int t = 0; t < TN; ++t)
#pragma unroll
      for (int i = 0; i < TM; ++i) red4[((wave * TN + t) * TM + i) * 64 + lane] = acc[i][t];
  }
  __syncthreads();
  __half* tile = reinterpret_cast<__half*>(smem + kRedBytes);
#pragma unroll
  for (int u = 0; u < kScN; ++u) {
    const int t = wave + u * KS;
    if (t < TN && sbase + t < a.n_strips) {
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        v4i v = red4[(t * TM + i) * 64 + lane];
#pragma unroll
        for (int w = 1; w < kRedWaves; ++w) v += red4[((w * TN + t) * TM + i) * 64 + lane];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if constexpr (I32OUT) {
            store_out<true>(a, m0 + i * 16 + 4 * j + r, (sbase + t) * 16 + c16, v[r], 0.0f, 0.0f);
          } else {
            const float y = static_cast<float>(v[r]) * fp16(sxh[i][r]) * fp16(sch[u]);
            tile[(i * 16 + 4 * j + r) * kTileCols + t * 16 + c16] = __float2half_rn(y);
          }
        }
      }
    }
  }
  if constexpr (!I32OUT) {
    // the block's FP16 rows, 16 bytes at a time where the output rows are
    // 16-byte aligned (element by element otherwise and at a ragged end)
    __syncthreads();
    const int rows = min(TM * 16, a.M - m0);
    const int col0 = sbase * 16;
    const int cols = min(kTileCols, a.N - col0);
    const bool vec = ((reinterpret_cast<uintptr_t>(a.out) | uintptr_t(a.ldo * 2)) & 15) == 0;
    constexpr int kSeg = kTileCols / 8;
    for (int e = threadIdx.x; e < TM * 16 * kSeg; e += 64 * KS) {
      const int row = e / kSeg, c = (e - row * kSeg) * 8;
      if (row < rows && c < cols) {
        __half* dst = static_cast<__half*>(a.out) + int64_t(m0 + row) * a.ldo + col0 + c;
        const __half* src = tile + row * kTileCols + c;
        if (vec && c + 8 <= cols) {
          *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
        } else {
          for (int q = 0; q < 8 && c + q < cols; ++q) dst[q] = src[q];
        }
      }
    }
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


template <int PF, int WF, bool I32OUT>
__global__ __launch_bounds__(512) void gemm_strip_kernel(GemmArgs a, int spb, int ks, int rp) {
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

  // activations -> LDS, RP = rp rows per group (16 or R, from the launch).
  // Lane l of a wave-wide copy fills LDS chunk base + l.  With 16 rows a group
  // (rows R..15 repeat row R-1, never stored) every copy moves 8 rows of one
  // group: the lane's offset is loop-invariant and the group a wave-uniform
  // soffset, so the copies cost no vector ALU work before the weight stream
  // starts.  Groups of R rows are packed densely (lanes past the end fetch a
  // valid chunk into the allocation's padding).
  const int RP = rp;
  const int n_chunks = a.G * RP * 8;
  if (RP == 16) {
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x8, R * int(K));
    int coff[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int lrow = (lane >> 3) + 8 * h;
      coff[h] = min(lrow, R - 1) * int(K) + (((lane & 7) ^ ((lrow >> 1) & 7)) << 4);
    }
    for (int c = wave; c < 2 * a.G; c += nwaves) {
      const int g = c >> 1;
      buf_load_lds16(xr, smem + (g * 16 + 8 * (c & 1)) * 128, (c & 1) ? coff[1] : coff[0], g * 128);
    }
  } else {
    for (int base = wave * 64; base < n_chunks; base += nwaves * 64) {
      const int pc = min(base + lane, n_chunks - 1);
      const int lrow = pc >> 3;
      const int q = (pc & 7) ^ ((lrow >> 1) & 7);
      const int g = lrow / R, r = lrow - g * R;
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(a.x8 + int64_t(r) * K + int64_t(g) * 128 + q * 16),
                                       (__attribute__((address_space(3))) void*)(smem + base * 16), 16, 0, 0);
    }
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
    const int lrow = g * RP + ra;
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
// ring: up to 64 rows when the strips alone give about one block per CU
// (decode with a wide N).  As in the strip kernel every wave streams one
// 16-channel strip over the whole K range as one contiguous run and keeps one
// accumulator tile per 16 rows, so PF groups of weights stay in flight.  The
// block's TM*16 activation rows do not fit in LDS whole: they pass through a
// ring of two batches of kRingBatch groups, copied by every wave of the block
// one batch ahead (direct-to-LDS loads), with one barrier per batch.
//
// LDS: batch slot b (of 2): kRingBatch group tiles of R = TM*16 rows x 128 B,
// row r of group u at row u*R + r, 16-byte chunk q stored at chunk
// q ^ ((row >> 1) & 7) (row tiles of 16 share one swizzle, 2048 bytes apart);
// then the metadata of the block's strips (g128), as in the strip kernel.
constexpr int kRingBatch = 8;
constexpr int ring_batch_bytes(int tm) { return kRingBatch * tm * 16 * 128; }

template <int TM, int SPB, int PF, int WF, bool I32OUT>
__global__ __launch_bounds__(64 * SPB) void gemm_ring_kernel(GemmArgs a) {
  static_assert(kRingBatch % PF == 0 || PF % kRingBatch == 0, "the weight ring turns over at a batch boundary");
  static_assert(PF * wf_vec(WF) + (PF + kRingBatch - 1) / kRingBatch * ((kRingBatch * TM * 16 * 8 / 64 + SPB - 1) / SPB) <= 63 &&
                    kRingBatch * wf_vec(WF) <= 63,
                "vmcnt holds at most 63");
  constexpr int spb = SPB;  // strips (waves) per block
  extern __shared__ __align__(16) int8_t smem[];
  constexpr int R = TM * 16;
  constexpr int kBatchChunks = kRingBatch * R * 8;  // 16-byte chunks per batch
  constexpr int kBatchBytes = ring_batch_bytes(TM);
  static_assert(kBatchChunks % 64 == 0, "whole wave-wide copies per batch");
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int sb = blockIdx.x * spb;
  const int strip = sb + wave;
  const bool live = strip < a.n_strips;
  const int cstrip = min(strip, a.n_strips - 1);
  const int c16 = lane & 15, j = lane >> 4;
  const int G = a.G;
  const int64_t K = int64_t(G) * 128;
  const int nb = (G + kRingBatch - 1) / kRingBatch;

  // Activation copies of batch bt into slot bt & 1.  Every wave issues the
  // same, compile-time number of copy instructions (a wave past the batch's
  // last 64 chunks repeats them: the same bytes to the same place), so the
  // compiler's waits for the weight registers and the hand-counted waits
  // below are exact for every wave.  Rows past M read row M-1 (never
  // stored).  One descriptor over the M activation rows: the per-lane offsets
  // of the ncp copies are loop-invariant and the batch is a wave-uniform
  // soffset, so the copies cost no vector ALU work (the plan keeps G a
  // multiple of kRingBatch, so every batch is whole; the copy issued after
  // the last batch re-reads it, never multiplied).
  constexpr int ncp = (kBatchChunks / 64 + spb - 1) / spb;
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(a.x8, int(int64_t(a.M) * K));
  int coff[ncp];
#pragma unroll
  for (int k = 0; k < ncp; ++k) {
    const int base = min((k * spb + wave) * 64, kBatchChunks - 64);
    const int pc = base + lane;
    const int lrow = pc >> 3;
    const int q = (pc & 7) ^ ((lrow >> 1) & 7);
    const int u = lrow / R, r = lrow - u * R;
    coff[k] = min(r, a.M - 1) * int(K) + u * 128 + q * 16;
  }
  auto copy_batch = [&](int bt) {
    int8_t* dst = smem + (bt & 1) * kBatchBytes;
    const int soff = min(bt, nb - 1) * (kRingBatch * 128);
#pragma unroll
    for (int k = 0; k < ncp; ++k) {
      const int base = min((k * spb + wave) * 64, kBatchChunks - 64);
      buf_load_lds16(xrs, dst + base * 16, coff[k], soff);
    }
  };
  // group metadata of the block's strips, after the ring (one contiguous run
  // of G4q * 64 bytes per strip); lanes past the end fetch a valid chunk into
  // the region's padding
  int8_t* meta_lds = smem + 2 * kBatchBytes;
  if constexpr (wf_group_meta(WF)) {
    const int m_chunks = min(spb, a.n_strips - sb) * a.G4q * 4;
    const int m_last = ((m_chunks - 1) >> 6) << 6;
    const int nmp = ((m_chunks + 63) / 64 + spb - 1) / spb;
    const int8_t* msrc = reinterpret_cast<const int8_t*>(a.meta) + int64_t(sb) * a.G4q * 64;
    for (int k = 0; k < nmp; ++k) {
      const int base = min((k * spb + wave) * 64, m_last);
      const int pc = min(base + lane, m_chunks - 1);
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(msrc + pc * 16),
                                       (__attribute__((address_space(3))) void*)(meta_lds + base * 16), 16, 0, 0);
    }
  }
  const uint32_t* lmeta = reinterpret_cast<const uint32_t*>(meta_lds) + wave * a.G4q * 16 + c16;

  constexpr int kVec = wf_vec(WF);
  constexpr int kBlk = wf_block_bytes(WF);
  const int strip_bytes = G * kBlk;
  const __amdgpu_buffer_rsrc_t wrs =
      make_rsrc(reinterpret_cast<const int8_t*>(a.qw) + int64_t(cstrip) * strip_bytes, live ? strip_bytes : 0);
  u32x4 bq[PF][kVec];
  auto load_b = [&](int g, u32x4 (&b)[kVec]) {
#pragma unroll
    for (int v = 0; v < kVec; ++v) b[v] = buf_load16<kCacheStream>(wrs, lane * 16 + v * 1024 + (g < G ? g * kBlk : kDeadOffset));
  };
  uint32_t S = 0, C = 0;
  if constexpr (WF == kWfPerChannel) meta_perchannel(a.meta8[cstrip * 16 + c16], S, C);

  // Prologue: batch 0, the metadata, then the first PF groups of weights;
  // wait for everything but those weights and meet the other waves.
  copy_batch(0);
  QOQ_COMPILER_FENCE();
#pragma unroll
  for (int p = 0; p < PF; ++p) load_b(p, bq[p]);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(PF * kVec));
  __builtin_amdgcn_s_barrier();
  QOQ_COMPILER_FENCE();

  v4i acc[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i) acc[i] = v4i{0, 0, 0, 0};
  // A fragments of one K half from group u of a slot (row tile i at +2048 i),
  // read in inline assembly with their own wait: the compiler cannot tell
  // which slot the copies in flight fill and would otherwise wait for all of
  // them before every read.
  // A fragments and metadata dword of group g (row u of a slot), one group
  // ahead: they are read right after the previous group's multiplies are
  // issued, so the read's round trip overlaps the matrix unit's work.  (The
  // formats without group metadata read, and ignore, a dword of the slot.)
  v4i fa[2][2][TM];
  uint32_t fm[2];
  auto read_next = [&](v4i (&af)[2][TM], uint32_t& mw, const int8_t* slot, int u, int g) {
    read_group_frags<TM>(af, mw, slot + strip_lds_off(u * R + c16, j), slot + strip_lds_off(u * R + c16, j + 4),
                         wf_group_meta(WF) ? lmeta + (min(g, G - 1) >> 2) * 16 : reinterpret_cast<const uint32_t*>(slot));
  };
  auto compute = [&](const v4i (&af)[2][TM], uint32_t mw, int g, const u32x4 (&bc)[kVec]) {
    if constexpr (wf_group_meta(WF)) meta_g128<WF>((mw >> (8 * (g & 3))) & 0xffu, S, C);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const v4i bf = b_op16<WF>(bc, h, S, C);
#pragma unroll
      for (int i = 0; i < TM; ++i) acc[i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[h][i], bf, acc[i], 0, 0, 0);
    }
  };
  // group u of a batch uses fragment buffer u % 2 (kRingBatch is even, so
  // every batch starts on buffer 0)
  static_assert(kRingBatch % 2 == 0, "fragment buffers alternate within a batch");
  read_next(fa[0], fm[0], smem, 0, 0);
  // one batch; group u of batch bt sits in weight slot (off + u) % PF, with
  // off a compile-time constant in the unrolled loop below
  auto batch = [&](int bt, int off) {
    // the next batch into the slot of batch bt - 1, which every wave is done
    // with (for every batch, so that every path through the loop issues the
    // same loads and the compiler's waits for the weights stay exact; after
    // the last batch it re-reads the last group)
    copy_batch(bt + 1);
    QOQ_COMPILER_FENCE();
    const int8_t* slot = smem + (bt & 1) * kBatchBytes;
    // Each group waits until its weights have landed: younger are the next
    // PF - 1 groups' loads and the copies of every batch begun since its
    // load was issued (PF groups earlier): for the batch's first
    // min(PF, kRingBatch) groups, ceil(PF / kRingBatch) batches' copies.
    constexpr int kFirst = PF < kRingBatch ? PF : kRingBatch;
    constexpr int kCross = (PF + kRingBatch - 1) / kRingBatch;
    static_for<kRingBatch>([&](auto uc) {
      constexpr int u = decltype(uc)::value;
      const int g = bt * kRingBatch + u;
      __builtin_amdgcn_s_waitcnt(waitcnt_vm((PF - 1) * kVec + (u < kFirst ? kCross * ncp : 0)));
      __builtin_amdgcn_sched_barrier(0);  // the weights' uses stay behind the wait
      compute(fa[u & 1], fm[u & 1], g, bq[(off + u) % PF]);
      QOQ_COMPILER_FENCE();
      load_b(g + PF, bq[(off + u) % PF]);
      if constexpr (u + 1 < kRingBatch) read_next(fa[(u + 1) & 1], fm[(u + 1) & 1], slot, u + 1, g + 1);
      QOQ_COMPILER_FENCE();
    });
    // the next batch's copies were issued before this batch's weight loads
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(kRingBatch * kVec));
    lds_barrier();
    // the next batch's first group (past the last batch: its copies of the
    // last group, never multiplied)
    read_next(fa[0], fm[0], smem + ((bt + 1) & 1) * kBatchBytes, 0, (bt + 1) * kRingBatch);
  };
  // PF > kRingBatch: the weight ring turns over every PF / kRingBatch
  // batches.  The plan keeps G a multiple of both, so that every batch is
  // whole: the loop has no data-dependent branch, and the compiler's waits
  // for the weight registers stay exact.
  constexpr int kUnrollB = PF > kRingBatch ? PF / kRingBatch : 1;
  for (int bt = 0; bt < nb; bt += kUnrollB) {
#pragma unroll
    for (int v = 0; v < kUnrollB; ++v) batch(bt + v, v * kRingBatch);
  }
  if (!live) return;

  // epilogue: lane holds rows 16 i + 4 (lane / 16) + r, column lane % 16
  const float sc = I32OUT ? 0.0f : col_scale(a, strip * 16 + c16);
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    float sxv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) sxv[r] = I32OUT ? 0.0f : row_scale(a, 16 * i + 4 * j + r);
#pragma unroll
    for (int r = 0; r < 4; ++r) store_out<I32OUT>(a, 16 * i + 4 * j + r, strip * 16 + c16, acc[i][r], sxv[r], sc);
  }
}

// ring2: the ring kernel with each strip's K range split over two waves
// (2 SPB waves a block, halves h = 0, 1 of the groups), so a CU holds twice
// the waves to hide each one's latency.  Both halves' activations pass
// through their own LDS ring of two batches of kRing2Batch groups (the block
// copies batch bt + 1 of both halves during batch bt, one barrier a batch);
// the halves' INT32 accumulators are added exactly through LDS at the end.
constexpr int kRing2Batch = 4;
constexpr int ring2_batch_bytes(int tm) { return 2 * kRing2Batch * tm * 16 * 128; }  // both halves

template <int TM, int SPB, int PF, int WF, bool I32OUT>
__global__ __launch_bounds__(128 * SPB) void gemm_ring2_kernel(GemmArgs a) {
  static_assert(PF == kRing2Batch, "one weight ring turn per batch");
  constexpr int NW = 2 * SPB;                             // waves
  constexpr int R = TM * 16;
  constexpr int kHalfChunks = kRing2Batch * R * 8;        // 16-byte chunks per batch and half
  constexpr int kBatchChunks = 2 * kHalfChunks;
  constexpr int kBatchBytes = ring2_batch_bytes(TM);
  constexpr int ncp = (kBatchChunks / 64 + NW - 1) / NW;  // copies per wave per batch
  static_assert(PF * wf_vec(WF) + ncp <= 63 && kRing2Batch * wf_vec(WF) <= 63, "vmcnt holds at most 63");
  extern __shared__ __align__(16) int8_t smem[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int ws = wave % SPB, hk = wave / SPB;             // strip of the block, K half
  const int sb = blockIdx.x * SPB;
  const int strip = sb + ws;
  const bool live = strip < a.n_strips;
  const int cstrip = min(strip, a.n_strips - 1);
  const int c16 = lane & 15, j = lane >> 4;
  const int G = a.G, Gh = G / 2;                          // the plan keeps G a multiple of 2 kRing2Batch
  const int64_t K = int64_t(G) * 128;
  const int nb = Gh / kRing2Batch;

  // Copies: chunk pc of a batch belongs to half pc / kHalfChunks, group u and
  // row r of it; every wave issues ncp copies (a wave past the last chunks
  // repeats them).  One descriptor over the M rows, loop-invariant lane
  // offsets, the batch a wave-uniform soffset; rows past M read row M-1.
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(a.x8, int(int64_t(a.M) * K));
  int coff[ncp];
#pragma unroll
  for (int k = 0; k < ncp; ++k) {
    const int base = min((k * NW + wave) * 64, kBatchChunks - 64);
    const int pc = base + lane;
    const int half = pc / kHalfChunks, ph = pc - half * kHalfChunks;
    const int lrow = ph >> 3;
    const int q = (ph & 7) ^ ((lrow >> 1) & 7);
    const int u = lrow / R, r = lrow - u * R;
    coff[k] = min(r, a.M - 1) * int(K) + (half * Gh + u) * 128 + q * 16;
  }
  auto copy_batch = [&](int bt) {
    int8_t* dst = smem + (bt & 1) * kBatchBytes;
    const int soff = min(bt, nb - 1) * (kRing2Batch * 128);
#pragma unroll
    for (int k = 0; k < ncp; ++k) {
      const int base = min((k * NW + wave) * 64, kBatchChunks - 64);
      buf_load_lds16(xrs, dst + base * 16, coff[k], soff);
    }
  };
  int8_t* meta_lds = smem + 2 * kBatchBytes;
  if constexpr (wf_group_meta(WF)) {
    const int m_chunks = min(SPB, a.n_strips - sb) * a.G4q * 4;
    const int m_last = ((m_chunks - 1) >> 6) << 6;
    const int nmp = ((m_chunks + 63) / 64 + NW - 1) / NW;
    const int8_t* msrc = reinterpret_cast<const int8_t*>(a.meta) + int64_t(sb) * a.G4q * 64;
    for (int k = 0; k < nmp; ++k) {
      const int base = min((k * NW + wave) * 64, m_last);
      const int pc = min(base + lane, m_chunks - 1);
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(msrc + pc * 16),
                                       (__attribute__((address_space(3))) void*)(meta_lds + base * 16), 16, 0, 0);
    }
  }
  const uint32_t* lmeta = reinterpret_cast<const uint32_t*>(meta_lds) + ws * a.G4q * 16 + c16;

  constexpr int kVec = wf_vec(WF);
  constexpr int kBlk = wf_block_bytes(WF);
  const int strip_bytes = G * kBlk;
  const int g0 = hk * Gh;  // first group of this wave's half
  const __amdgpu_buffer_rsrc_t wrs =
      make_rsrc(reinterpret_cast<const int8_t*>(a.qw) + int64_t(cstrip) * strip_bytes, live ? strip_bytes : 0);
  u32x4 bq[PF][kVec];
  auto load_b = [&](int g, u32x4 (&b)[kVec]) {  // g: group within the half
#pragma unroll
    for (int v = 0; v < kVec; ++v)
      b[v] = buf_load16<kCacheStream>(wrs, lane * 16 + v * 1024 + (g < Gh ? (g0 + g) * kBlk : kDeadOffset));
  };
  uint32_t S = 0, C = 0;
  if constexpr (WF == kWfPerChannel) meta_perchannel(a.meta8[cstrip * 16 + c16], S, C);

  copy_batch(0);
  QOQ_COMPILER_FENCE();
#pragma unroll
  for (int p = 0; p < PF; ++p) load_b(p, bq[p]);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(PF * kVec));
  __builtin_amdgcn_s_barrier();
  QOQ_COMPILER_FENCE();

  v4i acc[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i) acc[i] = v4i{0, 0, 0, 0};
  v4i fa[2][2][TM];
  uint32_t fm[2];
  const int hoff = hk * (kHalfChunks * 16);  // this half's tiles within a batch slot
  auto read_next = [&](v4i (&af)[2][TM], uint32_t& mw, const int8_t* slot, int u, int g) {
    read_group_frags<TM>(af, mw, slot + hoff + strip_lds_off(u * R + c16, j), slot + hoff + strip_lds_off(u * R + c16, j + 4),
                         wf_group_meta(WF) ? lmeta + ((g0 + min(g, Gh - 1)) >> 2) * 16 : reinterpret_cast<const uint32_t*>(slot));
  };
  auto compute = [&](const v4i (&af)[2][TM], uint32_t mw, int g, const u32x4 (&bc)[kVec]) {
    if constexpr (wf_group_meta(WF)) meta_g128<WF>((mw >> (8 * ((g0 + g) & 3))) & 0xffu, S, C);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const v4i bf = b_op16<WF>(bc, h, S, C);
#pragma unroll
      for (int i = 0; i < TM; ++i) acc[i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[h][i], bf, acc[i], 0, 0, 0);
    }
  };
  static_assert(kRing2Batch % 2 == 0, "fragment buffers alternate within a batch");
  read_next(fa[0], fm[0], smem, 0, 0);
  for (int bt = 0; bt < nb; ++bt) {
    copy_batch(bt + 1);
    QOQ_COMPILER_FENCE();
    const int8_t* slot = smem + (bt & 1) * kBatchBytes;
    // each group waits for its weights: younger are the next PF - 1 groups'
    // loads and this batch's copies (the weights of a batch's groups were
    // loaded during the batch before)
    static_for<kRing2Batch>([&](auto uc) {
      constexpr int u = decltype(uc)::value;
      const int g = bt * kRing2Batch + u;
      __builtin_amdgcn_s_waitcnt(waitcnt_vm((PF - 1) * kVec + ncp));
      __builtin_amdgcn_sched_barrier(0);
      compute(fa[u & 1], fm[u & 1], g, bq[u]);
      QOQ_COMPILER_FENCE();
      load_b(g + PF, bq[u]);
      if constexpr (u + 1 < kRing2Batch) read_next(fa[(u + 1) & 1], fm[(u + 1) & 1], slot, u + 1, g + 1);
      QOQ_COMPILER_FENCE();
    });
    // the next batch's copies were issued before this batch's weight loads
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(kRing2Batch * kVec));
    lds_barrier();
    read_next(fa[0], fm[0], smem + ((bt + 1) & 1) * kBatchBytes, 0, (bt + 1) * kRing2Batch);
  }

  // the trailing copies land, then half 1 parks its accumulators (16-byte
  // records [strip][i][lane]) and half 0 adds them
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  __syncthreads();
  v4i* red = reinterpret_cast<v4i*>(smem);
  if (hk == 1) {
#pragma unroll
    for (int i = 0; i < TM; ++i) red[(ws * TM + i) * 64 + lane] = acc[i];
  }
  __syncthreads();
  if (hk == 1 || !live) return;
#pragma unroll
  for (int i = 0; i < TM; ++i) acc[i] += red[(ws * TM + i) * 64 + lane];

  const float sc = I32OUT ? 0.0f : col_scale(a, strip * 16 + c16);
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    float sxv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) sxv[r] = I32OUT ? 0.0f : row_scale(a, 16 * i + 4 * j + r);
#pragma unroll
    for (int r = 0; r < 4; ++r) store_out<I32OUT>(a, 16 * i + 4 * j + r, strip * 16 + c16, acc[i][r], sxv[r], sc);
  }
}

// ---------------------------------------------------------------------------
// gemm_large: M > 64 (prefill, compute-bound).  Block = WM x WN waves, wave
// tile = TM*32 rows x TN*32 columns of v_mfma_i32_32x32x32_i8.
//
// Activations: a ring of kLargeRing tiles of BM rows x 128 bytes in LDS, the
// tile of group g in slot g % kLargeRing.  Each tile is copied global -> LDS
// by buffer loads with an LDS destination (no registers, no LDS write
// instructions), three groups ahead.  Lane i of a copy instruction writes LDS
// chunk base + i, so every lane fetches the global chunk that the swizzled
// layout keeps at that position.
// Weights: global -> VGPR, D groups ahead, dequantized in registers.
// A step multiplies one group per set of waves (one set unless K is split
// inside the block); the ring holds four steps' tiles, copied three steps
// ahead, with one barrier per step (see the kernel).
constexpr int kLargeRing = 4;

template <int BM, int THREADS>
struct ATile {
  static constexpr int kChunks = BM * 8;
  static constexpr int kPer = kChunks / THREADS;
  static_assert(kChunks % THREADS == 0, "A tile must split evenly over the block");
};



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

// Multiply one 128-wide K group (4 K steps of 32) from LDS tile `lds`.  A
// fragments are double-buffered across the steps: the reads of step s+1 are
// issued before the multiplies of step s, and during the last step the reads
// are those of step 0 of the next group (tile `lds_next`), left in af0.
// Weight slot 0 of a column tile holds K steps 0 and 2 (low / high half),
// slot 1 holds steps 1 and 3.
template <int TM, int TN, int WF, bool STAGE>
__device__ __forceinline__ void large_group(v16i (&acc)[TM][TN], const int8_t* lds, const int8_t* lds_next,
                                            v4i (&af0)[TM], const u32x4 (&b)[TN][wf_large_vec(WF)],
                                            const uint32_t (&m)[TN], uint32_t (&S)[TN], uint32_t (&C)[TN], int g,
                                            int row0, int c32, int hh) {
  if constexpr (wf_group_meta(WF)) {
#pragma unroll
    for (int t = 0; t < TN; ++t) meta_g128<WF>((m[t] >> (8 * (g & 3))) & 0xffu, S[t], C[t]);
  }
  v4i af1[TM];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    v4i (&cur)[TM] = (s & 1) ? af1 : af0;
    v4i (&nxt)[TM] = (s & 1) ? af0 : af1;
#pragma unroll
    for (int i = 0; i < TM; ++i)
      nxt[i] = *reinterpret_cast<const v4i*>((s < 3 ? lds : lds_next) +
                                             lds_off(row0 + i * 32 + c32, s < 3 ? 2 * (s + 1) + hh : hh));
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      const v4i bf = b_op32<WF>(b[t], s, S[t], C[t]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
        acc[i][t] = STAGE ? __builtin_amdgcn_mfma_i32_32x32x32_i8(bf, cur[i], acc[i][t], 0, 0, 0)
                          : __builtin_amdgcn_mfma_i32_32x32x32_i8(cur[i], bf, acc[i][t], 0, 0, 0);
    }
  }
}

// Dynamic LDS of the large kernel: the activation ring (the epilogue reuses
// its first BM floats for the row scales).
constexpr size_t large_lds_bytes(int bm) { return size_t(kLargeRing) * size_t(bm) * 128; }

// KI > 1 splits K inside the block: KI sets of WM x WN waves take the groups
// of a step in turn (set k multiplies group KI s + k of step s), so each wave
// can hold a taller tile (fewer dequantizations per MFMA) at the same number
// of blocks; the sets' INT32 partials are added exactly through LDS at the end.
template <int WM, int WN, int TM, int TN, int D, int KI, int WF, bool I32OUT, bool STAGE>
__global__ __launch_bounds__(64 * WM * WN * KI) void gemm_large_kernel(GemmArgs a) {
  static_assert(!STAGE || !I32OUT, "the staged epilogue writes FP16");
  constexpr int THREADS = 64 * WM * WN * KI;
  constexpr int BM = WM * TM * 32;
  constexpr int BN = WN * TN * 32;
  constexpr int TILE = BM * 128;
  constexpr int NA1 = ATile<BM, THREADS>::kPer;  // copies per thread per tile
  constexpr int NA = NA1 * KI;                   // copies per thread per step
  constexpr int NB = kLargeRing * KI;            // ring slots (tiles)
  extern __shared__ __align__(16) int8_t smem[];

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kset = wave / (WM * WN), wl = wave % (WM * WN);
  const int wm = wl / WN, wn = wl % WN;
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

  // Groups past the range are clamped to the last one (their copies and loads
  // stay inside the operands and are never multiplied).
  const int n = ge - gb;               // groups of this split
  const int nsteps = (n + KI - 1) / KI;
  auto gcl = [&](int l) { return gb + min(l, n - 1); };
  auto slot = [&](int l) { return smem + (l % NB) * TILE; };

  // Activation copies.  Copy instruction i of a thread moves LDS chunk p =
  // i * THREADS + threadIdx.x of the tile: row p / 8, stored position p % 8,
  // which holds the row's logical chunk (p % 8) ^ ((row >> 1) & 7).  Rows past
  // M read row M-1.  One descriptor over the block's rows; the group is a
  // wave-uniform soffset.

  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x8 + int64_t(m0) * K, int(min(BM, a.M - m0) * K));
  int aoff[NA1];
#pragma unroll
  for (int i = 0; i < NA1; ++i) {
    const int p = threadIdx.x + i * THREADS;
    const int row = p >> 3, kc = (p & 7) ^ ((row >> 1) & 7);
    aoff[i] = (min(m0 + row, a.M - 1) - m0) * int(K) + kc * 16;
  }
  // the KI tiles of step s (groups KI s .. KI s + KI - 1)
  auto a_copy = [&](int s) {
#pragma unroll
    for (int q = 0; q < KI; ++q) {
      const int l = KI * s + q;
      int8_t* dst = slot(l);
#pragma unroll
      for (int i = 0; i < NA1; ++i) buf_load_lds16(xr, dst + (i * THREADS + wave * 64) * 16, aoff[i], gcl(l) * 128);
    }
  };

  // Weights and group metadata: one descriptor over the (at most 2 TN)
  // strips of this wave's columns.  UINT4 blocks: lane (c32, hh) loads slots
  // c16 + 16 hh and c16 + 16 (2 + hh), K steps {0, 2} and {1, 3}; INT8 blocks:
  // K step st is K chunk 2 st + hh = 16 j + 64 h, slot c16 + 16 j + 64 h.
  // Per-lane offsets are loop-invariant; strips past N read the last strip.
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
      const int sl = WF == kWfW8 ? c16 + 16 * ((2 * v + hh) & 3) + 64 * ((2 * v + hh) >> 2) : c16 + 16 * (2 * v + hh);
      woff[t][v] = sb + sl * 16;
    }
  }
  const __amdgpu_buffer_rsrc_t mr =
      wf_group_meta(WF)
          ? make_rsrc(reinterpret_cast<const int8_t*>(a.meta) + int64_t(sfirst) * a.G4q * 64, nws * a.G4q * 64)
          : make_rsrc(a.qw, 0);
  int moff[TN];
#pragma unroll
  for (int t = 0; t < TN; ++t) moff[t] = ((strip[t] - sfirst) * a.G4q * 16 + c16) * 4;
  u32x4 rb[D][TN][kVec];
  uint32_t rm[D][TN];
  auto b_ld = [&](u32x4 (&b)[TN][kVec], uint32_t (&m)[TN], int g) {
#pragma unroll
    for (int t = 0; t < TN; ++t) {
#pragma unroll
      for (int v = 0; v < kVec; ++v) b[t][v] = buf_load16s<0>(wr, woff[t][v], g * kBlk);
      if constexpr (wf_group_meta(WF)) m[t] = buf_load4s(mr, moff[t], (g >> 2) * 64);
    }
  };
  // global loads of one b_ld, for the hand-written waits
  constexpr int kBLoads = TN * kVec + (wf_group_meta(WF) ? TN : 0);
  static_assert(NA + 2 * kBLoads <= 63 && NA + D * kBLoads <= 63, "vmcnt holds at most 63");

  // Prologue: the tiles of steps 0 and 1, the weight ring, the tiles of step
  // 2.  Steps 0 and 1 must have landed before the barrier (step 0 reads the
  // first fragments of both).
  a_copy(0);
  a_copy(1);
#pragma unroll
  for (int dd = 0; dd < D; ++dd) b_ld(rb[dd], rm[dd], gcl(KI * dd + kset));
  a_copy(2);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(NA + D * kBLoads));
  lds_barrier();
  v4i af0[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i) af0[i] = *reinterpret_cast<const v4i*>(slot(kset) + lds_off(row0 + i * 32 + c32, hh));

  // Step s: copy the tiles of step s+3 into the slots of step s-1, multiply
  // this wave's group of step s (reading the first fragments of its group of
  // step s+1), refill the weight slot with its group of step s+D, wait for the
  // tiles of step s+2 and meet the other waves.  After the barrier every wave
  // is done with step s's slots and the tiles of step s+2 are visible.
  // A set whose group lies past the range (odd group counts) skips it.
  auto step = [&](int s, int u) {
    a_copy(s + 3);
    QOQ_COMPILER_FENCE();
    const int l = KI * s + kset;
    if (KI == 1 || l < n)
      large_group<TM, TN, WF, STAGE>(acc, slot(l), slot(l + KI), af0, rb[u], rm[u], S, C, gb + l, row0, c32, hh);
    QOQ_COMPILER_FENCE();
    b_ld(rb[u], rm[u], gcl(KI * (s + D) + kset));
    // the tiles of step s+2 were issued one step ago; after them come the
    // weights of the last step, the tiles of step s+3 and this step's weights
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(NA + 2 * kBLoads));
    lds_barrier();
  };
  int s0 = 0;
  for (; s0 + D <= nsteps; s0 += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) step(s0 + u, u);
  }
  // the last nsteps % D steps' weights are already in the ring
  const int rem = nsteps - s0;
#pragma unroll
  for (int u = 0; u < D; ++u)
    if (u < rem) step(s0 + u, u);

  // the trailing (clamped) copies land before the LDS is reused
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  lds_barrier();
  if constexpr (KI > 1) {
    // exact sum of the K sets' partials: set k > 0 parks its accumulators as
    // 16-byte records [set-1][wave][i][t][4][lane]; set 0 adds them
    v4i* red = reinterpret_cast<v4i*>(smem);
    if (kset > 0) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int t = 0; t < TN; ++t)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            red[(((((kset - 1) * WM * WN + wl) * TM + i) * TN + t) * 4 + q) * 64 + lane] =
                v4i{acc[i][t][4 * q], acc[i][t][4 * q + 1], acc[i][t][4 * q + 2], acc[i][t][4 * q + 3]};
    }
    __syncthreads();
    if (kset == 0) {
#pragma unroll
      for (int k2 = 1; k2 < KI; ++k2)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int t = 0; t < TN; ++t)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const v4i v = red[(((((k2 - 1) * WM * WN + wl) * TM + i) * TN + t) * 4 + q) * 64 + lane];
#pragma unroll
              for (int e = 0; e < 4; ++e) acc[i][t][4 * q + e] += v[e];
            }
    }
  }
  if constexpr (STAGE) {
    // Staged epilogue (set 0; FP16 output rows 16-byte aligned, which the
    // launch checks).  The weights were the MFMA's first operand, so tile
    // (i, t) holds the transposed product: lane (c32, hh) holds token row
    // row0 + 32 i + c32 and, in values 4 q .. 4 q + 3, the four consecutive
    // columns 32 t + 8 q + 4 hh .. + 3 of the wave's columns.  The FP16
    // results of 32 rows at a time go through a wave-private LDS tile
    // (16-byte chunks XOR-swizzled by row, as the activation tiles) and leave
    // as whole 16-byte row segments: at 64 columns a wave, one store covers 8
    // rows of full 128-byte lines, against 2 rows of 64 bytes for the 2-byte
    // stores of the plain epilogue.  Row and column scales go through LDS,
    // past the partials, before the first store.
    constexpr int WTN = TN * 32;        // columns of a wave
    constexpr int CPR = WTN / 8;        // 16-byte chunks per staged row
    const int nb0 = n0 - wn * TN * 32;  // first column of the block
    float* sxs = reinterpret_cast<float*>(smem + (KI > 1 ? (KI - 1) * WM * WN * TM * TN * 4096 : 0));
    float* scs = sxs + BM;
    int8_t* stg = reinterpret_cast<int8_t*>(scs + BN) + wl * (32 * WTN * 2);
    for (int r = threadIdx.x; r < BM; r += THREADS) sxs[r] = row_scale(a, m0 + r);
    for (int c = threadIdx.x; c < BN; c += THREADS) scs[c] = col_scale(a, nb0 + c);
    __syncthreads();
    if (kset != 0) return;
    float4 cs[TN][4];
#pragma unroll
    for (int t = 0; t < TN; ++t)
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) cs[t][qq] = *reinterpret_cast<const float4*>(scs + wn * WTN + 32 * t + 8 * qq + 4 * hh);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const float sxr = sxs[row0 + i * 32 + c32];
      const int sw = (c32 >> 1) & (CPR - 1);
#pragma unroll
      for (int t = 0; t < TN; ++t)
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const float sv[4] = {cs[t][qq].x, cs[t][qq].y, cs[t][qq].z, cs[t][qq].w};
          unsigned short h[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            h[e] = __half_as_ushort(__float2half_rn(static_cast<float>(acc[i][t][4 * qq + e]) * sxr * sv[e]));
          *reinterpret_cast<uint2*>(stg + c32 * (CPR * 16) + (((4 * t + qq) ^ sw) << 4) + hh * 8) =
              make_uint2(uint32_t(h[0]) | (uint32_t(h[1]) << 16), uint32_t(h[2]) | (uint32_t(h[3]) << 16));
        }
      // read back whole chunks (this wave's LDS operations run in order; the
      // next tile's writes come after these reads)
#pragma unroll
      for (int k = 0; k < CPR / 2; ++k) {
        const int f = k * 64 + lane;
        const int rr = f / CPR, c = f % CPR;
        const uint4 v = *reinterpret_cast<const uint4*>(stg + rr * (CPR * 16) + ((c ^ ((rr >> 1) & (CPR - 1))) << 4));
        const int row = m0 + row0 + i * 32 + rr;
        const int col = n0 + 8 * c;
        if (row >= a.M) continue;
        unsigned short* o = static_cast<unsigned short*>(a.out) + int64_t(row) * a.ldo + col;
        if (col + 7 < a.N) {
          *reinterpret_cast<uint4*>(o) = v;
        } else {  // the row's last, partial chunk
          const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (col + e < a.N) o[e] = static_cast<unsigned short>(w[e >> 1] >> (16 * (e & 1)));
        }
      }
    }
  } else {
    // Epilogue (set 0): lane holds column lane%32 and rows 8*(r/4) + 4*(lane/32)
    // + r%4.  Every scale is fetched before the first store: stores count on
    // the same in-order counter as global loads, so a load issued after a store
    // waits for it.  The block's row scales go through LDS, past the partials.
    float sc[TN];
  #pragma unroll
    for (int t = 0; t < TN; ++t) sc[t] = I32OUT ? 0.0f : col_scale(a, n0 + 32 * t + c32);
    float* sxs = reinterpret_cast<float*>(smem + (KI > 1 ? (KI - 1) * WM * WN * TM * TN * 4096 : 0));
    if constexpr (!I32OUT) {
      for (int r = threadIdx.x; r < BM; r += THREADS) sxs[r] = row_scale(a, m0 + r);
      __syncthreads();
    }
    if (kset != 0) return;
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
// or 8 waves.
#ifndef QOQ_S1PF
#define QOQ_S1PF 4
#endif
constexpr int kStripWavesTarget = 1024;  // 4 waves per CU

// K parts (waves) per skinny block: 8 for the UINT4 formats when every part
// keeps at least 8 groups, else 4 (INT8 weights need twice the registers per
// group in flight, which two waves per SIMD cannot hold).  Ring depth: 2
// groups with 8 waves, 4 with 4 (2 for INT8 blocks, twice as large): the same
// bytes in flight per SIMD.
constexpr int kSkinnyKs8MinGroups = 64;
constexpr int skinny_ks(bool uint4, int G) { return uint4 && G >= kSkinnyKs8MinGroups ? 8 : 4; }
constexpr int skinny_pf(int wf, int ks) { return ks == 8 ? 2 : 4 / wf_vec(wf); }

template <int TM, int TN, int KS, int WF, bool I32>
hipError_t launch_skinny(const GemmArgs& a, hipStream_t st) {
  const dim3 grid((a.n_strips + TN - 1) / TN, (a.M + TM * 16 - 1) / (TM * 16));
  hipLaunchKernelGGL((gemm_skinny_kernel<TM, TN, KS, skinny_pf(WF, KS), WF, I32>), grid, dim3(64 * KS), 0, st, a);
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

// Most strips per skinny block: 8, or 7 with 64-row tiles (eight would not
// fit the register file beside four row tiles of accumulators).
constexpr int skinny_tn_max(int tm) { return tm >= 4 ? 7 : 8; }

// launch_skinny with TN = tn and KS = ks, instantiated for 1 <= TN <= T only
template <int TM, int WF, bool I32, int T>
hipError_t launch_skinny_upto(int tn, int ks, const GemmArgs& a, hipStream_t st) {
  if constexpr (T > 1) {
    if (tn < T) return launch_skinny_upto<TM, WF, I32, T - 1>(tn, ks, a, st);
  }
  if constexpr (WF != kWfW8) {
    if (ks == 8) return launch_skinny<TM, T, 8, WF, I32>(a, st);
  }
  return launch_skinny<TM, T, 4, WF, I32>(a, st);
}

// Dynamic LDS of the strip kernel: the activations, or the K-part partial
// sums, whichever is larger.
constexpr size_t kStripMaxLds = 160 * 1024;
inline size_t strip_lds_bytes_rows(int G, int rp, int spb, int ks, bool group_meta) {
  const size_t act = size_t(round_up(int64_t(G) * rp * 8 * 16, 1024));
  const size_t meta = group_meta ? size_t(round_up(int64_t(spb) * round_up(G, 4) / 4 * 64, 1024)) : 0;
  const size_t red = size_t(spb) * size_t(ks - 1) * 1024;
  return act + meta > red ? act + meta : red;
}
// LDS rows per group of the strip kernel's activations for R token rows: 16
// (group-major copies) from 8 rows on when that fits, else R (dense).
inline int strip_rows(int G, int R, int spb, int ks, bool group_meta) {
  return R >= 8 && strip_lds_bytes_rows(G, 16, spb, ks, group_meta) <= kStripMaxLds ? 16 : R;
}
inline size_t strip_lds_bytes(int G, int R, int spb, int ks, bool group_meta) {
  return strip_lds_bytes_rows(G, strip_rows(G, R, spb, ks, group_meta), spb, ks, group_meta);
}

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
  const int rp = strip_rows(a.G, a.M < 16 ? a.M : 16, spb, ks, wf_group_meta(WF));
  hipLaunchKernelGGL(fn, grid, dim3(64 * spb * ks), lds, st, a, spb, ks, rp);
  return hipGetLastError();
}

// Up to 16 rows: the strip kernel when the activations fit in LDS, else the
// K-split skinny kernel.  Strips per block as for the skinny kernel (rounds of
// 256 blocks); the K split fills a block up to 8 waves.  Returns false when
// the activations do not fit.
inline bool plan_strip(int64_t M, int n_strips, int G, bool group_meta, int* spb, int* ks, size_t* lds) {
  const int R = M < 16 ? int(M) : 16;
  *spb = pick_skinny_tn(n_strips, 1, 8);
  *ks = 8 / *spb;
  if (*ks < 1) *ks = 1;
  *lds = strip_lds_bytes(G, R, *spb, *ks, group_meta);
  return *lds <= kStripMaxLds;
}

// Row tiles of the ring kernel for M rows (M <= 64): 1, 2 or 4.
constexpr int ring_tm(int64_t M) { return M <= 16 ? 1 : (M <= 32 ? 2 : 4); }
inline size_t ring_lds_bytes(int tm, int G, int spb, bool group_meta) {
  const size_t meta = group_meta ? size_t(round_up(int64_t(spb) * round_up(G, 4) / 4 * 64, 1024)) : 0;
  return 2 * size_t(kRingBatch) * size_t(tm) * 16 * 128 + meta;
}
// Up to 64 rows, the ring kernel when one strip per wave and at least
// QOQ_RING_MIN_SPB strips per block still give about a block per CU (wide N:
// the decode projections) and K is a whole number of batches (and of weight
// rings); otherwise the K-split skinny kernel, whose waves share a strip's K
// range.
#ifndef QOQ_RING_MIN_SPB
#define QOQ_RING_MIN_SPB 5
#endif
// Longest per-wave chain (groups x row tiles) the ring kernel takes: a wave
// runs all G groups of its strip in sequence, against G / 8 groups of seven
// strips in the skinny kernel; past this the skinny kernel's shorter chains
// win (64 x 16384 x 28672: 55 us skinny, 60 us ring).
#ifndef QOQ_RING_MAX_WORK
#define QOQ_RING_MAX_WORK 256
#endif
// groups of weights in flight per wave of the ring kernel
#ifndef QOQ_RING_PF
#define QOQ_RING_PF 4
#endif
constexpr int kRingGroupStep = QOQ_RING_PF > kRingBatch ? QOQ_RING_PF : kRingBatch;
// From QOQ_RING2_MIN_G groups on, and for row tiles of up to 32 rows, the
// ring kernel splits each strip's K range over two waves (gemm_ring2_kernel,
// reported as 2 K parts): twice the waves a CU for the same work.  Shorter K
// keeps one wave a strip (a half would run a single batch), and so do 64-row
// tiles (even against one wave a strip across boxes).
#ifndef QOQ_RING2_MIN_G
#define QOQ_RING2_MIN_G 64
#endif
inline size_t ring2_lds_bytes(int tm, int G, int spb, bool group_meta) {
  const size_t meta = group_meta ? size_t(round_up(int64_t(spb) * round_up(G, 4) / 4 * 64, 1024)) : 0;
  return 2 * size_t(ring2_batch_bytes(tm)) + meta;
}
inline bool plan_ring(int64_t M, int n_strips, int G, bool group_meta, int* spb, int* ks, size_t* lds) {
  *spb = pick_skinny_tn(n_strips, 1, 8);
  *ks = G >= QOQ_RING2_MIN_G && G % (2 * kRing2Batch) == 0 && ring_tm(M) <= 2 ? 2 : 1;
  *lds = *ks == 2 ? ring2_lds_bytes(ring_tm(M), G, *spb, group_meta) : ring_lds_bytes(ring_tm(M), G, *spb, group_meta);
  return *spb >= QOQ_RING_MIN_SPB && G % kRingGroupStep == 0 && G * ring_tm(M) <= QOQ_RING_MAX_WORK &&
         *lds <= kStripMaxLds;
}

template <int TM, int SPB, int WF, bool I32>
hipError_t launch_ring_spb(const GemmArgs& a, int ks, hipStream_t st) {
  if (ks == 2) {
    auto* f2 = gemm_ring2_kernel<TM, SPB, kRing2Batch, WF, I32>;
    static const hipError_t attr2 = hipFuncSetAttribute(reinterpret_cast<const void*>(f2),
                                                        hipFuncAttributeMaxDynamicSharedMemorySize, int(kStripMaxLds));
    if (attr2 != hipSuccess) return attr2;
    hipLaunchKernelGGL(f2, dim3((a.n_strips + SPB - 1) / SPB), dim3(128 * SPB),
                       ring2_lds_bytes(TM, a.G, SPB, wf_group_meta(WF)), st, a);
    return hipGetLastError();
  }
  auto* fn = gemm_ring_kernel<TM, SPB, QOQ_RING_PF, WF, I32>;
  const size_t lds = ring_lds_bytes(TM, a.G, SPB, wf_group_meta(WF));
  if (lds > 64 * 1024) {
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(kStripMaxLds));
    if (attr != hipSuccess) return attr;
  }
  const dim3 grid((a.n_strips + SPB - 1) / SPB);
  hipLaunchKernelGGL(fn, grid, dim3(64 * SPB), lds, st, a);
  return hipGetLastError();
}
// strips per block: QOQ_RING_MIN_SPB .. 8 (the plan's range; with fewer
// strips a block leaves a SIMD with a single wave and the skinny kernel,
// whose waves split K, is faster)
template <int TM, int WF, bool I32>
hipError_t launch_ring(const GemmArgs& a, int spb, int ks, hipStream_t st) {
  static_assert(QOQ_RING_MIN_SPB >= 5, "ring blocks of 5 to 8 strips are instantiated");
  switch (spb) {
    case 5: return launch_ring_spb<TM, 5, WF, I32>(a, ks, st);
    case 6: return launch_ring_spb<TM, 6, WF, I32>(a, ks, st);
    case 7: return launch_ring_spb<TM, 7, WF, I32>(a, ks, st);
    default: return launch_ring_spb<TM, 8, WF, I32>(a, ks, st);
  }
}

// Large-M plans.  Tile 0: the big tile (128 x 512); tile 1: the small one
// (64 x 256), for problems with fewer than 192 big tiles; tile 2: the K-set
// tile (128 x 128), in place of the small one when every block runs at least
// QOQ_KSET_MIN_GROUPS groups (the sets' final reduction and the shorter runs
// per set cost more than they save below that).
struct LargePlan {
  int tile;    // 0, 1 or 2
  int ksplit;  // K splits
};

constexpr int kBigBM = QOQ_LWM * QOQ_LTM * 32, kBigBN = QOQ_LWN * QOQ_LTN * 32;
constexpr int kSmallBM = QOQ_SWM * QOQ_STM * 32, kSmallBN = QOQ_SWN * QOQ_STN * 32;

inline int64_t tiles_of(int64_t M, int64_t N_pad, int bm, int bn) { return ((M + bm - 1) / bm) * ((N_pad + bn - 1) / bn); }

// Pick a tile, then the K split with the least estimated time: ceil(blocks /
// 256) rounds of blocks, each G / ksplit groups long, plus, for a split, the
// INT32 partials written and read again by the reduction (about 5 TB/s)
// and its launch.  Per-group block times are the ones measured with every CU
// busy: about 0.8 us for a small tile and 2.2 us for a big one.  Every split
// keeps at least 4 groups (512 channels).
inline LargePlan plan_large(int64_t M, int64_t N, int64_t K) {
  const int64_t N_pad = round_up(N, kStrip);
  const int64_t G = K / kGroup;
  LargePlan p{0, 1};
  const int64_t big = tiles_of(M, N_pad, kBigBM, kBigBN);
  if (big < 192) p.tile = 1;
  const int64_t tiles = p.tile ? tiles_of(M, N_pad, kSmallBM, kSmallBN) : big;
  const int64_t group_ns = p.tile ? 800 : 2200;
  auto cost_ns = [&](int64_t ks) {
    const int64_t run = ((tiles * ks + 255) / 256) * ((G + ks - 1) / ks) * group_ns;
    return ks > 1 ? run + ks * M * N_pad * 8 / 5000 + 2000 : run;
  };
  for (int64_t ks = 2; G / ks >= 4; ks *= 2)
    if (cost_ns(ks) < cost_ns(p.ksplit)) p.ksplit = int(ks);
  if (p.tile == 1 && G / p.ksplit >= QOQ_KSET_MIN_GROUPS) p.tile = 2;
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

// The launch plan of one GEMM call.  kernel: the kernel family; tile: strips
// per block (strip and skinny kernels) or the large-M tile (0 big, 1 small,
// 2 K-set); ksplit: K parts per block (strip and skinny kernels) or K splits
// across blocks (large kernel).
enum GemmKernel { kPlanStrip = 0, kPlanSkinny16 = 1, kPlanSkinny32 = 2, kPlanSkinny64 = 3, kPlanLarge = 4, kPlanRing = 5 };
struct GemmPlan {
  int kernel, tile, ksplit;
};

// group_meta: per-group metadata (g128); uint4: UINT4 weights (else INT8).
inline GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K, bool group_meta, bool uint4 = true) {
  const int n_strips = int(round_up(N, kStrip) / kStrip);
  const int G = int(K / kGroup);
  const int ks = skinny_ks(uint4, G);
  if (M <= 16) {
    int spb, sks;
    size_t lds;
    if (plan_strip(M, n_strips, G, group_meta, &spb, &sks, &lds)) return {kPlanStrip, spb, sks};
  }
  if (M <= kSkinnyMaxM) {
    int spb, rks;
    size_t lds;
    if (plan_ring(M, n_strips, G, group_meta, &spb, &rks, &lds)) return {kPlanRing, spb, rks};
  }
  if (M <= 16) return {kPlanSkinny16, pick_skinny_tn(n_strips, int((M + 15) / 16), skinny_tn_max(1)), ks};
  if (M <= 32) return {kPlanSkinny32, pick_skinny_tn(n_strips, int((M + 31) / 32), skinny_tn_max(2)), ks};
  if (M <= kSkinnyMaxM || skinny_mid(M, N))
    return {kPlanSkinny64, pick_skinny_tn_rows(n_strips, int((M + 63) / 64), skinny_tn_max(4)), ks};
  const LargePlan p = plan_large(M, N, K);
  return {kPlanLarge, p.tile, p.ksplit};
}

inline size_t workspace_bytes_of(int64_t M, int64_t N, int64_t K) {
  const GemmPlan p = plan_gemm(M, N, K, false);
  return p.kernel == kPlanLarge && p.ksplit > 1
             ? size_t(p.ksplit) * size_t(M) * size_t(round_up(N, kStrip)) * sizeof(int)
             : 0;
}

template <int WM, int WN, int TM, int TN, int D, int KI, int WF, bool I32>
hipError_t launch_large(const GemmArgs& a, hipStream_t st) {
  constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
  constexpr size_t lds = large_lds_bytes(BM) * KI;
  // the staged FP16 epilogue: the K sets' partials, the block's row and
  // column scales, then one 32-row tile per wave of a set
  static_assert(size_t(KI > 1 ? (KI - 1) * WM * WN * TM * TN * 4096 : 0) + size_t(BM + BN) * 4 +
                        size_t(WM * WN) * 32 * TN * 32 * 2 <= lds,
                "the staged epilogue fits the ring");
  // FP16 rows 16-byte aligned: the staged epilogue (whole 16-byte row
  // segments); otherwise, and for INT32 output, the plain one
  const bool stage = !I32 && reinterpret_cast<uintptr_t>(a.out) % 16 == 0 && (a.ldo * 2) % 16 == 0;
  auto* fn = stage ? gemm_large_kernel<WM, WN, TM, TN, D, KI, WF, I32, !I32>
                   : gemm_large_kernel<WM, WN, TM, TN, D, KI, WF, I32, false>;
  if (lds > 64 * 1024) {
    static const hipError_t attr0 = hipFuncSetAttribute(
        reinterpret_cast<const void*>(gemm_large_kernel<WM, WN, TM, TN, D, KI, WF, I32, false>),
        hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    static const hipError_t attr1 = hipFuncSetAttribute(
        reinterpret_cast<const void*>(gemm_large_kernel<WM, WN, TM, TN, D, KI, WF, I32, !I32>),
        hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (attr0 != hipSuccess) return attr0;
    if (attr1 != hipSuccess) return attr1;
  }
  const dim3 grid((a.n_strips * 16 + BN - 1) / BN, (a.M + BM - 1) / BM, a.ksplit);
  hipLaunchKernelGGL(fn, grid, dim3(64 * WM * WN * KI), lds, st, a);
  return hipGetLastError();
}

template <int WF, bool I32>
hipError_t launch_large_tile(int tile, const GemmArgs& a, hipStream_t st) {
  if (tile == 0) return launch_large<QOQ_LWM, QOQ_LWN, QOQ_LTM, QOQ_LTN, QOQ_LD, 1, WF, I32>(a, st);
  if (tile == 1) return launch_large<QOQ_SWM, QOQ_SWN, QOQ_STM, QOQ_STN, QOQ_SD, 1, WF, I32>(a, st);
  return launch_large<QOQ_KWM, QOQ_KWN, QOQ_KTM, QOQ_KTN, QOQ_SD, QOQ_KKI, WF, I32>(a, st);
}

template <int WF, bool I32>
hipError_t dispatch(const GemmArgs& a0, void* ws, hipStream_t st) {
  const GemmPlan p = plan_gemm(a0.M, a0.N, int64_t(a0.G) * kGroup, wf_group_meta(WF), WF != kWfW8);
  switch (p.kernel) {
    case kPlanStrip: {
      const size_t lds = strip_lds_bytes(a0.G, a0.M < 16 ? a0.M : 16, p.tile, p.ksplit, wf_group_meta(WF));
      return launch_strip<WF, I32>(a0, p.tile, p.ksplit, lds, st);
    }
    case kPlanSkinny16: return launch_skinny_upto<1, WF, I32, skinny_tn_max(1)>(p.tile, p.ksplit, a0, st);
    case kPlanSkinny32: return launch_skinny_upto<2, WF, I32, skinny_tn_max(2)>(p.tile, p.ksplit, a0, st);
    case kPlanSkinny64: return launch_skinny_upto<4, WF, I32, skinny_tn_max(4)>(p.tile, p.ksplit, a0, st);
    case kPlanRing: {
      const int tm = ring_tm(a0.M);
      if (tm == 1) return launch_ring<1, WF, I32>(a0, p.tile, p.ksplit, st);
      if (tm == 2) return launch_ring<2, WF, I32>(a0, p.tile, p.ksplit, st);
      return launch_ring<4, WF, I32>(a0, p.tile, p.ksplit, st);
    }
    default: break;
  }
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
