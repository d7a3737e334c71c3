// W4A8 GEMM for gfx950 (MI355X): UINT4 weights dequantized to INT8 in
// registers, INT8 MFMA with INT32 accumulation, fused FP32 scale epilogue.
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
// Two kernels share the packed layout (see qoq.h):
//   gemm16: v_mfma_i32_16x16x64_i8, 16-row M tiles; for skinny M (decode).
//   gemm32: v_mfma_i32_32x32x32_i8, 32x32 tiles; for M > 64 (prefill).
// The activation tile of each 128-wide K group is staged in LDS (XOR-swizzled
// 16-byte chunks, double-buffered); weights go global -> VGPR directly and are
// prefetched a group ahead.  Both MFMA operands use the same K order per
// (lane group, byte), so the contraction is exact whatever order the matrix
// unit walks K in.

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include "qoq_internal.h"

namespace qoq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

__device__ __forceinline__ uint32_t pk_mad_u16(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t d;
  asm("v_pk_mad_u16 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
  return d;
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

// Metadata byte -> (S, C) operands of the dequantization.
__device__ __forceinline__ void meta_g128(uint32_t mbyte, uint32_t& S, uint32_t& C) {
  const uint32_t s1 = (mbyte & 15u) + 1u;
  const uint32_t z = mbyte >> 4;
  const uint32_t c = 128u - z * s1;
  S = s1 * 0x00010001u;
  C = c * 0x01010101u;
}
__device__ __forceinline__ void meta_perchannel(uint32_t z, uint32_t& S, uint32_t& C) {
  S = 0x00010001u;
  C = (128u - z) * 0x01010101u;
}

// LDS tile of BM rows x 128 bytes; 16-byte chunk kc of row r lives at chunk
// kc ^ (r & 7) so that 8 consecutive rows reading the same K chunk hit
// different banks.
__device__ __forceinline__ int lds_off(int row, int kc) { return row * 128 + ((kc ^ (row & 7)) << 4); }

template <int BM, int THREADS>
struct AStage {
  static constexpr int kChunks = BM * 8;
  static constexpr int kPer = (kChunks + THREADS - 1) / THREADS;
  uint4 r[kPer];

  __device__ __forceinline__ void load(const int8_t* __restrict__ x8, int64_t K, int m0, int M, int g) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int ch = threadIdx.x + i * THREADS;
      const int row = ch >> 3, kc = ch & 7;
      r[i] = make_uint4(0, 0, 0, 0);
      if ((kChunks % THREADS == 0 || ch < kChunks) && m0 + row < M)
        r[i] = *reinterpret_cast<const uint4*>(x8 + int64_t(m0 + row) * K + int64_t(g) * 128 + kc * 16);
    }
  }
  __device__ __forceinline__ void store(int8_t* lds) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int ch = threadIdx.x + i * THREADS;
      if (kChunks % THREADS == 0 || ch < kChunks)
        *reinterpret_cast<uint4*>(lds + lds_off(ch >> 3, ch & 7)) = r[i];
    }
  }
};

struct GemmArgs {
  const int8_t* x8;
  const unsigned short* sx;
  const uint4* qw;
  const uint32_t* meta;  // g128: dwords; per-channel: bytes read through meta8
  const uint8_t* meta8;
  const unsigned short* scale;
  void* out;
  int M, N, G, G4q;  // G4q = G4 / 4 (meta dwords per strip per channel)
  int n_strips;
  int64_t ldo;
};

template <bool I32OUT>
__device__ __forceinline__ void store_out(const GemmArgs& a, int row, int col, int acc, float sxr) {
  if (row < a.M && col < a.N) {
    if constexpr (I32OUT) {
      static_cast<int*>(a.out)[int64_t(row) * a.ldo + col] = acc;
    } else {
      const float sc = __half2float(__ushort_as_half(a.scale[col]));
      const float y = static_cast<float>(acc) * sxr * sc;
      static_cast<__half*>(a.out)[int64_t(row) * a.ldo + col] = __float2half_rn(y);
    }
  }
}

// ---------------------------------------------------------------------------
// gemm16: block = WN waves side by side along N, each wave TN strips of 16
// output channels; all waves share the BM = TM*16 rows of the block.
template <int WN, int TM, int TN, bool PERCH, bool I32OUT>
__global__ __launch_bounds__(64 * WN) void gemm16_kernel(GemmArgs a) {
  constexpr int THREADS = 64 * WN;
  constexpr int BM = TM * 16;
  __shared__ __align__(16) int8_t As[2][BM * 128];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m0 = blockIdx.y * BM;
  const int sbase = (blockIdx.x * WN + wave) * TN;
  const int64_t K = int64_t(a.G) * 128;
  const int c16 = lane & 15, j = lane >> 4;

  int strip[TN];
#pragma unroll
  for (int t = 0; t < TN; ++t) strip[t] = min(sbase + t, a.n_strips - 1);

  uint32_t S[TN], C[TN];
  if constexpr (PERCH) {
#pragma unroll
    for (int t = 0; t < TN; ++t) meta_perchannel(a.meta8[strip[t] * 16 + c16], S[t], C[t]);
  }

  v4i acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int t = 0; t < TN; ++t) acc[i][t] = v4i{0, 0, 0, 0};

  AStage<BM, THREADS> ast;
  uint4 bcur[TN], bnext[TN];
  uint32_t mcur[TN], mnext[TN];

  auto load_b = [&](int g, uint4* b, uint32_t* m) {
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      b[t] = a.qw[(int64_t(strip[t]) * a.G + g) * 64 + lane];
      if constexpr (!PERCH) m[t] = a.meta[(int64_t(strip[t]) * a.G4q + (g >> 2)) * 16 + c16];
    }
  };

  ast.load(a.x8, K, m0, a.M, 0);
  load_b(0, bcur, mcur);
  ast.store(As[0]);
  __syncthreads();

  for (int g = 0; g < a.G; ++g) {
    const bool more = g + 1 < a.G;
    if (more) {
      ast.load(a.x8, K, m0, a.M, g + 1);
      load_b(g + 1, bnext, mnext);
    }
    const int8_t* lds = As[g & 1];
    if constexpr (!PERCH) {
#pragma unroll
      for (int t = 0; t < TN; ++t) meta_g128((mcur[t] >> (8 * (g & 3))) & 0xffu, S[t], C[t]);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      v4i af[TM];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = *reinterpret_cast<const v4i*>(lds + lds_off(i * 16 + c16, 4 * h + j));
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        const uint32_t v0 = h ? bcur[t].z : bcur[t].x;
        const uint32_t v1 = h ? bcur[t].w : bcur[t].y;
        const v4i bf = dequant16(v0, v1, S[t], C[t]);
#pragma unroll
        for (int i = 0; i < TM; ++i) acc[i][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[i], bf, acc[i][t], 0, 0, 0);
      }
    }
    if (more) ast.store(As[(g + 1) & 1]);
    __syncthreads();
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      bcur[t] = bnext[t];
      mcur[t] = mnext[t];
    }
  }

  // epilogue: lane holds rows 4*(lane/16)+r of each 16x16 tile, column lane%16
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = m0 + i * 16 + 4 * j + r;
      float sxr = 0.0f;
      if constexpr (!I32OUT) sxr = row < a.M ? __half2float(__ushort_as_half(a.sx[row])) : 0.0f;
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        if (sbase + t < a.n_strips) store_out<I32OUT>(a, row, (sbase + t) * 16 + c16, acc[i][t][r], sxr);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// gemm32: block = WM x WN waves; wave tile = TM*32 rows x TN*32 columns.
template <int WM, int WN, int TM, int TN, bool PERCH, bool I32OUT>
__global__ __launch_bounds__(64 * WM * WN) void gemm32_kernel(GemmArgs a) {
  constexpr int THREADS = 64 * WM * WN;
  constexpr int BM = WM * TM * 32;
  constexpr int BN = WN * TN * 32;
  __shared__ __align__(16) int8_t As[2][BM * 128];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int m0 = blockIdx.y * BM;
  const int n0 = blockIdx.x * BN + wn * TN * 32;  // first column of this wave
  const int64_t K = int64_t(a.G) * 128;
  const int c32 = lane & 31, hh = lane >> 5;
  const int c16 = c32 & 15;

  // column tile t, lane: channel n0 + 32t + c32 -> strip, channel-in-strip c16
  int strip[TN];
#pragma unroll
  for (int t = 0; t < TN; ++t) strip[t] = min((n0 + 32 * t + c32) >> 4, a.n_strips - 1);

  uint32_t S[TN], C[TN];
  if constexpr (PERCH) {
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

  AStage<BM, THREADS> ast;
  // per column tile two 16-byte slots: slot c16+16*hh (K steps 0, 2) and
  // slot c16+16*(2+hh) (K steps 1, 3)
  uint4 bcur[TN][2], bnext[TN][2];
  uint32_t mcur[TN], mnext[TN];

  auto load_b = [&](int g, uint4 (*b)[2], uint32_t* m) {
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      const uint4* blk = a.qw + (int64_t(strip[t]) * a.G + g) * 64;
      b[t][0] = blk[c16 + 16 * hh];
      b[t][1] = blk[c16 + 16 * (2 + hh)];
      if constexpr (!PERCH) m[t] = a.meta[(int64_t(strip[t]) * a.G4q + (g >> 2)) * 16 + c16];
    }
  };

  ast.load(a.x8, K, m0, a.M, 0);
  load_b(0, bcur, mcur);
  ast.store(As[0]);
  __syncthreads();

  for (int g = 0; g < a.G; ++g) {
    const bool more = g + 1 < a.G;
    if (more) {
      ast.load(a.x8, K, m0, a.M, g + 1);
      load_b(g + 1, bnext, mnext);
    }
    const int8_t* lds = As[g & 1];
    if constexpr (!PERCH) {
#pragma unroll
      for (int t = 0; t < TN; ++t) meta_g128((mcur[t] >> (8 * (g & 3))) & 0xffu, S[t], C[t]);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      v4i af[TM];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = *reinterpret_cast<const v4i*>(lds + lds_off(wm * TM * 32 + i * 32 + c32, 2 * s + hh));
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        const uint4& q = bcur[t][s & 1];
        const uint32_t v0 = (s >> 1) ? q.z : q.x;
        const uint32_t v1 = (s >> 1) ? q.w : q.y;
        const v4i bf = dequant16(v0, v1, S[t], C[t]);
#pragma unroll
        for (int i = 0; i < TM; ++i) acc[i][t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf, acc[i][t], 0, 0, 0);
      }
    }
    if (more) ast.store(As[(g + 1) & 1]);
    __syncthreads();
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      bcur[t][0] = bnext[t][0];
      bcur[t][1] = bnext[t][1];
      mcur[t] = mnext[t];
    }
  }

  // epilogue: lane holds column lane%32 and rows 8*(r/4) + 4*(lane/32) + r%4
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = m0 + wm * TM * 32 + i * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
      float sxr = 0.0f;
      if constexpr (!I32OUT) sxr = row < a.M ? __half2float(__ushort_as_half(a.sx[row])) : 0.0f;
#pragma unroll
      for (int t = 0; t < TN; ++t) store_out<I32OUT>(a, row, n0 + 32 * t + c32, acc[i][t][r], sxr);
    }
  }
}

// ---------------------------------------------------------------------------
// Launch helpers.

template <int WN, int TM, int TN, bool PERCH, bool I32>
hipError_t launch16(const GemmArgs& a, hipStream_t st) {
  const int per_block = WN * TN;
  const dim3 grid((a.n_strips + per_block - 1) / per_block, (a.M + TM * 16 - 1) / (TM * 16));
  hipLaunchKernelGGL((gemm16_kernel<WN, TM, TN, PERCH, I32>), grid, dim3(64 * WN), 0, st, a);
  return hipGetLastError();
}

template <int WM, int WN, int TM, int TN, bool PERCH, bool I32>
hipError_t launch32(const GemmArgs& a, hipStream_t st) {
  constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
  const dim3 grid((a.n_strips * 16 + BN - 1) / BN, (a.M + BM - 1) / BM);
  hipLaunchKernelGGL((gemm32_kernel<WM, WN, TM, TN, PERCH, I32>), grid, dim3(64 * WM * WN), 0, st, a);
  return hipGetLastError();
}

template <bool PERCH, bool I32>
hipError_t dispatch(const GemmArgs& a, hipStream_t st) {
  if (a.M <= 16) return launch16<4, 1, 1, PERCH, I32>(a, st);
  if (a.M <= 32) return launch16<4, 2, 1, PERCH, I32>(a, st);
  if (a.M <= 64) return launch16<4, 4, 1, PERCH, I32>(a, st);
  return launch32<2, 2, 2, 2, PERCH, I32>(a, st);
}

int run_gemm(const char* fn, const int8_t* x8, const void* sx, const void* qweight, const void* meta,
             const void* scale, void* out, int64_t M, int64_t N, int64_t K, int64_t ldo, int32_t group_size,
             bool i32, hipStream_t st) {
  clear_error();
  if (!x8 || !qweight || !meta || !out || (!i32 && (!sx || !scale)))
    return fail(QOQ_ERR_INVALID_ARG, "%s: null pointer argument", fn);
  if (int stt = check_weight_shape(N, K, group_size)) return stt;
  if (M < 1 || M > 0x7fffffffLL - 4096) return fail(QOQ_ERR_UNSUPPORTED_SHAPE, "%s: M=%lld out of range", fn, (long long)M);
  if (ldo < N) return fail(QOQ_ERR_INVALID_ARG, "%s: leading dimension %lld < N=%lld", fn, (long long)ldo, (long long)N);
  const auto al = [](const void* p, uintptr_t n) { return reinterpret_cast<uintptr_t>(p) % n == 0; };
  if (!al(x8, 16) || !al(qweight, 16) || !al(meta, 4) || !al(out, i32 ? 4 : 2) || (!i32 && (!al(sx, 2) || !al(scale, 2))))
    return fail(QOQ_ERR_ALIGNMENT, "%s: x8/qweight need 16-byte, meta 4-byte, FP16 2-byte alignment", fn);
  GemmArgs a;
  a.x8 = x8;
  a.sx = static_cast<const unsigned short*>(sx);
  a.qw = static_cast<const uint4*>(qweight);
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
  hipError_t e;
  if (group_size) e = i32 ? dispatch<false, true>(a, st) : dispatch<false, false>(a, st);
  else e = i32 ? dispatch<true, true>(a, st) : dispatch<true, false>(a, st);
  if (e != hipSuccess) return fail(QOQ_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return QOQ_OK;
}

}  // namespace
}  // namespace qoq

using namespace qoq;

extern "C" size_t qoq_w4a8_gemm_workspace_size(int64_t, int64_t, int64_t, int32_t) { return 0; }

extern "C" int qoq_w4a8_gemm(const int8_t* x8, const void* sx_fp16, const void* qweight, const void* meta,
                             const void* scale_fp16, void* y_fp16, int64_t M, int64_t N, int64_t K, int64_t ldy,
                             int32_t group_size, void* workspace, size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  return run_gemm("qoq_w4a8_gemm", x8, sx_fp16, qweight, meta, scale_fp16, y_fp16, M, N, K, ldy, group_size, false,
                  static_cast<hipStream_t>(stream));
}

extern "C" int qoq_w4a8_gemm_i32(const int8_t* x8, const void* qweight, const void* meta, int32_t* acc, int64_t M,
                                 int64_t N, int64_t K, int64_t ldacc, int32_t group_size, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  return run_gemm("qoq_w4a8_gemm_i32", x8, nullptr, qweight, meta, nullptr, acc, M, N, K, ldacc, group_size, true,
                  static_cast<hipStream_t>(stream));
}
