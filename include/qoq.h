/*
 * qoq.h -- C ABI of the MI355X (gfx950) QoQ W4A8 GEMM library (libqoq.so).
 *
 * The library implements the W4A8 GEMM of QoQ progressive group quantization:
 * 4-bit weights, per-token 8-bit activations, INT8 matrix-core arithmetic with
 * INT32 accumulation and an FP16 output.  Sources, cited by tag below:
 *
 *   [PL]  "QServe: W4A8KV4 Quantization and System Co-design for Efficient LLM
 *         Serving", section summary page at paperlayer.ai abs/2405.04532v3;
 *         cited as [PL §n, bullet topic].
 *   [SS]  study.space summary page of the same paper.
 *
 * Notation: X[M,K] FP16 activations (tokens x input channels), W[N,K] FP16
 * weights (output x input channels), Y[M,N] = X W^T.  All matrices are
 * row-major.  FP16 values travel as uint16_t bit patterns (IEEE binary16).
 *
 * Conventions for every entry point:
 *   - The return value is a qoq_status.  On failure qoq_last_error() gives a
 *     thread-local description; nothing has been written to outputs unless
 *     stated otherwise.
 *   - No function allocates device memory.  The caller owns every buffer.
 *     Apart from that thread-local error text the library keeps no state
 *     between calls, except the per-GPU split-K scratch that
 *     qoq_w4a8_gemm_noalloc uses (declared below).
 *   - Host functions (pack / unpack / layout) run synchronously on the calling
 *     thread and touch host memory only.
 *   - Device functions take device pointers and a `stream` (a hipStream_t, or
 *     NULL for the null stream), enqueue their kernels on it and return without
 *     synchronizing.  Launch failures are reported as QOQ_ERR_HIP; faults inside
 *     a kernel surface at the caller's next synchronization.
 *   - K must be a positive multiple of 128 (one 128-wide group is the unit of
 *     the K loop, also for the per-channel variant), M >= 1, N >= 1, and
 *     127*127*K < 2^31 so the INT32 accumulator cannot overflow.
 */
#ifndef QOQ_H_
#define QOQ_H_

#include <stddef.h>
#include <stdint.h>

#if defined(QOQ_BUILD)
#define QOQ_API __attribute__((visibility("default")))
#else
#define QOQ_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum qoq_status {
  QOQ_OK = 0,
  QOQ_ERR_INVALID_ARG = 1,       /* null pointer, bad value, codes that break the INT8 bound */
  QOQ_ERR_UNSUPPORTED_SHAPE = 2, /* K not a multiple of 128, sizes out of range */
  QOQ_ERR_ALIGNMENT = 3,         /* a device pointer or leading dimension is misaligned */
  QOQ_ERR_HIP = 4,               /* the HIP runtime reported an error */
  QOQ_ERR_INTERNAL = 5
} qoq_status;

/* Version of the packed weight layout described below. */
#define QOQ_LAYOUT_ID 1
/* Group size of the g128 progressive variant ([PL §6, experimental setup]). */
#define QOQ_GROUP 128

/* Static description of a status code; never NULL. */
QOQ_API const char* qoq_status_string(int status);
/* Detail text of the last failure on this thread ("" if none); valid until the
 * thread's next library call. */
QOQ_API const char* qoq_last_error(void);

/*
 * Packed weight layout (QOQ_LAYOUT_ID 1).  The GEMM reads weights in the order
 * it computes with them ([PL §5, W4A8 GEMM optimization]: the weights are
 * rearranged offline so that the kernel fetches each thread's operands with
 * wide loads and no shuffling at run time).  Here the order follows the INT8
 * matrix-core operand fragments of gfx950.
 *
 *   N_pad   = N rounded up to a multiple of 16; padded channels are all-zero.
 *   G       = K / 128 groups along K.  G4 = G rounded up to a multiple of 4.
 *
 *   qweight (N_pad*K/2 bytes): 16-channel strips, each strip a run of G
 *     1024-byte group blocks, each block 64 slots of 16 bytes:
 *       offset = ((strip*G + g)*64 + slot)*16,  slot = c + 16*j  (c = channel
 *       in strip 0..15, j = 0..3).  Slot bytes form 4 little-endian dwords
 *       v[p], p = 0..3.  Byte b of v[p] holds two UINT4 codes: the low nibble
 *       is input channel k = 128g + 64*(p/2) + 16j + 8*(p%2) + b and the high
 *       nibble is that k + 4.
 *   meta, g128 ((N_pad/16)*G4*16 bytes): one byte per (channel, group),
 *       (s1 - 1) | (z << 4), at offset ((strip*(G4/4) + g/4)*16 + c)*4 + g%4.
 *     meta, per-channel (N_pad bytes): byte n = z[n] (0..15).
 *   scale (N_pad FP16): the per-channel FP16 scale -- s0 (g128) or s_w
 *     (per-channel); 0 for padded channels.
 *
 * The metadata of a format lives in one buffer: for g128 the 8-bit group scale
 * and the UINT4 zero share a byte (s1 <= 16 needs 4 bits), for per-channel
 * the byte is the zero; the FP16 per-channel scale is the separate `scale`.
 *
 * Code meaning ([PL §4, progressive group quantization]; [PL §5, W4A8 GEMM
 * optimization: subtraction after multiplication]):
 *   g128:         w8 = (q4 - z) * s1, s1 in [1,16], q4 and z in [0,15];
 *                 y  = fp16(sum_k x8*w8 * s_x * s0).
 *   per-channel:  w8 = q4 - z;  y = fp16(sum_k x8*w8 * s_x * s_w).
 */
typedef struct qoq_weight_layout {
  int32_t layout_id;     /* QOQ_LAYOUT_ID */
  int32_t group_size;    /* 128 (g128 progressive) or 0 (per-channel W4) */
  int64_t N, K;          /* logical shape of W */
  int64_t N_pad;         /* N rounded up to 16 */
  int64_t n_groups;      /* G = K / 128 */
  size_t qweight_bytes;  /* N_pad * K / 2 */
  size_t meta_bytes;     /* see above */
  size_t scale_bytes;    /* 2 * N_pad */
} qoq_weight_layout;

/* Sizes of the packed buffers for W[N,K].  group_size is 128 or 0. */
QOQ_API int qoq_weight_layout_query(int64_t N, int64_t K, int32_t group_size, qoq_weight_layout* out);

/*
 * Offline weight encode and pack (host).  [PL §4, progressive group
 * quantization]; [SS] (8-bit per-channel FP16 scales first, then 4 bits).
 *   group_size 128: level 0, per output channel n:
 *       s0 = fp16(max_k |W| / 119)  (FP32 divide, round half to even),
 *       q8 = clamp(round(W / s0), -119, 119)   -- the protective range;
 *     level 1, per (n, group of 128 along K) with lo/hi = min/max of q8:
 *       s1 = max(1, round((hi - lo) / 15)), z = clamp(round(-lo / s1), 0, 15),
 *       q4 = clamp(round(q8 / s1) + z, 0, 15).
 *   group_size 0 ([PL §6, experimental setup: per-channel counterpart]):
 *       s_w = fp16((max W - min W) / 15), z = clamp(round(-min W / s_w), 0, 15),
 *       q4 = clamp(round(W / s_w) + z, 0, 15).
 *   Rounding is half to even throughout; a zero scale gives all-zero codes.
 * w_fp16: host [N][K] row-major.  qweight/meta/scale_fp16: caller-owned host
 * buffers of the sizes qoq_weight_layout_query reports (fully written,
 * including padding).  Rejects non-finite weights (QOQ_ERR_INVALID_ARG).
 */
QOQ_API int qoq_pack_weights(const uint16_t* w_fp16, int64_t N, int64_t K, int32_t group_size,
                     void* qweight, void* meta, uint16_t* scale_fp16);

/*
 * Pack already-quantized codes (host): q4 [N][K] (0..15); for g128 s1 and z
 * are [N][K/128] (s1 1..16, z 0..15); for per-channel s1 is ignored (may be
 * NULL) and z is [N].  scale_fp16 [N] is copied.  Rejects codes whose
 * dequantized value (q4 - z)*s1 leaves [-128, 127] or whose z*s1 exceeds 128
 * (the packed-byte dequantization has no saturation), QOQ_ERR_INVALID_ARG.
 */
QOQ_API int qoq_pack_codes(const uint8_t* q4, const uint8_t* s1, const uint8_t* z,
                   const uint16_t* scale_fp16, int64_t N, int64_t K, int32_t group_size,
                   void* qweight, void* meta, uint16_t* scale_out);

/* Inverse of the packing (host, for tests and debugging): writes q4 [N][K],
 * s1 [N][K/128] (g128 only; may be NULL for per-channel), z ([N][K/128] or [N])
 * and scale_fp16 [N]. */
QOQ_API int qoq_unpack_weights(const void* qweight, const void* meta, const uint16_t* scale_in,
                       int64_t N, int64_t K, int32_t group_size,
                       uint8_t* q4, uint8_t* s1, uint8_t* z, uint16_t* scale_fp16);

/*
 * Per-token symmetric INT8 activation quantization (device).
 * [PL §6, experimental setup: per-token INT8 activations]; [PL §5, runtime
 * and precision mapping: activations enter the W4A8 GEMM as INT8].  Per row m:
 *   s_x[m] = fp16(max_k |X[m,k]| / 127)  (FP32 IEEE divide, round half even),
 *   x8[m,k] = clamp(rint(X[m,k] / s_x[m]), -127, 127)  (FP32 IEEE divide);
 *   a zero scale gives a zero row.  Non-finite X is undefined behaviour.
 * x_fp16: device [M][ldx] FP16, ldx >= K.  x8: device [M][K] int8 (row stride
 * K).  sx_fp16: device [M] FP16.  Here K needs only be >= 1; x_fp16 and ldx
 * need 16-byte / 8-element alignment for the vector path (otherwise a scalar
 * path runs).
 */
QOQ_API int qoq_quant_act_per_token(const void* x_fp16, int64_t M, int64_t K, int64_t ldx,
                            int8_t* x8, void* sx_fp16, void* stream);

/*
 * Fused producer (device): RMS normalization of each token row, then the
 * per-token INT8 quantization above, in one kernel that reads x once and
 * writes only x8 and s_x.  [PL §5, runtime and precision mapping: the
 * quantizer runs inside the normalization kernel that produces the
 * activations].  Per row m:
 *   S    = sum_k x[m,k]^2, exact (FP16 squares are integers times 2^-48);
 *   ms   = fp32(fp64(S) / K), r = 1 / sqrt(ms + eps) (FP32 IEEE add, sqrt and
 *          divide);
 *   h[k] = fp16((x[m,k] * r) * gamma[k]) (two FP32 products, round half even);
 *   then s_x[m] and x8[m,:] from h exactly as qoq_quant_act_per_token.
 * Each step rounds once, so the result does not depend on the launch shape.
 * x_fp16: device [M][ldx] FP16, ldx >= K.  gamma_fp16: device [K] FP16.
 * eps > 0 and finite (QOQ_ERR_INVALID_ARG otherwise).  x8: device [M][K]
 * int8.  sx_fp16: device [M].  Vector path when K and ldx are multiples of 8
 * and x, gamma are 16-byte aligned (else a scalar path).  Non-finite x or an
 * FP16 overflow of h is undefined behaviour.
 */
QOQ_API int qoq_rmsnorm_quant_per_token(const void* x_fp16, const void* gamma_fp16, float eps, int64_t M, int64_t K,
                                int64_t ldx, int8_t* x8, void* sx_fp16, void* stream);

/*
 * Fused producer (device) of a gated FFN's down-projection input: h = SiLU(gate)
 * * up per element, then the per-token INT8 quantization of h, in one kernel
 * that reads gate and up once and writes x8 and s_x (and h if asked).  [PL §5,
 * runtime and precision mapping: the quantizer also runs inside the
 * activation-function kernel that produces a layer's input].  Per element,
 * each step rounded once (round half to even):
 *   s = fp16(g / (1 + e^-g))  (the correctly rounded FP16 SiLU),
 *   h = fp16(s * u)           (the product of two halves is exact in FP32),
 * then s_x[m] and x8[m,:] from the row of h exactly as qoq_quant_act_per_token.
 * gate_fp16, up_fp16: device [M][ldg] and [M][ldu] FP16 (ldg, ldu >= K; the
 * two halves of a fused gate-up output are gate = base, up = base + K with
 * ldg = ldu = 2K).  x8: device [M][K] int8.  sx_fp16: device [M].  h_fp16:
 * device [M][ldh] FP16 (ldh >= K) that receives h, or NULL.  Vector path when
 * K and the leading dimensions are multiples of 8 and the FP16 pointers are
 * 16-byte aligned (else a scalar path).  Non-finite inputs or an FP16
 * overflow of h are undefined behaviour.
 */
QOQ_API int qoq_swiglu_quant_per_token(const void* gate_fp16, const void* up_fp16, int64_t M, int64_t K, int64_t ldg,
                               int64_t ldu, int8_t* x8, void* sx_fp16, void* h_fp16, int64_t ldh, void* stream);

/* Device workspace (bytes) qoq_w4a8_gemm / qoq_w4a8_gemm_i32 need for this
 * shape; 0 means the workspace arguments may be NULL / 0. */
QOQ_API size_t qoq_w4a8_gemm_workspace_size(int64_t M, int64_t N, int64_t K, int32_t group_size);

/*
 * W4A8 GEMM with fused epilogue (device).  [PL §5, runtime and precision
 * mapping: INT8 matrix-core GEMM with FP16 output]; [PL §3/§4: weights are
 * dequantized UINT4 -> INT8 inside the main loop, one INT32 accumulator spans
 * all of K]; [PL §5, W4A8 GEMM optimization: per-channel scale fused into the
 * epilogue].
 *   y[m,n] = fp16(float(acc[m,n]) * s_x[m] * scale[n]),
 *   acc[m,n] = sum_k x8[m,k] * w8[n,k]  (exact INT32).
 * x8: device [M][K] int8, 16-byte aligned.  sx_fp16: device [M].  qweight,
 * meta, scale_fp16: device copies of the packed buffers (qweight 16-byte
 * aligned).  y_fp16: device [M][ldy] FP16, ldy >= N.  The FP16 result is
 * within one FP16 ulp of the correctly rounded exact product.
 */
QOQ_API int qoq_w4a8_gemm(const int8_t* x8, const void* sx_fp16, const void* qweight, const void* meta,
                  const void* scale_fp16, void* y_fp16, int64_t M, int64_t N, int64_t K,
                  int64_t ldy, int32_t group_size, void* workspace, size_t workspace_bytes,
                  void* stream);

/*
 * Debug entry: the same main loop with an INT32 epilogue (device).  Writes the
 * exact accumulators acc[m][n] (row stride ldacc >= N) instead of y; no scales
 * are read.  Exists so that the integer contraction can be compared bit for bit.
 */
QOQ_API int qoq_w4a8_gemm_i32(const int8_t* x8, const void* qweight, const void* meta, int32_t* acc,
                      int64_t M, int64_t N, int64_t K, int64_t ldacc, int32_t group_size,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Launch plan qoq_w4a8_gemm takes for a shape (host, no GPU work), for tests
 * and tuning.  kernel: 0 strip kernel (up to 16 rows, activations in LDS),
 * 1 / 2 / 3 skinny kernel with 16- / 32- / 64-row tiles, 4 large-M kernel,
 * 5 ring kernel (up to 64 rows, a strip's K range streamed by one wave, or,
 * up to 32 rows and from 64 groups on, by two waves taking one half each;
 * activations through an LDS ring of group batches; wide N, K a multiple of
 * 1024).  tile: strips
 * per workgroup (kernels 0-3 and 5) or the large-M block tile (0: 128 x 512,
 * 1: 64 x 256, 2: 128 x 128 with K split inside the block).  ksplit: K parts
 * per workgroup (kernels 0-3: waves that split the K groups and sum their
 * partials in LDS; kernel 5: 1 or 2 waves a strip) or K splits across
 * workgroups with a reduction (kernel 4).  Same argument checks as
 * qoq_w4a8_gemm.
 */
QOQ_API int qoq_w4a8_gemm_plan(int64_t M, int64_t N, int64_t K, int32_t group_size, int32_t* kernel,
                       int32_t* tile, int32_t* ksplit);

/* Split-K scratch held by the library for qoq_w4a8_gemm_noalloc, per GPU. */
#define QOQ_NOALLOC_SCRATCH_BYTES (32u << 20)

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * GEMM as qoq_w4a8_gemm, same arguments without the workspace, calling no
 * allocating routine.  Where the launch plan splits K, the INT32 partials go
 * to a device array of QOQ_NOALLOC_SCRATCH_BYTES that the library holds on
 * each GPU it runs on until the process ends.  Shapes whose partials would
 * exceed it (qoq_w4a8_gemm_workspace_size() > QOQ_NOALLOC_SCRATCH_BYTES) are
 * rejected with QOQ_ERR_UNSUPPORTED_SHAPE before any launch.  Every call on
 * one GPU shares that array: calls that overlap on one GPU (concurrent
 * streams, or threads) race and give wrong results; calls ordered on one
 * stream are safe.  The GPU is the calling thread's current device, which
 * must be the stream's.  Results are bit-identical to qoq_w4a8_gemm's.
 */
QOQ_API int qoq_w4a8_gemm_noalloc(const int8_t* x8, const void* sx_fp16, const void* qweight, const void* meta,
                          const void* scale_fp16, void* y_fp16, int64_t M, int64_t N, int64_t K,
                          int64_t ldy, int32_t group_size, void* stream);

/* ---------------------------------------------------------------------------
 * Offline accuracy transforms (host).  [PL §4, activation optimizations:
 * a unitary rotation of a block's inputs, folded into the weights before it,
 * and per-channel smoothing for the layers where rotation is not used];
 * [PL §4, SmoothAttention: the keys' outlier channels are divided down and
 * the queries take the factor, alpha = 0.5].  Each is
 * an identity of the product, X W^T = (X H)(W H)^T = (X / l)(W * l)^T, so
 * the W4A8 path is run on the transformed tensors.  FP16 in and out, the
 * arithmetic in FP64 with one rounding to FP16 (half to even).
 */

/* out = in @ H for rows x K (row stride ld, in place allowed), H the
 * normalized Walsh-Hadamard matrix, block-diagonal with blocks of the largest
 * power of two dividing K (entries +-1/sqrt(block)). */
QOQ_API int qoq_hadamard_rotate(const uint16_t* in_fp16, int64_t rows, int64_t K, int64_t ld, uint16_t* out_fp16);

/* lambda[k] = act_absmax[k]^alpha / w_absmax[k]^(1 - alpha) (FP64, returned
 * as FP32), 1 where either maximum is 0; 0 <= alpha <= 1. */
QOQ_API int qoq_smoothing_factors(const float* act_absmax, const float* w_absmax, int64_t K, float alpha,
                          float* lambda);

/* out[r][k] = fp16(in[r][k] * factor[k]) (divide != 0: / factor[k]); factors
 * positive and finite.  Weights take lambda, activations 1/lambda. */
QOQ_API int qoq_scale_columns(const uint16_t* in_fp16, int64_t rows, int64_t K, int64_t ld, const float* factor,
                      int32_t divide, uint16_t* out_fp16);

/* ---------------------------------------------------------------------------
 * KV4: the INT4 KV cache and the decode attention that reads it.
 * [PL §6, experimental setup: per-head asymmetric INT4 KV caches]; [PL §5,
 * KV4 attention: per-head scaling factors and zero points computed at run
 * time; the attention runs in floating point on the vector units and is
 * memory-bound]; [PL §4, SmoothAttention: queries stay unquantized].
 * head_dim must be 128.
 *
 * Cache layout: one row per (token, kv head) of 128 values:
 *   codes [rows][64 bytes]: byte j = code of dim 2j | (code of dim 2j+1) << 4;
 *   scale FP16 [rows]; zero [rows] (one byte, 0..15).
 * The attention takes rows ordered [B][Hkv][T_max] (a head's tokens
 * consecutive).
 */

/*
 * Per-head asymmetric INT4 quantization (device) of n_rows rows of 128 FP16
 * values (row r at x_fp16 + r*ldx, ldx a multiple of 8 and >= 128; x 16-byte
 * aligned, codes 4-byte aligned), the same map as the
 * per-channel weights: s = fp16((max - min) / 15) (FP32 subtract and divide,
 * round half even), z = clamp(rint(-min / s), 0, 15),
 * q = clamp(rint(x / s) + z, 0, 15); s == 0 gives z = 0 and zero codes.
 * codes: device [n_rows][64]; scale_fp16, zero: device [n_rows].  n_rows >= 1.
 */
QOQ_API int qoq_kv4_quant(const void* x_fp16, int64_t n_rows, int32_t head_dim, int64_t ldx, uint8_t* codes,
                  void* scale_fp16, uint8_t* zero, void* stream);

/*
 * Decode attention over a KV4 cache (device).  For sequence b < B and query
 * head h < H (kv head g = h / (H / Hkv)), with L = lengths[b] (clamped to
 * [0, T_max]) cached tokens:
 *   k_t = (kc_t - kz_t) * ks_t, v_t = (vc_t - vz_t) * vs_t,
 *   a = softmax_t(softmax_scale * <q[b,h], k_t>),  o[b,h] = fp16(sum_t a_t v_t),
 * with scores ks_t * <q', kc_t - kz_t>, q' = softmax_scale * q: q' is split
 * into three INT8 pieces (q' ~ S0 b0 + S1 b1 + S2 b2, S0 = max|q'| / 127,
 * S_{p+1} = S_p / 254, within about 2^-23 max|q'|), whose dot products with
 * the codes are exact INT32 on the matrix cores, combined in FP32; the
 * softmax and the weighted sum of values are FP32.  L = 0 gives o = 0.
 * q_fp16: device [B][H][128]; the k and v arrays: cache rows
 * [B][Hkv][T_max]; lengths: device int32 [B]; o_fp16: device [B][H][128].
 * B, H, Hkv >= 1 with H a multiple of Hkv; 1 <= T_max <= 32768 (other
 * sizes: QOQ_ERR_UNSUPPORTED_SHAPE); q and the code arrays 16-byte aligned.  Accuracy:
 * each output within one FP16 ulp plus 2^-12 max_t |v_t| of the exact
 * attention over the dequantized cache.
 */
QOQ_API int qoq_kv4_decode_attention(const void* q_fp16, const uint8_t* k_codes, const void* k_scale_fp16,
                             const uint8_t* k_zero, const uint8_t* v_codes, const void* v_scale_fp16,
                             const uint8_t* v_zero, const int32_t* lengths, int32_t B, int32_t H, int32_t Hkv,
                             int32_t T_max, int32_t head_dim, float softmax_scale, void* o_fp16, void* stream);

/*
 * Workspace (bytes) qoq_kv4_decode_attention_split needs for this shape; 0
 * when the shape is not split (then that entry runs the single-pass kernel).
 * 0 also for arguments qoq_kv4_decode_attention would reject.
 */
QOQ_API size_t qoq_kv4_decode_attention_workspace_size(int32_t B, int32_t H, int32_t Hkv, int32_t T_max);

/*
 * Launch plan the decode attention takes for a shape (host, no GPU work): the
 * query heads each workgroup serves (4, 2 or 1 of a kv group) and the number
 * of token chunks (1: not split).  split != 0 asks for the plan of
 * qoq_kv4_decode_attention_split, 0 for qoq_kv4_decode_attention.  For tests
 * and tuning: it shows which kernel variant a shape reaches.  Returns
 * QOQ_ERR_UNSUPPORTED_SHAPE for shapes the attention rejects.
 */
QOQ_API int qoq_kv4_decode_attention_plan(int32_t B, int32_t H, int32_t Hkv, int32_t T_max, int32_t split,
                                  int32_t* heads_per_block, int32_t* token_chunks);

/*
 * The same decode attention with the cached tokens cut into chunks spread
 * over more workgroups, for batches too small to fill the GPU with one
 * workgroup per (sequence, kv-head group).  Each chunk keeps its own softmax
 * statistics (the chunk's largest score m_c, l_c = sum exp(s_t - m_c), and
 * the unnormalized sum of exp(s_t - m_c) v_t) in FP32 in the workspace; a
 * second kernel rescales them to the overall largest score M and writes
 * o = sum_c e^(m_c - M) o_c / sum_c e^(m_c - M) l_c.  The result equals
 * qoq_kv4_decode_attention's up to FP32 rounding order.  Arguments as
 * there, plus workspace: device, 16-byte aligned, at least
 * qoq_kv4_decode_attention_workspace_size(B, H, Hkv, T_max) bytes, owned by
 * the caller and overwritten (QOQ_ERR_INVALID_ARG if too small).  Calls
 * that share a workspace must be ordered on one stream.
 */
QOQ_API int qoq_kv4_decode_attention_split(const void* q_fp16, const uint8_t* k_codes, const void* k_scale_fp16,
                                   const uint8_t* k_zero, const uint8_t* v_codes, const void* v_scale_fp16,
                                   const uint8_t* v_zero, const int32_t* lengths, int32_t B, int32_t H,
                                   int32_t Hkv, int32_t T_max, int32_t head_dim, float softmax_scale,
                                   void* o_fp16, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Comparators of the W4A8 GEMM.  They run the same kernels, launch plans and
 * epilogue, so that the cost of the weight format is measured on its own.
 */

/*
 * W8A8 weights (host): per output channel n, symmetric INT8,
 *   s_w = fp16(max_k |W[n,k]| / 127)  (FP32 IEEE divide, round half to even),
 *   w8  = clamp(round(W / s_w), -127, 127); a zero scale gives a zero row.
 * This is the INT8-weight GEMM the pages compare the W4A8 GEMM with ([SS]:
 * the W4A8 GEMM against the W8A8 library GEMM; [PL §3, roofline analysis:
 * W4A16 against W8A8]; [PL §6, accuracy evaluation: W8A8 SmoothQuant]).
 * Layout: qweight8 (N_pad*K bytes) is 16-channel strips, each a run of G
 * 2048-byte group blocks of 128 slots of 16 bytes:
 *   offset = ((strip*G + g)*128 + slot)*16 + b,  slot = c + 16*j + 64*h
 *   (c = channel in strip, j = 0..3, h = 0..1, b = 0..15) holds
 *   w8[16*strip + c][128*g + 64*h + 16*j + b].
 * scale_fp16: N_pad entries, 0 for padded channels.  Same shape rules and
 * error behaviour as qoq_pack_weights.
 */
QOQ_API int qoq_pack_weights_w8(const uint16_t* w_fp16, int64_t N, int64_t K, void* qweight8, uint16_t* scale_fp16);

/* Workspace (bytes) qoq_w8a8_gemm / qoq_w8a8_gemm_i32 need for this shape. */
QOQ_API size_t qoq_w8a8_gemm_workspace_size(int64_t M, int64_t N, int64_t K);

/*
 * W8A8 GEMM (device): y[m,n] = fp16(float(acc[m,n]) * s_x[m] * s_w[n]) with
 * acc[m,n] = sum_k x8[m,k] * w8[n,k] (exact INT32).  Arguments as for
 * qoq_w4a8_gemm, with the INT8 packed weights in place of qweight/meta.
 */
QOQ_API int qoq_w8a8_gemm(const int8_t* x8, const void* sx_fp16, const void* qweight8, const void* scale_fp16,
                  void* y_fp16, int64_t M, int64_t N, int64_t K, int64_t ldy, void* workspace,
                  size_t workspace_bytes, void* stream);

/* W8A8 debug entry: writes the exact INT32 accumulators (row stride ldacc). */
QOQ_API int qoq_w8a8_gemm_i32(const int8_t* x8, const void* qweight8, int32_t* acc, int64_t M, int64_t N,
                      int64_t K, int64_t ldacc, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Saturating-dequantization ablation of the g128 W4A8 GEMM (device).  [PL §4,
 * progressive group quantization]: the protective range [-119, 119] keeps
 * (q4 - z)*s1 inside INT8 so the GEMM can dequantize with plain packed-byte
 * arithmetic; without it every value must be clamped, which the pages report
 * as costly.  This entry clamps: w8 = clamp((q4 - z)*s1, -128, 127), computed
 * in 16-bit lanes, for any s1 in [1,16] and z in [0,15].  For weights packed
 * by qoq_pack_weights or qoq_pack_codes the result equals qoq_w4a8_gemm's
 * (group_size 128), bit for bit.  Same arguments as qoq_w4a8_gemm with
 * group_size 128 (workspace size from qoq_w4a8_gemm_workspace_size).
 */
QOQ_API int qoq_w4a8_gemm_saturating(const int8_t* x8, const void* sx_fp16, const void* qweight, const void* meta,
                             const void* scale_fp16, void* y_fp16, int64_t M, int64_t N, int64_t K,
                             int64_t ldy, void* workspace, size_t workspace_bytes, void* stream);

/* Saturating ablation, INT32 debug entry. */
QOQ_API int qoq_w4a8_gemm_saturating_i32(const int8_t* x8, const void* qweight, const void* meta, int32_t* acc,
                                 int64_t M, int64_t N, int64_t K, int64_t ldacc, void* workspace,
                                 size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QOQ_H_ */
