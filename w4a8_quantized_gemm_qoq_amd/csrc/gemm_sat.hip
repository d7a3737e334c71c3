// C-ABI entry points of the saturating-dequantization ablation: the g128
// W4A8 GEMM with every dequantized weight clamped to INT8 in a 16-bit lane
// instead of the packed-byte form that the protective level-0 range makes
// exact ("QServe: W4A8KV4 Quantization and System Co-design for Efficient LLM
// Serving", paperlayer.ai summary, §4 progressive group quantization: the
// range [-119, 119] keeps the intermediates inside INT8, and saturating
// arithmetic would cost throughput).  Same packed weights, kernels and plans
// as qoq_w4a8_gemm with group_size 128; the kernels are in gemm_kernels.h.

#include "gemm_kernels.h"

using namespace qoq;

extern "C" int qoq_w4a8_gemm_saturating(const int8_t* x8, const void* sx_fp16, const void* qweight, const void* meta,
                                        const void* scale_fp16, void* y_fp16, int64_t M, int64_t N, int64_t K,
                                        int64_t ldy, void* workspace, size_t workspace_bytes, void* stream) {
  return run_gemm<kWfG128Sat>("qoq_w4a8_gemm_saturating", x8, sx_fp16, qweight, meta, scale_fp16, y_fp16, M, N, K,
                              ldy, kGroup, workspace, workspace_bytes, false, static_cast<hipStream_t>(stream));
}

extern "C" int qoq_w4a8_gemm_saturating_i32(const int8_t* x8, const void* qweight, const void* meta, int32_t* acc,
                                            int64_t M, int64_t N, int64_t K, int64_t ldacc, void* workspace,
                                            size_t workspace_bytes, void* stream) {
  return run_gemm<kWfG128Sat>("qoq_w4a8_gemm_saturating_i32", x8, nullptr, qweight, meta, nullptr, acc, M, N, K,
                              ldacc, kGroup, workspace, workspace_bytes, true, static_cast<hipStream_t>(stream));
}
