// C-ABI entry points of the W4A8 GEMM: progressive g128 and per-channel UINT4
// weights ("QServe: W4A8KV4 Quantization and System Co-design for Efficient
// LLM Serving", paperlayer.ai summary, §4 progressive group quantization, §5
// W4A8 GEMM optimization, §6 per-channel counterpart).  The kernels are in
// gemm_kernels.h.

#include "gemm_kernels.h"

using namespace qoq;

extern "C" size_t qoq_w4a8_gemm_workspace_size(int64_t M, int64_t N, int64_t K, int32_t group_size) {
  return workspace_size_query(M, N, K, group_size);
}

extern "C" int qoq_w4a8_gemm(const int8_t* x8, const void* sx_fp16, const void* qweight, const void* meta,
                             const void* scale_fp16, void* y_fp16, int64_t M, int64_t N, int64_t K, int64_t ldy,
                             int32_t group_size, void* workspace, size_t workspace_bytes, void* stream) {
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (group_size == 0)
    return run_gemm<kWfPerChannel>("qoq_w4a8_gemm", x8, sx_fp16, qweight, meta, scale_fp16, y_fp16, M, N, K, ldy,
                                   group_size, workspace, workspace_bytes, false, st);
  return run_gemm<kWfG128>("qoq_w4a8_gemm", x8, sx_fp16, qweight, meta, scale_fp16, y_fp16, M, N, K, ldy, group_size,
                           workspace, workspace_bytes, false, st);
}

extern "C" int qoq_w4a8_gemm_i32(const int8_t* x8, const void* qweight, const void* meta, int32_t* acc, int64_t M,
                                 int64_t N, int64_t K, int64_t ldacc, int32_t group_size, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (group_size == 0)
    return run_gemm<kWfPerChannel>("qoq_w4a8_gemm_i32", x8, nullptr, qweight, meta, nullptr, acc, M, N, K, ldacc,
                                   group_size, workspace, workspace_bytes, true, st);
  return run_gemm<kWfG128>("qoq_w4a8_gemm_i32", x8, nullptr, qweight, meta, nullptr, acc, M, N, K, ldacc, group_size,
                           workspace, workspace_bytes, true, st);
}
