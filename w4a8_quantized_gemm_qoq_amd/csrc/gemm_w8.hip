// C-ABI entry points of the W8A8 comparator GEMM: per-channel INT8 weights
// multiplied as they are, in the same kernels, launch plans and epilogue as
// the W4A8 GEMM.  It measures on this chip the comparison the pages draw
// between the W4A8 GEMM and an INT8 GEMM ("QServe: W4A8KV4 Quantization and
// System Co-design for Efficient LLM Serving", study.space summary: the W4A8
// GEMM against the W8A8 library GEMM; paperlayer.ai summary §3, the
// W4A16 / W8A8 roofline).  The kernels are in gemm_kernels.h.

#include "gemm_kernels.h"

using namespace qoq;

extern "C" size_t qoq_w8a8_gemm_workspace_size(int64_t M, int64_t N, int64_t K) {
  return workspace_size_query(M, N, K, kGroup);
}

extern "C" int qoq_w8a8_gemm(const int8_t* x8, const void* sx_fp16, const void* qweight8, const void* scale_fp16,
                             void* y_fp16, int64_t M, int64_t N, int64_t K, int64_t ldy, void* workspace,
                             size_t workspace_bytes, void* stream) {
  return run_gemm<kWfW8>("qoq_w8a8_gemm", x8, sx_fp16, qweight8, nullptr, scale_fp16, y_fp16, M, N, K, ldy, kGroup,
                         workspace, workspace_bytes, false, static_cast<hipStream_t>(stream));
}

extern "C" int qoq_w8a8_gemm_i32(const int8_t* x8, const void* qweight8, int32_t* acc, int64_t M, int64_t N,
                                 int64_t K, int64_t ldacc, void* workspace, size_t workspace_bytes, void* stream) {
  return run_gemm<kWfW8>("qoq_w8a8_gemm_i32", x8, nullptr, qweight8, nullptr, nullptr, acc, M, N, K, ldacc, kGroup,
                         workspace, workspace_bytes, true, static_cast<hipStream_t>(stream));
}
