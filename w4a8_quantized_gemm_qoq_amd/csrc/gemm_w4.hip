// C-ABI entry points of the W4A8 GEMM: progressive g128 and per-channel UINT4
// weights ("QServe: W4A8KV4 Quantization and System Co-design for Efficient
// LLM Serving", paperlayer.ai summary, §4 progressive group quantization, §5
// W4A8 GEMM optimization, §6 per-channel counterpart).  The kernels are in
// gemm_kernels.h.

#include <mutex>

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

extern "C" int qoq_w4a8_gemm_plan(int64_t M, int64_t N, int64_t K, int32_t group_size, int32_t* kernel,
                                  int32_t* tile, int32_t* ksplit) {
  clear_error();
  if (!kernel || !tile || !ksplit) return fail(QOQ_ERR_INVALID_ARG, "qoq_w4a8_gemm_plan: null pointer argument");
  if (int st = check_weight_shape(N, K, group_size)) return st;
  if (M < 1 || M > 0x7fffffffLL - 4096)
    return fail(QOQ_ERR_UNSUPPORTED_SHAPE, "qoq_w4a8_gemm_plan: M=%lld out of range", (long long)M);
  const GemmPlan p = plan_gemm(M, N, K, group_size != 0);
  *kernel = p.kernel;
  *tile = p.tile;
  *ksplit = p.ksplit;
  return QOQ_OK;
}

// ---------------------------------------------------------------------------
// Allocation-free variant of qoq_w4a8_gemm.  The split-K INT32 partials live
// in this file-scope device array instead of a caller workspace.  Each GPU
// the library runs on holds its own copy until the process ends; every call
// on that GPU shares it.  The partials of each split are written in full
// before the reduction reads them, so nothing in it has to start at zero.
static __device__ __align__(256) int scratch[QOQ_NOALLOC_SCRATCH_BYTES / sizeof(int)];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the calling thread's current device, looked
// up once per device (in host code the array's name is only a stand-in for
// the symbol, not a device address).
int scratch_address(const char* fn, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(QOQ_ERR_HIP, "%s: hipGetDevice failed: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(QOQ_ERR_INTERNAL, "%s: device %d beyond %d", fn, dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(QOQ_ERR_HIP, "%s: hipGetSymbolAddress(scratch) failed on device %d: %s", fn, dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return QOQ_OK;
}

}  // namespace

extern "C" int qoq_w4a8_gemm_noalloc(const int8_t* x8, const void* sx_fp16, const void* qweight, const void* meta,
                                     const void* scale_fp16, void* y_fp16, int64_t M, int64_t N, int64_t K,
                                     int64_t ldy, int32_t group_size, void* stream) {
  clear_error();
  const size_t need = workspace_size_query(M, N, K, group_size);
  if (need > size_t(QOQ_NOALLOC_SCRATCH_BYTES))
    return fail(QOQ_ERR_UNSUPPORTED_SHAPE,
                "qoq_w4a8_gemm_noalloc: M=%lld N=%lld K=%lld needs %zu bytes of split-K scratch, above the "
                "library's %zu (use qoq_w4a8_gemm with a caller workspace)",
                (long long)M, (long long)N, (long long)K, need, size_t(QOQ_NOALLOC_SCRATCH_BYTES));
  void* ws = nullptr;
  if (need) {
    if (const int s = scratch_address("qoq_w4a8_gemm_noalloc", &ws)) return s;
  }
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (group_size == 0)
    return run_gemm<kWfPerChannel>("qoq_w4a8_gemm_noalloc", x8, sx_fp16, qweight, meta, scale_fp16, y_fp16, M, N, K,
                                   ldy, group_size, ws, need ? size_t(QOQ_NOALLOC_SCRATCH_BYTES) : 0, false, st);
  return run_gemm<kWfG128>("qoq_w4a8_gemm_noalloc", x8, sx_fp16, qweight, meta, scale_fp16, y_fp16, M, N, K, ldy,
                           group_size, ws, need ? size_t(QOQ_NOALLOC_SCRATCH_BYTES) : 0, false, st);
}
