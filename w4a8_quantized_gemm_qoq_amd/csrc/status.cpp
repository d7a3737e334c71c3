// Status strings and the thread-local error text of libqoq.so.

#include <cstdarg>
#include <cstdio>

#include "qoq_internal.h"

namespace qoq {
namespace {
thread_local char g_err[512] = {0};
}

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return status;
}

void clear_error() { g_err[0] = 0; }

}  // namespace qoq

extern "C" const char* qoq_status_string(int status) {
  switch (status) {
    case QOQ_OK: return "ok";
    case QOQ_ERR_INVALID_ARG: return "invalid argument";
    case QOQ_ERR_UNSUPPORTED_SHAPE: return "unsupported shape";
    case QOQ_ERR_ALIGNMENT: return "misaligned pointer or leading dimension";
    case QOQ_ERR_HIP: return "HIP runtime error";
    case QOQ_ERR_INTERNAL: return "internal error";
    default: return "unknown status";
  }
}

extern "C" const char* qoq_last_error(void) { return qoq::g_err; }
