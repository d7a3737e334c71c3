// Internal helpers shared by the host packer, the device launchers and the
// C-ABI shims of libqoq.so.  Not part of the public interface (include/qoq.h).
#pragma once

#include <cstdint>
#include <cstdio>
#include <cstdarg>
#include <string>

#include "qoq.h"

namespace qoq {

// Record a failure for qoq_last_error() and return the status.
int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

constexpr int kGroup = QOQ_GROUP;   // K-loop unit and g128 group size
constexpr int kStrip = 16;          // output channels per packed strip
constexpr int kSlots = 64;          // 16-byte slots per (strip, group) block
constexpr int kBlockBytes = kSlots * 16;
constexpr int kBlockBytesW8 = 2 * kBlockBytes;  // INT8 weights: 128 slots per (strip, group)

inline int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }

// Largest K for which 127*127*K stays below 2^31 (exact INT32 accumulation).
constexpr int64_t kMaxK = (int64_t(1) << 31) / (127 * 127) - 1;

// Shape checks common to packer and GEMM; returns QOQ_OK or a failure.
int check_weight_shape(int64_t N, int64_t K, int32_t group_size);

// Byte offset of the UINT4 code of (channel c of strip, input k) inside a
// 1024-byte (strip, group) block, and whether it is the high nibble.
// Slot (c, j) holds k_local in {16j + 64h + 8(p%2) + b (+4 for the high
// nibble)}: see the layout comment in qoq.h.
inline void code_position(int c, int k_local, int* byte_off, int* high) {
  const int h64 = k_local >> 6;        // which 64-wide half of the group
  const int r = k_local & 63;
  const int j = r >> 4;                // 16-wide quarter -> slot row
  const int t = r & 15;                // position inside the 16 values
  const int d = (h64 << 2) | (t >> 2); // output dword index 0..7
  const int b = t & 3;
  const int p = d >> 1;
  *high = d & 1;
  *byte_off = (c + 16 * j) * 16 + p * 4 + b;
}

}  // namespace qoq
