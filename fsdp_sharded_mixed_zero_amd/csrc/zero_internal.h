// Internal declarations shared by the host partitioner (layout.cpp) and the
// device code (kernels.hip) of libzero_mi355x.so. Not part of the C ABI.
#pragma once

#include <cstdint>
#include <vector>

#include "zero.h"

struct zero_layout_s {
  std::vector<int64_t> sizes;
  std::vector<int64_t> offsets;  // flat offset of each tensor
  std::vector<zero_segment> segs;
  zero_layout_info info;
};

namespace zero {

// Record a message for zero_last_error() and return `code`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Clear the calling thread's message and return ZERO_OK.
int ok();

}  // namespace zero
