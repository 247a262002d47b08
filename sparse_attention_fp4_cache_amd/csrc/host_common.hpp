// host_common.hpp -- host-side helpers of the C ABI entry points.
#pragma once

#include <hip/hip_runtime.h>

#include "csa2fp4.h"

namespace csa2 {

// Every entry point validates on the host first; a launch error afterwards maps
// to CSA2_ERR_LAUNCH.  hipGetLastError also clears the sticky launch error.
inline int launch_status() { return hipGetLastError() == hipSuccess ? CSA2_OK : CSA2_ERR_LAUNCH; }

inline bool cache_ok(const csa2_fp4_cache* c) {
  return c && c->main_codes && c->main_scales && c->idx_codes && c->idx_scales;
}

inline bool cache_shape_ok(const csa2_fp4_cache* c) {
  return c->page_size == CSA2_PAGE_SIZE && c->num_slots > 0 && c->num_slots % CSA2_PAGE_SIZE == 0;
}

inline unsigned ceil_div(long long a, long long b) { return (unsigned)((a + b - 1) / b); }

// Compute units of the current device (read once per device; 256 on MI355X).
inline int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

}  // namespace csa2
