// Internal helpers shared by the library's translation units (not installed).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "dtree.h"

namespace dt {

#define DT_TRY_HIP(expr)                      \
  do {                                        \
    hipError_t dt_e_ = (expr);                \
    if (dt_e_ != hipSuccess) return DT_ERR_HIP; \
  } while (0)

// Compute-unit count of the current device, cached once per device.
int current_device_cus(int* cus);

inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline size_t round_up(size_t a, size_t b) { return (a + b - 1) / b * b; }

// After enqueueing kernels: report a launch failure as DT_ERR_HIP.
inline int launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? DT_OK : DT_ERR_HIP;
}

}  // namespace dt
