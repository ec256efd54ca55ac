// host_common.h -- host-side helpers of libfp8q (launch plumbing, device queries).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "fp8q.h"

namespace fp8q {

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Compute units of the current device, cached per device ordinal.
inline int current_device_cus(int* cus) {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FP8Q_EHIP;
  if (dev >= 0 && dev < 64) {
    int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *cus = c;
      return FP8Q_OK;
    }
  }
  int c = 0;
  if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0)
    return FP8Q_EHIP;
  if (dev >= 0 && dev < 64) cache[dev].store(c, std::memory_order_relaxed);
  *cus = c;
  return FP8Q_OK;
}

inline int launch_status(hipError_t e) { return e == hipSuccess ? FP8Q_OK : FP8Q_EHIP; }

}  // namespace fp8q
