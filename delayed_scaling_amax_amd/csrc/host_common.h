// host_common.h -- host-side helpers of libfp8q (launch plumbing, device queries).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "fp8q.h"
#include "update_grid.h"

namespace fp8q {

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Compute units of the current device, cached per device ordinal.
// The current device's index, for per-device caches of launch shapes: 0..63, or -1 (and
// FP8Q_EHIP from the caller) when it cannot be read or is out of range.
inline int current_device_index() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return -1;
  return dev;
}

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

// Host checks of fp8_amax_and_scale_update's arguments (shared with the fused step).
inline int validate_update(const float* amax, const float* hist, const float* scale,
                           const float* scale_inv, const uint8_t* formats, int64_t n,
                           int64_t history_len, int algo, int margin) {
  if (n < 0 || history_len < 1) return FP8Q_EINVAL;
  if (algo != FP8Q_AMAX_MAX && algo != FP8Q_AMAX_MOST_RECENT) return FP8Q_EINVAL;
  if (margin < -126 || margin > 126) return FP8Q_EINVAL;
  if (n == 0) return FP8Q_OK;
  if (!amax || !hist || !scale || !scale_inv || !formats) return FP8Q_EINVAL;
  if (history_len > (INT64_MAX / 8) / n) return FP8Q_EINVAL;  // H*n floats must be addressable
  // the update kernel addresses the history with 32-bit buffer offsets
  if (history_len * n >= kUpdateMaxElems) return FP8Q_EUNSUPPORTED;
  return FP8Q_OK;
}

}  // namespace fp8q
