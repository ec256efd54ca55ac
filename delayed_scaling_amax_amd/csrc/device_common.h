// device_common.h -- small gfx950 device helpers shared by the libfp8q kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8q {

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr float kE4M3Max = 448.0f;    // largest finite float8_e4m3fn
constexpr float kE5M2Max = 57344.0f;  // largest finite float8_e5m2

__device__ __forceinline__ float as_float(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t as_uint(float f) { return __float_as_uint(f); }

// Lane-wise unsigned max of the two 16-bit halves (one v_pk_max_u16).
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                __builtin_bit_cast(u16x2, b)));
}

// Max over the 64 lanes of a wavefront (butterfly through ds_swizzle/bpermute).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    uint32_t o = __shfl_xor(v, off, 64);
    v = v > o ? v : o;
  }
  return v;
}

// Block-wide max of one value per thread; every thread gets the result.  `red`
// holds one slot per wavefront.  Contains two barriers: all threads must call it.
template <int kBlock>
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* red) {
  v = wave_max_u32(v);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  uint32_t r = red[0];
#pragma unroll
  for (int w = 1; w < kBlock / 64; ++w) r = r > red[w] ? r : red[w];
  __syncthreads();  // red may be reused right after
  return r;
}

// Max-accumulate a block's amax bits v into the tensor's amax at p (binary32 bit
// patterns, unsigned order, device scope).  The atomic is skipped when p already holds v
// or more: p only grows, so any value read from it is at most the final one.  Hundreds
// of blocks that finish together would otherwise queue atomics on one address (measured
// ~3 us on a 16M-element launch of 512 blocks).
__device__ __forceinline__ void amax_accumulate(uint32_t* p, uint32_t v) {
  const uint32_t cur = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (v > cur) atomicMax(p, v);
}

// New scale of one tensor from its selected amax (bit pattern `sel_bits`): RN32(sel /
// FP8_MAX) * 2^margin, or the previous scale when sel or the result is not finite or
// not > 0 ("User Guide on Native XLA-FP8", section "JAX": scale = amax / FP8_MAX).
__device__ __forceinline__ float next_scale(uint32_t sel_bits, uint32_t fmt, float s_old,
                                            int margin) {
  const float sel = as_float(sel_bits);
  const float fmax = fmt ? kE5M2Max : kE4M3Max;
  float s = s_old;
  if (__builtin_isfinite(sel) && sel > 0.0f) {
    float c = sel / fmax;
    c = ldexpf(c, margin);
    if (__builtin_isfinite(c) && c > 0.0f) s = c;
  }
  return s;
}

}  // namespace fp8q
