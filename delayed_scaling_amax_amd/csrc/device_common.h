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

// One step of a DPP max: lanes whose DPP source is invalid or whose row is outside
// kRowMask read 0 (the identity of the unsigned max) and keep v.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ uint32_t dpp_max_step(uint32_t v) {
  const uint32_t t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kCtrl, kRowMask, 0xF, false);
  return v > t ? v : t;
}

// Max over the 64 lanes of a wavefront on the DPP network (no LDS round trips): xor-1
// and xor-2 within quads, rotations by 4 and 8 within each 16-lane row, then rows 0 and
// 1, 2 and 3 (row_bcast15) and the two halves (row_bcast31) into lane 63, whose value
// every lane gets through a scalar register.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = dpp_max_step<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v = dpp_max_step<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v = dpp_max_step<0x124, 0xF>(v);  // row_ror:4
  v = dpp_max_step<0x128, 0xF>(v);  // row_ror:8
  v = dpp_max_step<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v = dpp_max_step<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Max of v over the lanes of the wavefront whose index agrees with this lane's modulo
// `tpr` (a power of two, 1..32; wave-uniform), returned in every lane, without LDS:
// lane l with l + 32 and l + 16 through the gfx950 lane-swap instructions
// (v_permlane32_swap / v_permlane16_swap with both operands v: one result holds each
// lane's partner), then rotations by 8 and 4 within each 16-lane row and the xor-2 and
// xor-1 quad permutations on the DPP network.
__device__ __forceinline__ uint32_t lane_class_max(uint32_t v, int tpr) {
  if (tpr <= 32) {
    const auto w = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    v = (uint32_t)w[0] > (uint32_t)w[1] ? (uint32_t)w[0] : (uint32_t)w[1];
  }
  if (tpr <= 16) {
    const auto w = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = (uint32_t)w[0] > (uint32_t)w[1] ? (uint32_t)w[0] : (uint32_t)w[1];
  }
  if (tpr <= 8) v = dpp_max_step<0x128, 0xF>(v);  // row_ror:8
  if (tpr <= 4) v = dpp_max_step<0x124, 0xF>(v);  // row_ror:4
  if (tpr <= 2) v = dpp_max_step<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  if (tpr <= 1) v = dpp_max_step<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  return v;
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
