// quant_math.h -- element arithmetic of the FP8 quantize shared by the quantize kernels
// (plain, gelu prologue, LayerNorm prologue): saturate, the corrected division by the
// scale, the native OCP convert, the fixed-code patch for inf/NaN/huge quotients, the
// 8-element group forms, magnitude maxima and the bf16 round-to-nearest-even pack.
#pragma once

#include "device_common.h"

namespace fp8q {

// ---------------------------------------------------------------- element math
template <int kFmt>
__device__ __forceinline__ float saturate(float q) {
  constexpr float m = kFmt == FP8Q_E4M3 ? kE4M3Max : kE5M2Max;
  return __builtin_amdgcn_fmed3f(q, -m, m);
}

template <int kFmt>
__device__ __forceinline__ uint32_t pack4(float c0, float c1, float c2, float c3) {
  // the first convert fills bytes 0-1 and the second bytes 2-3, so the initial
  // contents of the word are irrelevant: seed it with a register already live
  int w = __builtin_bit_cast(int, c0);
  if constexpr (kFmt == FP8Q_E4M3) {
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c0, c1, w, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c2, c3, w, true);
  } else {
    w = __builtin_amdgcn_cvt_pk_bf8_f32(c0, c1, w, false);
    w = __builtin_amdgcn_cvt_pk_bf8_f32(c2, c3, w, true);
  }
  return (uint32_t)w;
}

// Quotient for bf16 x inside the window: one Markstein correction.
__device__ __forceinline__ float div_corrected1(float x, float s, float r) {
  float q0 = x * r;
  float e = __builtin_fmaf(q0, s, -x);
  return __builtin_fmaf(-e, r, q0);
}

// Quotient for fp32 x inside the window: two corrections (the first makes the
// quotient faithful, the second rounds it correctly).
__device__ __forceinline__ float div_corrected2(float x, float s, float r) {
  float q0 = x * r;
  float e0 = __builtin_fmaf(q0, s, -x);
  float q1 = __builtin_fmaf(-e0, r, q0);
  float e1 = __builtin_fmaf(q1, s, -x);
  return __builtin_fmaf(-e1, r, q1);
}

// Inside the window an element with |x| >= xlim (magnitude bits) is +-inf, NaN, or
// finite with |x/s| >= 2^125: its code is fixed without any division -- NaN gives 0x7F,
// everything else saturates to the largest finite code -- with the sign bit of x.
template <int kFmt>
__device__ __forceinline__ uint32_t fixed_code(uint32_t mag, uint32_t inf_bits, uint32_t sign) {
  constexpr uint32_t kMaxCode = kFmt == FP8Q_E4M3 ? 0x7Eu : 0x7Bu;
  return (mag > inf_bits ? 0x7Fu : kMaxCode) | sign;
}

// Replace byte k of the 8 codes wherever element k has magnitude >= xlim.  `mag[k]`
// and `sign[k]` (0 or 0x80) are in the source's own bit layout; inf_bits likewise.
template <int kFmt>
__device__ __forceinline__ uint2 patch_codes(uint2 codes, const uint32_t (&mag)[8],
                                             const uint32_t (&sign)[8], uint32_t xlim,
                                             uint32_t inf_bits) {
  uint32_t w[2] = {codes.x, codes.y};
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int sh = 8 * (k & 3);
    const uint32_t fixed = (w[k >> 2] & ~(0xFFu << sh)) |
                           (fixed_code<kFmt>(mag[k], inf_bits, sign[k]) << sh);
    w[k >> 2] = mag[k] >= xlim ? fixed : w[k >> 2];
  }
  return make_uint2(w[0], w[1]);
}

// One element through the IEEE divide: any x, any scale (head/tail elements and
// tensors whose scale lies outside the window).
template <int kFmt>
__device__ __forceinline__ uint32_t code_ieee(float x, float s) {
  const float v = x / s;
  const float c = saturate<kFmt>(v);
  const uint32_t code = pack4<kFmt>(c, c, c, c) & 0xFFu;
  return (v != v) ? (0x7Fu | ((as_uint(x) >> 24) & 0x80u)) : code;
}

// ---------------------------------------------------------------- 8-element groups
// bf16: w holds 8 bf16 values; acc keeps the packed 16-bit magnitude max.
template <int kFmt>
__device__ __forceinline__ uint2 quant8_bf16(uint4 w, float s, float r, uint32_t xlim,
                                             uint32_t& acc) {
  const uint32_t m = pk_max_u16(pk_max_u16(w.x & 0x7FFF7FFFu, w.y & 0x7FFF7FFFu),
                                pk_max_u16(w.z & 0x7FFF7FFFu, w.w & 0x7FFF7FFFu));
  acc = pk_max_u16(acc, m);
  const uint32_t mlo = m & 0xFFFFu, mhi = m >> 16;
  const uint32_t mm = mlo > mhi ? mlo : mhi;
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
  float c[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float x = as_float((k & 1) ? (u[k >> 1] & 0xFFFF0000u) : (u[k >> 1] << 16));
    c[k] = saturate<kFmt>(div_corrected1(x, s, r));
  }
  uint2 out = make_uint2(pack4<kFmt>(c[0], c[1], c[2], c[3]), pack4<kFmt>(c[4], c[5], c[6], c[7]));
  if (mm >= xlim) {  // rare: inf/NaN or a quotient far beyond the FP8 range
    uint32_t mag[8], sign[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t h = (k & 1) ? (u[k >> 1] >> 16) : (u[k >> 1] & 0xFFFFu);
      mag[k] = h & 0x7FFFu;
      sign[k] = (h >> 8) & 0x80u;
    }
    out = patch_codes<kFmt>(out, mag, sign, xlim, 0x7F80u);
  }
  return out;
}

// fp32: lo/hi hold 8 floats; acc keeps the 32-bit magnitude max.
template <int kFmt>
__device__ __forceinline__ uint2 quant8_f32(uint4 lo, uint4 hi, float s, float r, uint32_t xlim,
                                            uint32_t& acc) {
  const uint32_t u[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  uint32_t m = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t a = u[k] & 0x7FFFFFFFu;
    m = m > a ? m : a;
  }
  acc = acc > m ? acc : m;
  float c[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) c[k] = saturate<kFmt>(div_corrected2(as_float(u[k]), s, r));
  uint2 out = make_uint2(pack4<kFmt>(c[0], c[1], c[2], c[3]), pack4<kFmt>(c[4], c[5], c[6], c[7]));
  if (m >= xlim) {
    uint32_t mag[8], sign[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      mag[k] = u[k] & 0x7FFFFFFFu;
      sign[k] = (u[k] >> 24) & 0x80u;
    }
    out = patch_codes<kFmt>(out, mag, sign, xlim, 0x7F800000u);
  }
  return out;
}

// ---------------------------------------------------------------- pass helpers
// The streaming body splits a group's work so that the patch test runs once per pass:
// magnitude max of the group, codes assuming no element needs the fixed-code path,
// and the patch, applied only where the pass max shows it is needed.
__device__ __forceinline__ uint32_t mag8_bf16(uint4 w) {  // packed 16-bit magnitude max
  return pk_max_u16(pk_max_u16(w.x & 0x7FFF7FFFu, w.y & 0x7FFF7FFFu),
                    pk_max_u16(w.z & 0x7FFF7FFFu, w.w & 0x7FFF7FFFu));
}

__device__ __forceinline__ uint32_t mag8_f32(uint4 lo, uint4 hi) {
  const uint32_t u[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  uint32_t m = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t a = u[k] & 0x7FFFFFFFu;
    m = m > a ? m : a;
  }
  return m;
}

template <int kFmt>
__device__ __forceinline__ uint2 codes8_bf16(uint4 w, float s, float r) {
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
  float c[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float x = as_float((k & 1) ? (u[k >> 1] & 0xFFFF0000u) : (u[k >> 1] << 16));
    c[k] = saturate<kFmt>(div_corrected1(x, s, r));
  }
  return make_uint2(pack4<kFmt>(c[0], c[1], c[2], c[3]), pack4<kFmt>(c[4], c[5], c[6], c[7]));
}

// The codes of 8 bf16 values whose quotients cannot exceed FP8_MAX in magnitude (the
// caller has checked that every |x| is at most the value of sat_limit_bf16(s)): the
// saturation step would change nothing and is left out.
template <int kFmt>
__device__ __forceinline__ uint2 codes8_bf16_unsaturated(uint4 w, float s, float r) {
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
  float c[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float x = as_float((k & 1) ? (u[k >> 1] & 0xFFFF0000u) : (u[k >> 1] << 16));
    c[k] = div_corrected1(x, s, r);
  }
  return make_uint2(pack4<kFmt>(c[0], c[1], c[2], c[3]), pack4<kFmt>(c[4], c[5], c[6], c[7]));
}

// Largest bf16 magnitude (bit pattern) whose quotient by s cannot exceed FP8_MAX: two
// binary32 steps below RN(FP8_MAX * s), truncated to bf16, is at most FP8_MAX * s
// exactly, so |x| <= it gives |x / s| <= FP8_MAX and RN32(x / s) <= FP8_MAX.  (s inside
// the division window, so FP8_MAX * s is normal or +inf; +inf gives the largest finite.)
template <int kFmt>
__device__ __forceinline__ uint32_t sat_limit_bf16(float s) {
  constexpr float m = kFmt == FP8Q_E4M3 ? kE4M3Max : kE5M2Max;
  const uint32_t b = as_uint(m * s) - 2u;
  return (b >> 16) < 0x7F7Fu ? (b >> 16) : 0x7F7Fu;
}

template <int kFmt>
__device__ __forceinline__ uint2 codes8_f32(uint4 lo, uint4 hi, float s, float r) {
  const uint32_t u[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  float c[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) c[k] = saturate<kFmt>(div_corrected2(as_float(u[k]), s, r));
  return make_uint2(pack4<kFmt>(c[0], c[1], c[2], c[3]), pack4<kFmt>(c[4], c[5], c[6], c[7]));
}

template <int kFmt>
__device__ __forceinline__ uint2 patch8_bf16(uint2 codes, uint4 w, uint32_t xlim) {
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
  uint32_t mag[8], sign[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t h = (k & 1) ? (u[k >> 1] >> 16) : (u[k >> 1] & 0xFFFFu);
    mag[k] = h & 0x7FFFu;
    sign[k] = (h >> 8) & 0x80u;
  }
  return patch_codes<kFmt>(codes, mag, sign, xlim, 0x7F80u);
}

template <int kFmt>
__device__ __forceinline__ uint2 patch8_f32(uint2 codes, uint4 lo, uint4 hi, uint32_t xlim) {
  const uint32_t u[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  uint32_t mag[8], sign[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    mag[k] = u[k] & 0x7FFFFFFFu;
    sign[k] = (u[k] >> 24) & 0x80u;
  }
  return patch_codes<kFmt>(codes, mag, sign, xlim, 0x7F800000u);
}

__device__ __forceinline__ uint32_t max_halves(uint32_t m) {
  const uint32_t lo = m & 0xFFFFu, hi = m >> 16;
  return lo > hi ? lo : hi;
}

// ---------------------------------------------------------------- bf16 pack, NaN test
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two binary32 values -> packed bf16 (lo in bits 0-15), round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16_rne(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Nonzero if either 16-bit half of a packed magnitude max is a NaN (> 0x7F80).
__device__ __forceinline__ uint32_t halves_nan(uint32_t mg) {
  return (mg + 0x007F007Fu) & 0x80008000u;
}

// ---------------------------------------------------------------- wave-uniform values
__device__ __forceinline__ uint32_t uniform(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ float uniform(float v) {
  return as_float(__builtin_amdgcn_readfirstlane(as_uint(v)));
}

}  // namespace fp8q
