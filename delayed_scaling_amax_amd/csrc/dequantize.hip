// dequantize.hip -- FP8 codes times scale, to fp32 or bf16.
//
// What it computes ("User Guide on Native XLA-FP8", section "JAX": dequantization
// casts the FP8 tensor up to a wide type and multiplies it by its scale):
//   y = RN32(decode(code) * scale), written as fp32, or rounded to nearest even to bf16.
// A NaN result is written as the quiet NaN 0x7FC00000 (bf16 0x7FC0) with the code's
// sign bit.  Decoding uses the native OCP converts v_cvt_pk_f32_fp8 / _bf8 (exact).
//
// Schedule: grid-stride over 8-code groups (8-byte loads; 32- or 16-byte stores)
// with the unaligned head/tail element-wise, like the quantize kernel.
#include "device_common.h"
#include "host_common.h"

namespace fp8q {

constexpr int kDBlock = 256;
constexpr int kDBlocksPerCU = 8;

template <int kFmt>
__device__ __forceinline__ void decode4(uint32_t w, float* d) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  f32x2 lo, hi;
  if constexpr (kFmt == FP8Q_E4M3) {
    lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
    hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  } else {
    lo = __builtin_amdgcn_cvt_pk_f32_bf8((int)w, false);
    hi = __builtin_amdgcn_cvt_pk_f32_bf8((int)w, true);
  }
  d[0] = lo[0]; d[1] = lo[1]; d[2] = hi[0]; d[3] = hi[1];
}

// y bits for one decoded value: NaN results canonicalised with the code's sign.
__device__ __forceinline__ uint32_t scaled_bits(float d, float s, uint32_t code) {
  const float y = d * s;
  return (y != y) ? (0x7FC00000u | ((code & 0x80u) << 24)) : as_uint(y);
}

// binary32 bits -> bf16 bits, round to nearest even (NaN already canonical).
__device__ __forceinline__ uint32_t bf16_rne(uint32_t u) {
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return u >> 16;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

template <int kFmt, bool kBF16Out>
__global__ __launch_bounds__(kDBlock) void dequantize_kernel(const uint8_t* __restrict__ src,
                                                             void* __restrict__ dst,
                                                             const float* __restrict__ scale,
                                                             int64_t head, int64_t n_vec,
                                                             int64_t numel) {
  const float s = *scale;
  const int64_t stride = (int64_t)gridDim.x * kDBlock;
  const uint2* in = (const uint2*)(src + head);
  for (int64_t g = (int64_t)blockIdx.x * kDBlock + threadIdx.x; g < n_vec; g += stride) {
    const uint2 c = in[g];
    float d[8];
    decode4<kFmt>(c.x, d);
    decode4<kFmt>(c.y, d + 4);
    uint32_t y[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) y[k] = scaled_bits(d[k], s, (k < 4 ? c.x : c.y) >> (8 * (k & 3)));
    if constexpr (kBF16Out) {
      uint4 o;
      o.x = bf16_rne(y[0]) | (bf16_rne(y[1]) << 16);
      o.y = bf16_rne(y[2]) | (bf16_rne(y[3]) << 16);
      o.z = bf16_rne(y[4]) | (bf16_rne(y[5]) << 16);
      o.w = bf16_rne(y[6]) | (bf16_rne(y[7]) << 16);
      ((uint4*)((uint16_t*)dst + head))[g] = o;
    } else {
      uint4* o = (uint4*)((float*)dst + head) + 2 * g;
      o[0] = make_uint4(y[0], y[1], y[2], y[3]);
      o[1] = make_uint4(y[4], y[5], y[6], y[7]);
    }
  }
  // head [0, head) and tail [head + 8*n_vec, numel), element-wise
  const int64_t n_scalar = numel - 8 * n_vec;
  for (int64_t j = (int64_t)blockIdx.x * kDBlock + threadIdx.x; j < n_scalar; j += stride) {
    const int64_t i = j < head ? j : j + 8 * n_vec;
    const uint32_t code = src[i];
    float d[4];
    decode4<kFmt>(code, d);
    const uint32_t y = scaled_bits(d[0], s, code);
    if constexpr (kBF16Out) ((uint16_t*)dst)[i] = (uint16_t)bf16_rne(y);
    else ((uint32_t*)dst)[i] = y;
  }
}

}  // namespace fp8q

using namespace fp8q;

extern "C" int fp8_dequantize(const uint8_t* src, int format, void* dst, int dst_dtype,
                              int64_t numel, const float* scale, void* stream) {
  if (numel < 0 || scale == nullptr) return FP8Q_EINVAL;
  if (format != FP8Q_E4M3 && format != FP8Q_E5M2) return FP8Q_EINVAL;
  if (dst_dtype != FP8Q_BF16 && dst_dtype != FP8Q_F32) return FP8Q_EINVAL;
  if (numel > 0 && (src == nullptr || dst == nullptr)) return FP8Q_EINVAL;
  if (numel == 0) return FP8Q_OK;
  const int64_t osz = dst_dtype == FP8Q_BF16 ? 2 : 4;
  int64_t head = -1;
  for (int64_t h = 0; h < 8; ++h)
    if (((uintptr_t)src + h) % 8 == 0 && ((uintptr_t)dst + h * osz) % 16 == 0) {
      head = h;
      break;
    }
  int64_t n_vec = 0;
  if (head < 0 || numel < head + 8) head = numel;
  else n_vec = (numel - head) / 8;
  int cus = 0;
  int st = current_device_cus(&cus);
  if (st != FP8Q_OK) return st;
  int64_t work = n_vec > 0 ? n_vec : numel;
  int64_t blocks = ceil_div(work, kDBlock);
  if (blocks > (int64_t)cus * kDBlocksPerCU) blocks = (int64_t)cus * kDBlocksPerCU;
  if (blocks < 1) blocks = 1;
  void* args[] = {(void*)&src, &dst, (void*)&scale, &head, &n_vec, &numel};
  const void* fn;
  if (format == FP8Q_E4M3)
    fn = dst_dtype == FP8Q_BF16 ? (const void*)dequantize_kernel<FP8Q_E4M3, true>
                                : (const void*)dequantize_kernel<FP8Q_E4M3, false>;
  else
    fn = dst_dtype == FP8Q_BF16 ? (const void*)dequantize_kernel<FP8Q_E5M2, true>
                                : (const void*)dequantize_kernel<FP8Q_E5M2, false>;
  return launch_status(hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(kDBlock), args, 0,
                                       (hipStream_t)stream));
}
