// bw_probe.hip -- measurement probes for the benchmark (libfp8q_probe.so), not part of
// the library's interface.  They move memory the way the delayed-scaling kernels do,
// without the method's arithmetic, so that the benchmark can put the kernels' rates
// next to what the same traffic achieves on the same device:
//
//  * probe_stream: the quantize pass's traffic without its arithmetic.  Each 16-byte
//    unit of the source (8 bf16) is read and 8 bytes are written (the high byte of each
//    element), i.e. 2 bytes read per byte written, with the same cache policies as the
//    quantize kernel (non-temporal loads, device-scope stores, non-temporal as well for
//    launches whose codes exceed the Infinity Cache) or the default ones; also
//    read-only and write-only forms.  Plain persistent grid-stride loop: each thread
//    issues U 16-byte loads, then U 8-byte stores, per iteration; the benchmark sweeps U
//    and the blocks per CU and reports the fastest.
//  * probe_update_floor: the batched scale update's launch (same grid, block and column
//    mapping) with (mode 0) an empty body, or (mode 1) one load -> barrier -> store round
//    trip of exactly the history locations the update loads, stored back unchanged.
//    These are the floors under the update kernel: launch and dispatch alone, and the
//    one memory round trip its in-place roll cannot avoid.
//  * probe_mfma: the matrix cores' sustained rate on the FP8 GEMM's instruction
//    (v_mfma_scale_f32_32x32x64_f8f6f4) with register operands only: each wavefront
//    issues `iters` rounds of 16 independent MFMAs into 16 accumulator tiles (the GEMM's
//    4 x 4 tile grid per wavefront), then stores one checksum per lane.  The ceiling the
//    GEMM's data path and epilogue are measured against.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "update_grid.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// kMode: 0 = read 16 B + write 8 B per unit, 1 = read only, 2 = write only.
// kPolicy: 1 = non-temporal loads and device-scope (sc1) stores, 2 = non-temporal loads
// and non-temporal device-scope (nt | sc1) stores, 0 = default policies.
template <int kMode, int kU, int kPolicy>
__global__ __launch_bounds__(256) void stream_kernel(const uint4* __restrict__ src,
                                                     uint2* __restrict__ dst, int64_t units,
                                                     uint32_t* __restrict__ sink) {
  constexpr int kLd = kPolicy ? 2 : 0;
  constexpr int kSt = kPolicy == 2 ? 18 : kPolicy ? 16 : 0;
  const int64_t step = (int64_t)gridDim.x * 256 * kU;
  uint32_t acc = 0;
  for (int64_t base = (int64_t)blockIdx.x * 256 * kU; base < units; base += step) {
    // a window of 256 * kU units; the descriptor's range drops what lies past the end
    const int64_t left = units - base;
    const uint32_t nu = (uint32_t)(left < 256 * kU ? left : 256 * kU);
    const __amdgpu_buffer_rsrc_t rin = rsrc(src + base, nu * 16);
    const __amdgpu_buffer_rsrc_t rout = rsrc(dst + base, nu * 8);
    uint4 w[kU];
    if constexpr (kMode != 2) {
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const u32x4 q = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rin, threadIdx.x * 16, u * 4096, kLd));
        w[u] = make_uint4(q[0], q[1], q[2], q[3]);
      }
    } else {
#pragma unroll
      for (int u = 0; u < kU; ++u) w[u] = make_uint4((uint32_t)base, u, 0, 0);
    }
    if constexpr (kMode == 1) {
#pragma unroll
      for (int u = 0; u < kU; ++u) acc ^= w[u].x ^ w[u].y ^ w[u].z ^ w[u].w;
    } else {
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        // the high byte of each of the 8 bf16 elements
        const uint32_t lo = __builtin_amdgcn_perm(w[u].y, w[u].x, 0x07050301u);
        const uint32_t hi = __builtin_amdgcn_perm(w[u].w, w[u].z, 0x07050301u);
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{lo, hi}, rout, threadIdx.x * 8, u * 2048,
                                              kSt);
      }
    }
  }
  if constexpr (kMode == 1)
    if (acc == 0x9E3779B9u) sink[0] = acc;  // keeps the loads; practically never taken
}

template <int kMode, int kU, int kPolicy>
const void* stream_fn() {
  return (const void*)stream_kernel<kMode, kU, kPolicy>;
}

template <int kMode, int kPolicy>
const void* stream_fn_u(int u) {
  switch (u) {
    case 2: return stream_fn<kMode, 2, kPolicy>();
    case 4: return stream_fn<kMode, 4, kPolicy>();
    case 8: return stream_fn<kMode, 8, kPolicy>();
    case 16: return stream_fn<kMode, 16, kPolicy>();
    default: return nullptr;
  }
}

using fp8q::kUBlock;
using fp8q::kUCols;
using fp8q::kURows;

__global__ __launch_bounds__(kUBlock) void update_empty_kernel(float* hist, int64_t n, int64_t H,
                                                             int64_t groups,
                                                             int64_t groups_per_xcd, int tpr) {
  const int64_t g = fp8q::update_group(blockIdx.x, groups_per_xcd);
  if (g >= groups) return;
  if (H < 0) hist[threadIdx.x] = 0.0f;  // never: the host passes H >= 1
}

// The update kernel's history traffic (tpr lanes of 4 columns per row, every row it loads
// issued before one barrier), with each row stored back where it was read.
__global__ __launch_bounds__(kUBlock) void update_roundtrip_kernel(float* hist, int64_t n,
                                                                 int64_t H, int64_t groups,
                                                                 int64_t groups_per_xcd,
                                                                 int tpr) {
  const int64_t g = fp8q::update_group(blockIdx.x, groups_per_xcd);
  if (g >= groups) return;
  const int tid = threadIdx.x;
  const int rpp = kUBlock / tpr;
  const uint32_t row_bytes = (uint32_t)(n * 4);
  const int64_t c = g * kUCols + (int64_t)(tid & (tpr - 1)) * 4;
  const uint32_t col_off = (uint32_t)(c * 4);
  const __amdgpu_buffer_rsrc_t r = rsrc(hist, (uint32_t)((H - 1) * n * 4));
  u32x4 v[kURows];
  uint32_t off[kURows];
#pragma unroll
  for (int k = 0; k < kURows; ++k) {
    const int64_t s = tid / tpr + (int64_t)k * rpp;  // source rows [0, H-1)
    off[k] = c < n && s < H - 1 ? (uint32_t)s * row_bytes + col_off : 0x80000000u;
    v[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off[k], 0, 0));
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kURows; ++k) __builtin_amdgcn_raw_buffer_store_b128(v[k], r, off[k], 0, 0);
}

typedef int mfma_v8i __attribute__((ext_vector_type(8)));
typedef float mfma_v16f __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void mfma_kernel(int iters, float* sink) {
  // operands: E4M3 1.0 (0x38) in every byte, chosen at run time so that nothing folds
  const uint32_t one = iters > 0 ? 0x38383838u : 0u;
  const mfma_v8i a = {(int)one, (int)one, (int)one, (int)one, (int)one, (int)one, (int)one, (int)one};
  mfma_v16f acc[16];
#pragma unroll
  for (int t = 0; t < 16; ++t) acc[t] = mfma_v16f{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int t = 0; t < 16; ++t)
      acc[t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, a, acc[t], 0, 0, 0, 127, 0,
                                                               127);
  }
  float sum = 0.0f;
#pragma unroll
  for (int t = 0; t < 16; ++t) sum += acc[t][0];
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = sum;
}

}  // namespace

extern "C" {

// `blocks` blocks of 256 threads, each wavefront `iters` x 16 MFMAs of 32 x 32 x 64 (FP8):
// blocks * 4 * iters * 16 * 131072 flops.  sink: device float[blocks * 256].  start/stop as
// probe_stream.  Returns 0, -1 for an invalid argument, -3 for a launch failure.
int probe_mfma(int blocks, int iters, float* sink, void* stream, void* start, void* stop) {
  if (blocks <= 0 || iters <= 0 || !sink) return -1;
  void* args[] = {&iters, &sink};
  const void* fn = (const void*)mfma_kernel;
  const hipError_t e =
      start || stop
          ? hipExtLaunchKernel(fn, dim3((unsigned)blocks), dim3(256), args, 0,
                               (hipStream_t)stream, (hipEvent_t)start, (hipEvent_t)stop, 0)
          : hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(256), args, 0, (hipStream_t)stream);
  return e == hipSuccess ? 0 : -3;
}

// Stream `units` 16-byte units: mode 0 reads src and writes dst (8 bytes per unit),
// 1 reads src only, 2 writes dst only.  u in {2, 4, 8, 16} loads in flight per thread,
// blocks = grid size (persistent, grid-stride), policy 1 = the quantize kernel's cache
// policies, 0 = defaults.  src holds units * 16 bytes, dst units * 8; sink: a device
// uint32 (mode 1).  start/stop: hipEvent_t or NULL; when given, they take the kernel's own
// start and stop time (hipExtLaunchKernel), as the quantize entry point's timed form does.
// Returns 0, or -1 for an invalid argument, -3 for a launch failure.
int probe_stream(const void* src, void* dst, int64_t units, int mode, int u, int blocks,
                 int policy, uint32_t* sink, void* stream, void* start, void* stop) {
  if (units <= 0 || blocks <= 0 || mode < 0 || mode > 2 || (mode != 2 && !src) ||
      (mode != 1 && !dst) || (mode == 1 && !sink))
    return -1;
  const void* fn = nullptr;
  if (policy < 0 || policy > 2) return -1;
  if (mode == 0)
    fn = policy == 2 ? stream_fn_u<0, 2>(u) : policy ? stream_fn_u<0, 1>(u) : stream_fn_u<0, 0>(u);
  if (mode == 1) fn = policy ? stream_fn_u<1, 1>(u) : stream_fn_u<1, 0>(u);
  if (mode == 2)
    fn = policy == 2 ? stream_fn_u<2, 2>(u) : policy ? stream_fn_u<2, 1>(u) : stream_fn_u<2, 0>(u);
  if (fn == nullptr) return -1;
  void* args[] = {(void*)&src, &dst, &units, &sink};
  const hipError_t e =
      start || stop
          ? hipExtLaunchKernel(fn, dim3((unsigned)blocks), dim3(256), args, 0,
                               (hipStream_t)stream, (hipEvent_t)start, (hipEvent_t)stop, 0)
          : hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(256), args, 0, (hipStream_t)stream);
  return e == hipSuccess ? 0 : -3;
}

// The update's launch for n tensors x H history rows (hist: device float[H][n], n % 4 == 0,
// 16-byte aligned, H * n < 2^29): mode 0 = empty body, mode 1 = one load -> barrier ->
// store round trip of the rows the update loads (stored back unchanged).
int probe_update_floor(float* hist, int64_t n, int64_t H, int mode, void* stream) {
  if (!hist || n <= 0 || n % 4 != 0 || H < 1 || H * n >= fp8q::kUpdateMaxElems ||
      (uintptr_t)hist % 16 != 0 || (mode != 0 && mode != 1))
    return -1;
  int tpr = fp8q::update_tpr(n, 4);
  if (mode == 1 && H - 1 > (int64_t)(kUBlock / tpr) * kURows) return -1;
  const fp8q::UpdateGrid grid = fp8q::update_grid(n);
  int64_t groups = grid.groups, per_xcd = grid.groups_per_xcd;
  void* args[] = {&hist, &n, &H, &groups, &per_xcd, &tpr};
  const void* fn = mode == 0 ? (const void*)update_empty_kernel
                             : (const void*)update_roundtrip_kernel;
  return hipLaunchKernel(fn, dim3((unsigned)grid.blocks), dim3(kUBlock), args, 0,
                         (hipStream_t)stream) == hipSuccess
             ? 0
             : -3;
}

}  // extern "C"
