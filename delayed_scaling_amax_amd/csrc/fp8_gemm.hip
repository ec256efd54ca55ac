// fp8_gemm.hip -- the consumer of the quantized tensors: an FP8 GEMM with per-tensor
// scales on the gfx950 matrix cores.
//
// What it computes ("User Guide on Native XLA-FP8", section "JAX": FP8 operands are cast
// up, multiplied by their scales, and fed to the dot; the page's matmul takes two FP8
// tensors and two binary32 scalar scales):
//   C[m][n] = sa * sb * sum_k decode(A[m][k]) * decode(B[n][k])
// with A (M x K) and B (N x K) both K-contiguous (the layout FP8 matmuls require; a
// weight stored K x N is quantized from its transpose), C (M x N) row-major in bf16 or
// fp32.  The FP8 products are exact; the matrix cores accumulate them in binary32.
//
// Design (v1):
//  * Block tile 256 x 256, 4 wavefronts as 2 x 2, each owning 128 x 128 = 4 x 4 tiles of
//    v_mfma_scale_f32_32x32x64_f8f6f4 (E8M0 scales fixed at 1; the per-tensor scales are
//    applied once in the epilogue).  256 binary32 accumulators per lane.
//  * K advances 64 bytes per step: the block's A and B tiles (256 x 64 bytes each) go
//    global -> registers -> LDS through 16-byte buffer loads, double-buffered in LDS so
//    the next tile's loads are in flight while the matrix cores work on the current
//    one; one barrier per step.  Rows are padded to 80 bytes in LDS.
//  * Each lane's MFMA operand is 32 bytes of one row (row = lane mod 32, bytes 32 x
//    (lane / 32) of the 64-byte step), read with two ds_read_b128; A and B use the same
//    lane -> k assignment, so every output is the dot product over the same k set.
//  * Edges: rows past M or N and 16-byte chunks past K are loaded through offsets outside
//    the buffer resource, which the hardware returns as zeros; stores are masked.
#include "device_common.h"
#include "host_common.h"
#include "quant_math.h"
#include "fp8q.h"

namespace fp8q {

constexpr int kGBM = 256;      // block tile rows (A)
constexpr int kGBN = 256;      // block tile columns (B rows)
constexpr int kGBK = 64;       // bytes of K per step (one MFMA)
constexpr int kGPitch = 80;    // LDS row pitch in bytes (64 + 16)
constexpr int kGThreads = 256;
constexpr int kGStage = (kGBM + kGBN) * kGPitch;  // bytes per LDS stage

struct GemmArgs {
  const uint8_t* A;
  const uint8_t* B;
  void* C;
  const float* sa;
  const float* sb;
  int64_t M, N, K;
  int64_t nbn;  // column tiles
};

typedef int g_v8i __attribute__((ext_vector_type(8)));
typedef float g_v16f __attribute__((ext_vector_type(16)));
typedef uint32_t g_u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t g_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ uint4 g_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  const g_u32x4 v = __builtin_bit_cast(g_u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// The thread's 4 chunks of a 256-row x 64-byte tile: chunk c = tid + 256 i covers row
// c / 4, bytes 16 (c mod 4) .. +15 of the step.  Chunks past K read as zeros.
__device__ __forceinline__ void g_tile_load(uint4 (&st)[4], __amdgpu_buffer_rsrc_t r, int64_t K,
                                            int64_t k0, int tid) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + kGThreads * i;
    const int row = c >> 2;
    const int64_t k = k0 + 16 * (c & 3);
    const uint32_t voff = k < K ? (uint32_t)(row * K + k) : 0xFFFFFFF0u;  // past the resource
    st[i] = g_load16(r, voff);
  }
}

__device__ __forceinline__ void g_tile_store(const uint4 (&st)[4], uint8_t* tile, int tid) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + kGThreads * i;
    *(uint4*)(tile + (c >> 2) * kGPitch + 16 * (c & 3)) = st[i];
  }
}

// 32 bytes of row `row` of a tile: the lane's MFMA operand.
__device__ __forceinline__ g_v8i g_frag(const uint8_t* tile, int row, int half) {
  const uint4 lo = *(const uint4*)(tile + row * kGPitch + 32 * half);
  const uint4 hi = *(const uint4*)(tile + row * kGPitch + 32 * half + 16);
  return g_v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

template <int kFa, int kFb, bool kBf16Out>
__global__ __launch_bounds__(kGThreads) void fp8_gemm_kernel(const GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kGStage];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t bm = blockIdx.x / g.nbn, bn = blockIdx.x % g.nbn;
  const int64_t m0 = bm * kGBM, n0 = bn * kGBN;
  const int64_t rows_a = g.M - m0 < kGBM ? g.M - m0 : kGBM;
  const int64_t rows_b = g.N - n0 < kGBN ? g.N - n0 : kGBN;
  // resources over exactly the block's rows (whole K): rows past M / N read as zeros
  const __amdgpu_buffer_rsrc_t ra = g_rsrc(g.A + m0 * g.K, (uint32_t)(rows_a * g.K));
  const __amdgpu_buffer_rsrc_t rb = g_rsrc(g.B + n0 * g.K, (uint32_t)(rows_b * g.K));

  g_v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = g_v16f{};

  const int64_t nk = (g.K + kGBK - 1) / kGBK;
  uint4 sa_[4], sb_[4];
  if (nk > 0) {
    g_tile_load(sa_, ra, g.K, 0, tid);
    g_tile_load(sb_, rb, g.K, 0, tid);
    g_tile_store(sa_, lds, tid);
    g_tile_store(sb_, lds + kGBM * kGPitch, tid);
  }
  __syncthreads();
  const int frow = lane & 31, fhalf = lane >> 5;
  for (int64_t kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    if (more) {
      g_tile_load(sa_, ra, g.K, (kt + 1) * kGBK, tid);
      g_tile_load(sb_, rb, g.K, (kt + 1) * kGBK, tid);
    }
    const uint8_t* ta = lds + (kt & 1) * kGStage;
    const uint8_t* tb = ta + kGBM * kGPitch;
    g_v8i af[4], bf[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) af[i] = g_frag(ta, wm * 128 + i * 32 + frow, fhalf);
#pragma unroll
    for (int j = 0; j < 4; ++j) bf[j] = g_frag(tb, wn * 128 + j * 32 + frow, fhalf);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bf[j], acc[i][j], kFa,
                                                                   kFb, 0, 127, 0, 127);
    if (more) {
      uint8_t* nxt = lds + ((kt + 1) & 1) * kGStage;
      g_tile_store(sa_, nxt, tid);
      g_tile_store(sb_, nxt + kGBM * kGPitch, tid);
    }
    __syncthreads();
  }

  // epilogue: C = acc * (sa * sb); accumulator r of a 32 x 32 tile holds row
  // (r mod 4) + 8 (r / 4) + 4 (lane / 32), column lane mod 32
  const float s = uniform(*g.sa) * uniform(*g.sb);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t col = n0 + wn * 128 + j * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * 128 + i * 32 + (r & 3) + 8 * (r >> 2) + 4 * (lane >> 5);
        if (row < g.M && col < g.N) {
          const float v = acc[i][j][r] * s;
          if constexpr (kBf16Out)
            ((uint16_t*)g.C)[row * g.N + col] = (uint16_t)(pack_bf16_rne(v, 0.0f) & 0xFFFFu);
          else
            ((float*)g.C)[row * g.N + col] = v;
        }
      }
    }
}

template <int kFa, int kFb>
static int gemm_launch(const GemmArgs& g, bool bf16_out, hipStream_t stream) {
  const void* fn = bf16_out ? (const void*)fp8_gemm_kernel<kFa, kFb, true>
                            : (const void*)fp8_gemm_kernel<kFa, kFb, false>;
  const int64_t nbm = (g.M + kGBM - 1) / kGBM;
  const int64_t blocks = nbm * g.nbn;
  void* args[] = {(void*)&g};
  return launch_status(hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(kGThreads), args, 0, stream));
}

}  // namespace fp8q

using namespace fp8q;

extern "C" int fp8_gemm(const uint8_t* A, int a_format, const uint8_t* B, int b_format,
                        int64_t M, int64_t N, int64_t K, const float* a_scale,
                        const float* b_scale, void* C, int c_dtype, void* stream) {
  if (M < 0 || N < 0 || K < 0) return FP8Q_EINVAL;
  if ((a_format != FP8Q_E4M3 && a_format != FP8Q_E5M2) ||
      (b_format != FP8Q_E4M3 && b_format != FP8Q_E5M2))
    return FP8Q_EINVAL;
  if (c_dtype != FP8Q_BF16 && c_dtype != FP8Q_F32) return FP8Q_EINVAL;
  if (a_scale == nullptr || b_scale == nullptr) return FP8Q_EINVAL;
  if (M == 0 || N == 0) return FP8Q_OK;
  if (C == nullptr || (K > 0 && (A == nullptr || B == nullptr))) return FP8Q_EINVAL;
  if (K % 16 != 0) return FP8Q_EUNSUPPORTED;
  if ((uintptr_t)A % 16 != 0 || (uintptr_t)B % 16 != 0) return FP8Q_EUNSUPPORTED;
  if ((uintptr_t)C % (c_dtype == FP8Q_BF16 ? 2 : 4) != 0) return FP8Q_EINVAL;
  // a block's operand resource (256 rows x K bytes) must fit 32-bit offsets
  if (K > ((int64_t)1 << 23)) return FP8Q_EUNSUPPORTED;
  const int64_t nbm = (M + kGBM - 1) / kGBM, nbn = (N + kGBN - 1) / kGBN;
  if (nbm > INT32_MAX / nbn) return FP8Q_EUNSUPPORTED;
  GemmArgs g;
  g.A = A;
  g.B = B;
  g.C = C;
  g.sa = a_scale;
  g.sb = b_scale;
  g.M = M;
  g.N = N;
  g.K = K;
  g.nbn = nbn;
  const bool bf16 = c_dtype == FP8Q_BF16;
  const hipStream_t st = (hipStream_t)stream;
  if (a_format == FP8Q_E4M3)
    return b_format == FP8Q_E4M3 ? gemm_launch<0, 0>(g, bf16, st) : gemm_launch<0, 1>(g, bf16, st);
  return b_format == FP8Q_E4M3 ? gemm_launch<1, 0>(g, bf16, st) : gemm_launch<1, 1>(g, bf16, st);
}
