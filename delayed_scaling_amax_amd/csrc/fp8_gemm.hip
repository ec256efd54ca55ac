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
// Design:
//  * Block tile 256 x 256, 4 wavefronts as 2 x 2, each owning 128 x 128 = 4 x 4 tiles of
//    v_mfma_scale_f32_32x32x64_f8f6f4 (E8M0 scales fixed at 1; the per-tensor scales are
//    applied once in the epilogue).  256 binary32 accumulators per lane.
//  * K advances 128 bytes per stage (whole 128-byte lines of every row, so no line is
//    fetched twice) through a 2-stage LDS ring filled by LDS DMA (buffer loads that
//    write LDS directly: no registers, no LDS store instructions).  A stage is consumed
//    in two MFMA sub-steps of 64 bytes; the fragments of the next sub-step are read from
//    LDS while the 16 MFMAs of the current one run, and the DMA of stage t + 2 is issued
//    right after the one barrier per stage.  Tiles are unpadded 128-byte rows with the
//    16-byte chunks XOR-swizzled by row pair, so the fragment reads are free of bank
//    conflicts.
//  * Each lane's MFMA operand is 32 bytes of one row (row = lane mod 32, logical chunks
//    4 h + 2 (lane / 32) and + 1 in sub-step h), read with two ds_read_b128; A and B use
//    the same lane -> k assignment, so every output is the dot product over the same k
//    set.
//  * Edges: rows past M or N and 16-byte chunks past K are loaded through offsets outside
//    the buffer resource, which the hardware returns as zeros; stores are masked.
//  * Epilogue: bf16 output with N a multiple of 8 goes through LDS (the ring is free by
//    then) and leaves as 16-byte row-contiguous stores; otherwise element stores.
//  * Tile order: row-major over the tile grid (block b is tile b).  A and B of the MLP
//    shapes (tens of MB) stay in the 256 MB MALL, so re-reads of a slice by blocks on
//    other XCDs rarely reach HBM; a remap giving each XCD a contiguous tile range measured
//    slower on the large shapes.
#include "device_common.h"
#include "host_common.h"
#include "quant_math.h"
#include "fp8q.h"

namespace fp8q {

constexpr int kGBM = 256;      // block tile rows (A)
constexpr int kGBN = 256;      // block tile columns (B rows)
constexpr int kGBK = 128;      // bytes of K per stage (two MFMA steps)
constexpr int kGThreads = 256;
constexpr int kGStages = 2;    // LDS ring: stage t + 2 loads while t + 1 waits
constexpr int kGTileBytes = kGBM * kGBK;  // 32 KB per operand per stage
constexpr int kGDmaPerWave = kGTileBytes / 1024 / (kGThreads / 64);  // 1 KB DMA ops per wave

struct GemmArgs {
  const uint8_t* A;
  const uint8_t* B;
  void* C;
  const float* sa;
  const float* sb;
  int64_t M, N, K;
  int64_t nbn;    // column tiles
  int32_t vec_c;  // bf16 C with N % 8 == 0 and 16-byte alignment: 16-byte row stores
  int32_t pad;
};

typedef int g_v8i __attribute__((ext_vector_type(8)));
typedef float g_v16f __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void g_lds_t;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t g_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// LDS layout of a stage tile: row r (128 bytes = 8 chunks of 16), logical chunk c stored
// in slot c ^ swz(r), swz(r) = (r >> 1) & 7: the 16 rows read together by a fragment
// load (rows r0 .. r0 + 15, r0 even) fall in 16 distinct 16-byte groups of the 256-byte
// bank space.
__device__ __forceinline__ int g_swz(int r) { return (r >> 1) & 7; }

// Wavefront's share of one stage of both operands: 1 KB DMA op j (tile rows
// 8 (w kGDmaPerWave + j) .. +7) writes lane l's 16 bytes to row 8 j' + l / 8, slot
// l mod 8, loading the logical chunk held there.  A and B tiles have the same shape, so
// one offset serves both.  Rows past the resource (M or N) and chunks past K load zeros
// (offset 0xFFFFFFF0 is past every resource; K is a multiple of 16, so in-range offsets
// have their low 4 bits clear and the OR below yields that offset).
__device__ __forceinline__ void g_stage_dma(g_lds_t* ta, g_lds_t* tb, __amdgpu_buffer_rsrc_t ra,
                                            __amdgpu_buffer_rsrc_t rb, int64_t K, int64_t k0,
                                            int wave, int lane) {
#pragma unroll
  for (int j = 0; j < kGDmaPerWave; ++j) {
    const int blk = wave * kGDmaPerWave + j;
    const int row = 8 * blk + (lane >> 3);
    const int c = (lane & 7) ^ g_swz(row);
    const int64_t k = k0 + 16 * c;
    const uint32_t past = 0u - (uint32_t)(k >= K);
    const uint32_t voff = (uint32_t)(row * K + k) | (past & 0xFFFFFFF0u);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (g_lds_t*)((__attribute__((address_space(3))) uint8_t*)ta + 1024 * blk),
                                             16, voff, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (g_lds_t*)((__attribute__((address_space(3))) uint8_t*)tb + 1024 * blk),
                                             16, voff, 0, 0, 0);
  }
}

// 32 bytes (logical chunks ch, ch + 1) of tile row `row`: a lane's MFMA operand.
__device__ __forceinline__ g_v8i g_frag(const uint8_t* tile, int row, int ch) {
  const int sw = g_swz(row);
  const uint4 lo = *(const uint4*)(tile + row * kGBK + 16 * (ch ^ sw));
  const uint4 hi = *(const uint4*)(tile + row * kGBK + 16 * ((ch + 1) ^ sw));
  return g_v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// s_waitcnt: at most n vector-memory operations outstanding (the LDS counter left
// free, or, in the second form, drained too).
#define G_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (0x7 << 4) | (0xF << 8) | (((n) >> 4) << 14))
#define G_WAIT_VMCNT_LGKM0(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (0x7 << 4) | (((n) >> 4) << 14))

template <int kFa, int kFb, bool kBf16Out>
__global__ __launch_bounds__(kGThreads) void fp8_gemm_kernel(const GemmArgs g) {
  // one LDS object per stage and operand: the compiler tracks the DMA writes of each
  // separately and waits only for the stage being read
  __shared__ __attribute__((aligned(16))) uint8_t a0[kGTileBytes], a1[kGTileBytes],
      b0[kGTileBytes], b1[kGTileBytes];
  uint8_t* const sa_[kGStages] = {a0, a1};
  uint8_t* const sb_[kGStages] = {b0, b1};
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t tile = blockIdx.x;
  const int64_t bm = tile / g.nbn, bn = tile % g.nbn;
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

  // Software pipeline over K stages t (128 bytes each, ring slot t mod 2), each consumed
  // in two sub-steps of 64 bytes.  Sub-step (t, 0): the 16 MFMAs on the fragments of
  // (t, 0) run while those of (t, 1) are read from the same slot.  Sub-step (t, 1): a
  // wave waits for its own DMA of stage t + 1 (the only one in flight) and its LDS reads,
  // and after the barrier (every wave's DMA of stage t + 1 has landed, every wave has
  // finished reading slot t) refills slot t with stage t + 2 and reads (t + 1, 0) while
  // the MFMAs of (t, 1) run.  Stages are rounded up to a multiple of the ring size;
  // stages past K load zeros (and touch no memory).
  const int64_t nk = ((g.K + kGBK - 1) / kGBK + kGStages - 1) / kGStages * kGStages;
  const int frow = lane & 31, fch = 2 * (lane >> 5);
  const int ra0 = wm * 128 + frow, rb0 = wn * 128 + frow;
#pragma unroll
  for (int s = 0; s < kGStages; ++s)
    g_stage_dma((g_lds_t*)sa_[s], (g_lds_t*)sb_[s], ra, rb, g.K, s * kGBK, wave, lane);
  g_v8i af[2][4], bf[2][4];
  G_WAIT_VMCNT(2 * kGDmaPerWave);
  __builtin_amdgcn_s_barrier();
#pragma unroll
  for (int i = 0; i < 4; ++i) af[0][i] = g_frag(sa_[0], ra0 + 32 * i, fch);
#pragma unroll
  for (int j = 0; j < 4; ++j) bf[0][j] = g_frag(sb_[0], rb0 + 32 * j, fch);
  for (int64_t kt = 0; kt < nk; kt += kGStages) {
#pragma unroll
    for (int s = 0; s < kGStages; ++s) {
      // sub-step (t, 0)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 4; ++i) af[1][i] = g_frag(sa_[s], ra0 + 32 * i, fch + 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) bf[1][j] = g_frag(sb_[s], rb0 + 32 * j, fch + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[0][i], bf[0][j],
                                                                     acc[i][j], kFa, kFb, 0, 127,
                                                                     0, 127);
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      // sub-step (t, 1)
      G_WAIT_VMCNT_LGKM0(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      g_stage_dma((g_lds_t*)sa_[s], (g_lds_t*)sb_[s], ra, rb, g.K, (kt + s + kGStages) * kGBK,
                  wave, lane);
      const int s1 = (s + 1) % kGStages;
#pragma unroll
      for (int i = 0; i < 4; ++i) af[0][i] = g_frag(sa_[s1], ra0 + 32 * i, fch);
#pragma unroll
      for (int j = 0; j < 4; ++j) bf[0][j] = g_frag(sb_[s1], rb0 + 32 * j, fch);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[1][i], bf[1][j],
                                                                     acc[i][j], kFa, kFb, 0, 127,
                                                                     0, 127);
      // each MFMA is followed by one fragment read and one DMA issue
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
    }
  }
  // no LDS DMA may still be in flight when the ring is reused or the block exits
  G_WAIT_VMCNT(0);

  // epilogue: C = acc * (sa * sb); accumulator r of a 32 x 32 tile holds row
  // (r mod 4) + 8 (r / 4) + 4 (lane / 32), column lane mod 32
  const float s = uniform(*g.sa) * uniform(*g.sb);
  if constexpr (kBf16Out) {
    if (g.vec_c) {
      // through LDS (the ring is free now): each wave writes its 128 x 128 bf16 tile
      // into one 32 KB object (128 rows of 256 bytes) and stores it back row by row, 16
      // bytes per lane
      __syncthreads();
      uint8_t* const e = wave == 0 ? a0 : wave == 1 ? a1 : wave == 2 ? b0 : b1;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int rl = i * 32 + (r & 3) + 8 * (r >> 2) + 4 * (lane >> 5);
            const int cl = j * 32 + (lane & 31);
            uint8_t* o = e + rl * 256 + 2 * cl;
            *(uint16_t*)o = (uint16_t)(pack_bf16_rne(acc[i][j][r] * s, 0.0f) & 0xFFFFu);
          }
#pragma unroll 4
      for (int c = 0; c < 32; ++c) {
        const int qi = lane + 64 * c;  // 16-byte chunk of the wave tile
        const int rl = qi >> 4, cl = 8 * (qi & 15);
        const uint4 v = *(const uint4*)(e + rl * 256 + 2 * cl);
        const int64_t row = m0 + wm * 128 + rl, col = n0 + wn * 128 + cl;
        if (row < g.M && col < g.N) *(uint4*)((uint16_t*)g.C + row * g.N + col) = v;
      }
      return;
    }
  }
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
  g.vec_c = c_dtype == FP8Q_BF16 && N % 8 == 0 && (uintptr_t)C % 16 == 0;
  g.pad = 0;
  const bool bf16 = c_dtype == FP8Q_BF16;
  const hipStream_t st = (hipStream_t)stream;
  if (a_format == FP8Q_E4M3)
    return b_format == FP8Q_E4M3 ? gemm_launch<0, 0>(g, bf16, st) : gemm_launch<0, 1>(g, bf16, st);
  return b_format == FP8Q_E4M3 ? gemm_launch<1, 0>(g, bf16, st) : gemm_launch<1, 1>(g, bf16, st);
}
