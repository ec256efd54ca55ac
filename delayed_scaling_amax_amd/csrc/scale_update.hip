// scale_update.hip -- batched delayed-scaling update of n tensors in one launch.
//
// What it computes ("Implement fused kernel for FP8 scale update", TransformerEngine
// PR 593: the history roll, the amax selection and the scale computation fused into
// one in-place kernel; "User Guide on Native XLA-FP8", section "JAX": scale =
// amax / FP8_MAX; "Gradient accumulation of FP8 params": FP8 meta combines with max):
//   hist[h][t] <- hist[h-1][t] (h = H-1..1, oldest row dropped), hist[0][t] <- amax[t]
//   sel = max_h hist[h][t] by bit pattern (or amax[t] for most-recent)
//   scale[t] = RN32(sel / FP8_MAX) * 2^margin if that is finite and > 0, else kept
//   scale_inv[t] = RN32(1 / scale[t]);  amax[t] = 0 if reset_amax
//
// Layout and schedule.  hist is [H][n] row-major.  A block owns kUCols adjacent tensors
// (columns, a 64-byte row segment, read as float4s by kUCols/4 threads) and all H rows,
// so the in-place roll never races with another block: each thread loads its rows
// into registers, a barrier separates every load of a chunk from every store, and
// the stores go one row down.  Chunks of rows run from the oldest row upward, so
// a chunk's stores only overwrite rows that were already loaded.  The per-tensor
// inputs (amax, scale, format) are fetched at kernel start, alongside the history,
// so the update costs one memory round trip.  Blocks with the same blockIdx % 8 land
// on the same XCD; they get adjacent column groups so the lines they share stay in
// one L2.
#include "device_common.h"
#include "host_common.h"

namespace fp8q {

#ifndef FP8Q_U_BLOCK
#define FP8Q_U_BLOCK 512
#endif
#ifndef FP8Q_U_COLS
#define FP8Q_U_COLS 8
#endif
#ifndef FP8Q_U_ROWS
#define FP8Q_U_ROWS 2
#endif
#ifndef FP8Q_U_XCD
#define FP8Q_U_XCD 1
#endif
// Cache policy of the history stores (buffer-op aux bits: 16 = sc1, device scope).
#ifndef FP8Q_U_ST_AUX
#define FP8Q_U_ST_AUX 0
#endif
constexpr int kUBlock = FP8Q_U_BLOCK;
constexpr int kUCols = FP8Q_U_COLS;            // tensors (history columns) per block
constexpr int kUTpr = kUCols / 4;              // threads per history row, 4 columns each
constexpr int kURowsPerPass = kUBlock / kUTpr;
constexpr int kURowsPerThread = FP8Q_U_ROWS;
constexpr int kUChunk = kURowsPerPass * kURowsPerThread;  // history rows per chunk
static_assert(kUCols % 4 == 0 && 64 % kUTpr == 0, "column group must split into float4s");

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Columns c0+4*lc .. c0+4*lc+3 of one history row.  kVec: n % 4 == 0 and the history
// is 16-byte aligned, so the 4 columns are one aligned float4 present in full or not
// at all; otherwise each column is checked against ncols.
template <bool kVec>
__device__ __forceinline__ void load_row(const float* __restrict__ row, int c, int ncols,
                                         uint32_t (&v)[4]) {
  if constexpr (kVec) {
    if (c < ncols) {
      const u32x4 q = *(const u32x4*)row;
      v[0] = q[0]; v[1] = q[1]; v[2] = q[2]; v[3] = q[3];
    } else {
      v[0] = v[1] = v[2] = v[3] = 0u;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = c + j < ncols ? as_uint(row[j]) : 0u;
  }
}

// kVec stores go through a buffer resource over the whole history (the launcher
// picks this form only when the history spans < 2^31 bytes) with the store policy.
template <bool kVec>
__device__ __forceinline__ void store_row(float* __restrict__ row, __amdgpu_buffer_rsrc_t rh,
                                          uint32_t off, int c, int ncols,
                                          const uint32_t (&v)[4]) {
  if constexpr (kVec) {
    if (c < ncols)
      __builtin_amdgcn_raw_buffer_store_b128(u32x4{v[0], v[1], v[2], v[3]}, rh, off, 0,
                                             FP8Q_U_ST_AUX);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (c + j < ncols) row[j] = as_float(v[j]);
  }
}

template <bool kVec>
__global__ __launch_bounds__(kUBlock) void amax_and_scale_update_kernel(
    float* __restrict__ amax, float* __restrict__ hist, float* __restrict__ scale,
    float* __restrict__ scale_inv, const uint8_t* __restrict__ formats, int64_t n, int64_t H,
    int algo, int margin, int reset_amax, int64_t groups, int64_t groups_per_xcd) {
  __shared__ uint32_t red[kUBlock / 64][kUCols];
#if FP8Q_U_XCD
  const int64_t g = (int64_t)(blockIdx.x % 8) * groups_per_xcd + blockIdx.x / 8;
#else
  const int64_t g = blockIdx.x;
#endif
  if (g >= groups) return;  // whole block, before any barrier
  const int64_t c0 = g * kUCols;
  const int ncols = (int)min((int64_t)kUCols, n - c0);
  const int tid = threadIdx.x;
  const int lc = tid % kUTpr;       // which 4 columns of the group
  const int rr = tid / kUTpr;       // row within a pass
  const int cl = 4 * lc;            // first column (local) of this thread

  // per-tensor inputs, fetched now so their latency overlaps the history loads (every
  // lane loads, lanes past ncols the group's first tensor, so no merge waits for them)
  const int64_t ct = c0 + (tid < ncols ? tid : 0);
  const float a_in = amax[ct];
  const float s_old = scale[ct];
  uint32_t fmt = formats[ct];

  const __amdgpu_buffer_rsrc_t rh = __builtin_amdgcn_make_buffer_rsrc(
      hist, (short)0, (int)(kVec ? H * n * 4 : 0), 0x00020000);
  uint32_t m[4] = {0u, 0u, 0u, 0u};
  // destination rows d in [1, H) take source row d-1; oldest chunk first
  for (int64_t d_hi = H; d_hi > 1; d_hi -= kUChunk) {
    const int64_t d_lo = d_hi - kUChunk > 1 ? d_hi - kUChunk : 1;
    uint32_t v[kURowsPerThread][4];
#pragma unroll
    for (int k = 0; k < kURowsPerThread; ++k) {
      const int64_t d = d_lo + rr + (int64_t)k * kURowsPerPass;
      if (d < d_hi) load_row<kVec>(hist + (d - 1) * n + c0 + cl, cl, ncols, v[k]);
    }
#pragma unroll
    for (int k = 0; k < kURowsPerThread; ++k) {
      const int64_t d = d_lo + rr + (int64_t)k * kURowsPerPass;
      if (d < d_hi)
#pragma unroll
        for (int j = 0; j < 4; ++j) m[j] = m[j] > v[k][j] ? m[j] : v[k][j];
    }
    __syncthreads();  // every load of this chunk (values already in registers) ...
#pragma unroll
    for (int k = 0; k < kURowsPerThread; ++k) {  // ... before any store one row down
      const int64_t d = d_lo + rr + (int64_t)k * kURowsPerPass;
      if (d < d_hi)
        store_row<kVec>(hist + d * n + c0 + cl, rh, (uint32_t)((d * n + c0 + cl) * 4), cl, ncols,
                        v[k]);
    }
  }

  // block max per column over the rolled window (row 0 = the new amax, added below):
  // lanes with the same lc hold the same columns
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t w = m[j];
#pragma unroll
    for (int off = 32; off >= kUTpr; off >>= 1) {
      const uint32_t o = __shfl_xor(w, off, 64);
      w = w > o ? w : o;
    }
    if ((tid & 63) < kUTpr) red[tid >> 6][cl + j] = w;
  }
  __syncthreads();
  if (tid < ncols) {
    const int64_t t = c0 + tid;
    const uint32_t ab = as_uint(a_in);
    uint32_t sel_bits = ab;
#pragma unroll
    for (int w = 0; w < kUBlock / 64; ++w) sel_bits = sel_bits > red[w][tid] ? sel_bits : red[w][tid];
    hist[t] = a_in;  // row 0; row 0 was loaded (as source of row 1) before the last barrier
    if (algo == FP8Q_AMAX_MOST_RECENT) sel_bits = ab;
    // opaque rebind (no instruction): without it the compiler tests fmt right after its
    // load, which makes every history load wait for that load first
    asm volatile("" : "+v"(fmt));
    const float s = next_scale(sel_bits, fmt, s_old, margin);
    scale[t] = s;
    scale_inv[t] = 1.0f / s;
    if (reset_amax) amax[t] = 0.0f;
  }
}

}  // namespace fp8q

using namespace fp8q;

extern "C" int fp8_amax_and_scale_update(float* amax, float* amax_history, float* scale,
                                         float* scale_inv, const uint8_t* formats, int64_t n,
                                         int64_t history_len, int algo, int margin,
                                         int reset_amax, void* stream) {
  const int st = validate_update(amax, amax_history, scale, scale_inv, formats, n, history_len,
                                 algo, margin);
  if (st != FP8Q_OK || n == 0) return st;
  const int64_t groups = ceil_div(n, kUCols);
  const int64_t per_xcd = ceil_div(groups, 8);
  const int64_t blocks = 8 * per_xcd;
  if (blocks > 0x7FFFFFFF) return FP8Q_EINVAL;
  const bool vec = (n % 4 == 0) && ((uintptr_t)amax_history % 16 == 0) &&
                   history_len * n < ((int64_t)1 << 29);  // buffer offsets stay < 2^31
  int rm = reset_amax ? 1 : 0;
  void* args[] = {&amax, &amax_history, &scale, &scale_inv, (void*)&formats, &n, &history_len,
                  &algo, &margin, &rm, (void*)&groups, (void*)&per_xcd};
  const void* fn = vec ? (const void*)amax_and_scale_update_kernel<true>
                       : (const void*)amax_and_scale_update_kernel<false>;
  return launch_status(hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(kUBlock), args, 0,
                                       (hipStream_t)stream));
}
