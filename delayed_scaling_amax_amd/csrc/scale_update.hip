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
// (columns) and all H rows, so the in-place roll never races with another block.  The
// work is latency-bound (4.7 MB of history for 1152 tensors x 1024 rows), so the
// schedule is built around one memory round trip: every thread issues the loads of all
// its history rows (up to kURows each, one row of the block's columns per load) before
// the block's single barrier, then stores them one row down.  The loads and stores are
// buffer operations whose range check does the masking: the load descriptor ends at
// row H-1 (the dropped oldest row reads as 0, the identity of the unsigned max), the
// store descriptor at row H, and a lane without a row (past the chunk or past the last
// column) uses an offset beyond both, so nothing is branched on and the compiler places
// one wait for all loads.  Histories too deep for one round trip run in chunks of rows
// from the oldest upward, so a chunk only overwrites rows already loaded.  The
// per-tensor inputs (amax, scale, format) are loaded at kernel start, alongside the
// history.  Blocks with the same blockIdx % 8 land on the same XCD; they get adjacent
// column groups, so the cache lines they share stay in one L2.
#include "device_common.h"
#include "host_common.h"
#include "update_grid.h"

namespace fp8q {

// Cache policy of the history stores (buffer-op aux bits: 16 = sc1, device scope).
#ifndef FP8Q_U_ST_AUX
#define FP8Q_U_ST_AUX 0
#endif

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// An offset no history buffer reaches (every real offset is below 2^31): a buffer
// access there is out of range -- a load returns 0, a store is dropped.
constexpr uint32_t kUOff = 0x80000000u;

template <int W>
__device__ __forceinline__ void hist_load(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                          uint32_t (&v)[W]) {
  if constexpr (W == 4) {
    const u32x4 q = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    v[0] = q[0]; v[1] = q[1]; v[2] = q[2]; v[3] = q[3];
  } else {
    v[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
  }
}

template <int W>
__device__ __forceinline__ void hist_store(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                           const uint32_t (&v)[W]) {
  if constexpr (W == 4)
    __builtin_amdgcn_raw_buffer_store_b128(u32x4{v[0], v[1], v[2], v[3]}, r, off, 0,
                                           FP8Q_U_ST_AUX);
  else
    __builtin_amdgcn_raw_buffer_store_b32(v[0], r, off, 0, FP8Q_U_ST_AUX);
}

// W = 4: a lane takes 4 adjacent columns of a row as one 16-byte access (n % 4 == 0 and
// the history 16-byte aligned); W = 1: one column per lane.  tpr lanes cover a row of the
// block's columns (a power of two, update_tpr), kUBlock / tpr rows per pass.
template <int W>
__global__ __launch_bounds__(kUBlock) void amax_and_scale_update_kernel(
    float* __restrict__ amax, float* __restrict__ hist, float* __restrict__ scale,
    float* __restrict__ scale_inv, const uint8_t* __restrict__ formats, int64_t n, int64_t H,
    int algo, int margin, int reset_amax, int64_t groups, int64_t groups_per_xcd, int tpr) {
  __shared__ uint32_t red[kUBlock / 64][kUCols];
  const int64_t g = update_group(blockIdx.x, groups_per_xcd);
  if (g >= groups) return;  // whole block, before any barrier
  const int64_t c0 = g * kUCols;
  const int tid = threadIdx.x;
  const int lc = tid & (tpr - 1);  // which W columns of the group
  const int rr = tid / tpr;        // row within a pass
  const int rpp = kUBlock / tpr;   // rows per pass
  const int64_t chunk = (int64_t)rpp * kURows;  // destination rows per round trip
  const int64_t c = c0 + (int64_t)lc * W;
  const bool col_ok = c < n;  // W == 4: whole groups of 4 (n % 4 == 0)

  // per-tensor inputs: loaded right after the first chunk's history loads (below), so
  // their latency overlaps the history's without the history values waiting behind them
  // (loads complete in issue order for the wait counter); every lane loads, lanes past the
  // group's columns its first tensor, so no merge waits
  const int ncols = (int)min((int64_t)kUCols, n - c0);
  const int64_t ct = c0 + (tid < ncols ? tid : 0);
  float a_in = 0.0f, s_old = 0.0f;
  uint32_t fmt = 0;
  bool have_inputs = false;

  // loads see rows [0, H-1) (the oldest row is dropped by the roll), stores rows [0, H)
  const uint32_t row_bytes = (uint32_t)(n * 4);
  const __amdgpu_buffer_rsrc_t rld =
      __builtin_amdgcn_make_buffer_rsrc(hist, (short)0, (int)((H - 1) * n * 4), 0x00020000);
  const __amdgpu_buffer_rsrc_t rst =
      __builtin_amdgcn_make_buffer_rsrc(hist, (short)0, (int)(H * n * 4), 0x00020000);
  const uint32_t col_off = (uint32_t)(c * 4);
  uint32_t m[W];
#pragma unroll
  for (int j = 0; j < W; ++j) m[j] = 0u;
  // destination rows d in [1, H) take source row d - 1, a chunk of rows per round trip,
  // the oldest chunk first; the last (newest) chunk also reduces the column maxima
  // before its barrier, so the new scales are stored along with its rows.  (H == 1: one
  // pass with no rows.)
  for (int64_t d_hi = H;;) {
    const int64_t d_lo = d_hi - chunk > 1 ? d_hi - chunk : 1;
    uint32_t v[kURows][W];
    uint32_t off[kURows];  // offset of the source row; the destination is one row down
#pragma unroll
    for (int k = 0; k < kURows; ++k) {
      const int64_t d = d_lo + rr + (int64_t)k * rpp;
      off[k] = col_ok && d < d_hi ? (uint32_t)(d - 1) * row_bytes + col_off : kUOff;
      hist_load<W>(rld, off[k], v[k]);
    }
    if (!have_inputs) {  // uniform: the first chunk
      a_in = amax[ct];
      s_old = scale[ct];
      fmt = formats[ct];
      have_inputs = true;
    }
#pragma unroll
    for (int k = 0; k < kURows; ++k)
#pragma unroll
      for (int j = 0; j < W; ++j) m[j] = m[j] > v[k][j] ? m[j] : v[k][j];
    const bool last = d_lo == 1;  // uniform
    if (last) {
      // column maxima over the rolled window but its row 0 (the new amax, added below):
      // the lanes of one class (same lc) hold the same columns
#pragma unroll
      for (int j = 0; j < W; ++j) m[j] = lane_class_max(m[j], tpr);
      if ((tid & 63) < tpr)
#pragma unroll
        for (int j = 0; j < W; ++j) red[tid >> 6][lc * W + j] = m[j];
    }
    __syncthreads();  // every load of this chunk (values in registers) before any store
#pragma unroll
    for (int k = 0; k < kURows; ++k) hist_store<W>(rst, off[k] + row_bytes, v[k]);
    if (last) break;
    d_hi = d_lo;
  }

  if (tid < ncols) {
    const int64_t t = c0 + tid;
    const uint32_t ab = as_uint(a_in);
    uint32_t sel_bits = ab;
#pragma unroll
    for (int w = 0; w < kUBlock / 64; ++w) sel_bits = sel_bits > red[w][tid] ? sel_bits : red[w][tid];
    hist[t] = a_in;  // row 0; it was loaded (as the source of row 1) before the barrier
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
  if (st != FP8Q_OK || n == 0) return st;  // (histories of 2^29 elements or more refused)
  const UpdateGrid grid = update_grid(n);
  if (grid.blocks > 0x7FFFFFFF) return FP8Q_EINVAL;
  const bool vec = (n % 4 == 0) && ((uintptr_t)amax_history % 16 == 0);
  int rm = reset_amax ? 1 : 0;
  int64_t groups = grid.groups, per_xcd = grid.groups_per_xcd;
  int tpr = update_tpr(n, vec ? 4 : 1);
  void* args[] = {&amax, &amax_history, &scale, &scale_inv, (void*)&formats, &n, &history_len,
                  &algo, &margin, &rm, (void*)&groups, (void*)&per_xcd, &tpr};
  const void* fn = vec ? (const void*)amax_and_scale_update_kernel<4>
                       : (const void*)amax_and_scale_update_kernel<1>;
  return launch_status(hipLaunchKernel(fn, dim3((unsigned)grid.blocks), dim3(kUBlock), args, 0,
                                       (hipStream_t)stream));
}
