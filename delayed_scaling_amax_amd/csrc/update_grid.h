// update_grid.h -- launch geometry of the batched scale update (amax_and_scale_update_kernel).
// Kept in one place so that the floor measurements taken beside the kernel run on exactly
// its grid.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8q {

// Threads per block, tensors (history columns) per block, and history rows per thread
// per round trip.  The roll moves the whole history through the CUs' load and store paths,
// so a block takes 32 adjacent tensors -- a whole 128-byte line of every row, read by 8
// lanes as 16-byte pieces -- and all rows: measured against 4, 8 and 16 columns (16-, 32-
// and 64-byte pieces of a line per block, on more CUs) on 1152 tensors x 1024 rows, one
// load -> barrier -> store round trip of the history takes 3.6 us against 5.5, 3.9 and
// 3.9 us.  1024 threads x 8 rows cover 1024 destination rows, so a history of up to 1025
// rows rolls in one round trip.
#ifndef FP8Q_U_BLOCK
#define FP8Q_U_BLOCK 1024
#endif
#ifndef FP8Q_U_COLS
#define FP8Q_U_COLS 32
#endif
#ifndef FP8Q_U_ROWS
#define FP8Q_U_ROWS 8
#endif
#ifndef FP8Q_U_XCD
#define FP8Q_U_XCD 1
#endif
constexpr int kUBlock = FP8Q_U_BLOCK;
constexpr int kUCols = FP8Q_U_COLS;
constexpr int kURows = FP8Q_U_ROWS;
static_assert(kUCols % 4 == 0 && kUCols <= 32 && (kUCols & (kUCols - 1)) == 0 &&
                  kUBlock % 64 == 0,
              "a row of the block's columns splits into whole 16-byte accesses of <= 32 lanes");
// History elements a launch may address (32-bit buffer offsets, kept below 2^31 bytes).
constexpr int64_t kUpdateMaxElems = (int64_t)1 << 29;

// Lanes per history row: enough lanes of W columns each for the block's columns (at most
// kUCols, fewer when n is smaller), rounded up to a power of two (the lane-class max
// reduces over power-of-two classes).
inline int update_tpr(int64_t n, int W) {
  const int64_t cols = n < kUCols ? n : kUCols;
  const int64_t lanes = (cols + W - 1) / W;
  int t = 1;
  while (t < lanes) t *= 2;
  return t;
}

struct UpdateGrid {
  int64_t groups;          // column groups of kUCols tensors
  int64_t groups_per_xcd;  // consecutive groups given to one XCD
  int64_t blocks;          // 8 * groups_per_xcd (blocks past `groups` exit at once)
};

inline UpdateGrid update_grid(int64_t n) {
  UpdateGrid g;
  g.groups = (n + kUCols - 1) / kUCols;
  g.groups_per_xcd = (g.groups + 7) / 8;
  g.blocks = 8 * g.groups_per_xcd;
  return g;
}

// Column group of block b.  Workgroups are dispatched to the 8 XCDs round-robin, so the
// blocks with the same b % 8 share an L2: they get consecutive column groups.
__device__ __forceinline__ int64_t update_group(unsigned b, int64_t groups_per_xcd) {
#if FP8Q_U_XCD
  return (int64_t)(b % 8) * groups_per_xcd + b / 8;
#else
  (void)groups_per_xcd;
  return b;
#endif
}

}  // namespace fp8q
