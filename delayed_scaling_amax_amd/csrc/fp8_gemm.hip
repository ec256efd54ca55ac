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
//  * Registers: 256 accumulators in AGPRs, two fragment sets (128 VGPRs); lane-derived
//    offsets are rebuilt per tile so nothing spills.
//  * Epilogue: B is the MFMA's first operand, so each lane holds four consecutive
//    columns of a C row per register quad.  With C 16-byte aligned and N a multiple of
//    8 (bf16) or 4 (fp32), lanes l and l + 32 exchange quads (v_permlane32_swap) so that
//    each holds 8 consecutive bf16 columns, and every lane issues 16-byte buffer stores,
//    the same number per tile whatever the edges (masked elements use an offset past the
//    resource).  Otherwise element stores.
//  * Persistent blocks, twice as many as compute units (one resident per CU at a time),
//    walk the tiles with a stride of the grid size.  The last two ring refills of a tile fetch the next tile's first two stages,
//    so the epilogue's stores overlap those loads.  Tile order: the 32 blocks of one XCD
//    (blocks are dealt to the 8 XCDs in turn) work on one super-tile of 4 x 8 tiles at a
//    time, so per stage they read 4 A and 8 B slices through their shared L2; A and B of
//    the MLP shapes (tens of MB) stay in the 256 MB MALL behind it.
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
#ifndef FP8Q_GEMM_ST_AUX
#define FP8Q_GEMM_ST_AUX 0
#endif
// C store cache policy: the default.  The epilogue writes each 128-byte line of C in
// quarter-line pieces over a few consecutive stores, which merge in L2; non-temporal
// stores bypass that merge and measured 20-25% slower on the MLP shapes.
constexpr int kGStAux = FP8Q_GEMM_ST_AUX;

struct GemmArgs {
  const uint8_t* A;
  const uint8_t* B;
  void* C;
  const float* sa;
  const float* sb;
  int64_t M, N, K;
  uint32_t nbm;     // row tiles
  uint32_t nbn;     // column tiles
  uint32_t ntiles;  // row tiles x column tiles (< 2^31)
  uint32_t pad2;
  int32_t vec_c;   // 16-byte C stores (see fp8_gemm below)
  int32_t pad;
};

typedef int g_v8i __attribute__((ext_vector_type(8)));
typedef uint32_t g_u32x4 __attribute__((ext_vector_type(4)));
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
// (offset 0xFFFFFFF0 is past every resource).
__device__ __forceinline__ void g_stage_dma(g_lds_t* ta, g_lds_t* tb, __amdgpu_buffer_rsrc_t ra,
                                            __amdgpu_buffer_rsrc_t rb, uint32_t K, uint32_t k0,
                                            int wave, int lane) {
  // 32-bit offsets: rows < 256, K <= 2^23, k0 < K + 512
  const uint32_t rl = lane >> 3, rlK = rl * K;
#pragma unroll
  for (int j = 0; j < kGDmaPerWave; ++j) {
    const uint32_t row0 = 8 * (wave * kGDmaPerWave + j);  // wave-uniform
    const uint32_t c = (lane & 7) ^ (((row0 + rl) >> 1) & 7);
    const uint32_t k = k0 + 16 * c;
    const uint32_t voff = k < K ? rlK + row0 * K + k : 0xFFFFFFF0u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (g_lds_t*)((__attribute__((address_space(3))) uint8_t*)ta + 1024 * (row0 / 8)),
                                             16, voff, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (g_lds_t*)((__attribute__((address_space(3))) uint8_t*)tb + 1024 * (row0 / 8)),
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

// Tile order: super-tiles of 4 row tiles x 8 column tiles (smaller at the edges), in
// row-major order, row-major inside.  When the column-tile count is a multiple of 8, the
// 8 columns of super-tile column group G are G, G + S, ..., G + 7 S (S = count / 8)
// rather than 8 G .. 8 G + 7: same L2 sharing, measured 4% faster on the 64-column MLP
// grid.  Linear index L -> tile (bm, bn); a bijection of [0, ntiles) onto the grid.
__device__ __forceinline__ void g_tile_coords(const GemmArgs& g, uint32_t L, uint32_t& bm,
                                              uint32_t& bn) {
  const uint32_t R = L / (4 * g.nbn);
  const uint32_t hR = g.nbm - 4 * R < 4 ? g.nbm - 4 * R : 4;
  const uint32_t Lr = L - R * 4 * g.nbn;
  const uint32_t G = Lr / (hR * 8);
  const uint32_t wG = g.nbn - 8 * G < 8 ? g.nbn - 8 * G : 8;
  const uint32_t loc = Lr - G * hR * 8;
  bm = 4 * R + loc / wG;
  bn = g.nbn % 8 == 0 ? G + (g.nbn / 8) * (loc % 8) : 8 * G + loc % wG;
}

// Buffer resources over the block rows of the tile at linear index L (whole K); an index
// past the grid gives empty resources, whose loads return zeros without touching memory.
__device__ __forceinline__ void g_tile_rsrc(const GemmArgs& g, uint32_t L,
                                            __amdgpu_buffer_rsrc_t& ra,
                                            __amdgpu_buffer_rsrc_t& rb) {
  const bool live = L < g.ntiles;
  uint32_t bm = 0, bn = 0;
  if (live) g_tile_coords(g, L, bm, bn);
  const int64_t m0 = (int64_t)bm * kGBM, n0 = (int64_t)bn * kGBN;
  const int64_t rows_a = live ? (g.M - m0 < kGBM ? g.M - m0 : kGBM) : 0;
  const int64_t rows_b = live ? (g.N - n0 < kGBN ? g.N - n0 : kGBN) : 0;
  ra = g_rsrc(g.A + m0 * g.K, (uint32_t)(rows_a * g.K));
  rb = g_rsrc(g.B + n0 * g.K, (uint32_t)(rows_b * g.K));
}

template <int kFa, int kFb, bool kBf16Out>
__global__ __launch_bounds__(kGThreads) void fp8_gemm_kernel(const GemmArgs g) {
  // one LDS object per stage and operand: the compiler tracks the DMA writes of each
  // separately
  __shared__ __attribute__((aligned(16))) uint8_t a0[kGTileBytes], a1[kGTileBytes],
      b0[kGTileBytes], b1[kGTileBytes];
  uint8_t* const sa_[kGStages] = {a0, a1};
  uint8_t* const sb_[kGStages] = {b0, b1};
  const int tid = threadIdx.x;
  const int lane0 = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const float s = uniform(*g.sa) * uniform(*g.sb);

  // Persistent blocks: block b computes tiles b, b + G, b + 2G, ... (G = grid size), in
  // row-major order over the tile grid.  Per tile, K is consumed in stages t of 128
  // bytes (ring slot t mod 2), each in two sub-steps of 64 bytes.  Sub-step (t, 0): the
  // 16 MFMAs on the fragments of (t, 0) run while those of (t, 1) are read from the same
  // slot.  Sub-step (t, 1): a wave waits for its own DMA of stage t + 1 (the only one in
  // flight) and its LDS reads; after the barrier (every wave's DMA of stage t + 1 has
  // landed, every wave has finished reading slot t) it refills slot t with stage t + 2,
  // or, for the last two stages, with stage 0 or 1 of its next tile, and reads (t + 1, 0)
  // while the MFMAs of (t, 1) run.  So a tile's epilogue overlaps the loads of the next.
  // Stages are rounded up to a multiple of the ring size; stages past K load zeros (and
  // touch no memory).
  const int64_t nk0 = ((g.K + kGBK - 1) / kGBK + kGStages - 1) / kGStages * kGStages;
  const int64_t nk = nk0 > kGStages ? nk0 : kGStages;  // at least one round (K = 0 too)
  // Block b takes linear indices L = w G + pos(b), w = 0, 1, ... (G = grid size).  Blocks
  // are dealt to the 8 XCDs in turn, so pos gives the G / 8 blocks of one XCD consecutive
  // indices: one super-tile per XCD per wave of G tiles.
  const uint32_t gsz = gridDim.x;
  const uint32_t pos = gsz % 8 == 0 ? (blockIdx.x % 8) * (gsz / 8) + blockIdx.x / 8 : blockIdx.x;
  uint32_t tile = pos;  // linear index, wave-uniform throughout
  __amdgpu_buffer_rsrc_t ra, rb, rna, rnb;
  g_tile_rsrc(g, tile, ra, rb);
#pragma unroll
  for (int st = 0; st < kGStages; ++st)
    g_stage_dma((g_lds_t*)sa_[st], (g_lds_t*)sb_[st], ra, rb, (uint32_t)g.K, st * kGBK, wave,
                lane0);
  g_v8i af[2][4], bf[2][4];
  G_WAIT_VMCNT(2 * kGDmaPerWave);  // stage 0 (stage 1 stays in flight)
  __builtin_amdgcn_s_barrier();
#pragma unroll
  for (int i = 0; i < 4; ++i) af[0][i] = g_frag(sa_[0], wm * 128 + (lane0 & 31) + 32 * i, 2 * (lane0 >> 5));
#pragma unroll
  for (int j = 0; j < 4; ++j) bf[0][j] = g_frag(sb_[0], wn * 128 + (lane0 & 31) + 32 * j, 2 * (lane0 >> 5));

  while (tile < g.ntiles) {
    // Lane-derived offsets are rebuilt per tile from an opaque copy of the lane index:
    // hoisted to the kernel start they would stay live across the whole tile loop and
    // spill (each reload then waits for every memory op in flight).
    int lane = lane0;
    asm volatile("" : "+v"(lane));
    const int frow = lane & 31, fch = 2 * (lane >> 5);
    const int ra0 = wm * 128 + frow, rb0 = wn * 128 + frow;
    const uint32_t next = __builtin_amdgcn_readfirstlane(tile + gridDim.x);
    g_tile_rsrc(g, next, rna, rnb);
    g_v16f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = g_v16f{};
    // One round = kGStages stages.  The first round of a tile is peeled off the loop: the
    // same code, but the register allocation of the peeled form measured free of spills
    // (the plain loop spilled ~100 VGPRs).
    auto round = [&](int64_t kt) {
      // refills of this round: stages kt + 2, kt + 3 of this tile, or the next tile's
      // first two stages when this is the tile's last round
      const bool last = kt + kGStages >= nk;
      const __amdgpu_buffer_rsrc_t qa = last ? rna : ra, qb = last ? rnb : rb;
      const int64_t qk = last ? 0 : (kt + kGStages) * kGBK;
#pragma unroll
      for (int st = 0; st < kGStages; ++st) {
        // sub-step (t, 0)
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < 4; ++i) af[1][i] = g_frag(sa_[st], ra0 + 32 * i, fch + 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) bf[1][j] = g_frag(sb_[st], rb0 + 32 * j, fch + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                bf[0][j], af[0][i], acc[i][j], kFb, kFa, 0, 127, 0, 127);
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        // sub-step (t, 1).  A full drain: with loads and the previous tile's epilogue
        // stores both outstanding, vmcnt is not guaranteed to drain in issue order, and
        // the barrier below publishes this wave's DMA of stage t + 1 to the others.
        G_WAIT_VMCNT_LGKM0(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        g_stage_dma((g_lds_t*)sa_[st], (g_lds_t*)sb_[st], qa, qb, (uint32_t)g.K,
                    (uint32_t)(qk + st * kGBK), wave, lane);
        const int s1 = (st + 1) % kGStages;
#pragma unroll
        for (int i = 0; i < 4; ++i) af[0][i] = g_frag(sa_[s1], ra0 + 32 * i, fch);
#pragma unroll
        for (int j = 0; j < 4; ++j) bf[0][j] = g_frag(sb_[s1], rb0 + 32 * j, fch);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                bf[1][j], af[1][i], acc[i][j], kFb, kFa, 0, 127, 0, 127);
        // each MFMA is followed by one fragment read and one DMA issue
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
      }
    };
    round(0);
    for (int64_t kt = kGStages; kt < nk; kt += kGStages) round(kt);

    // epilogue: C = acc * (sa * sb).  With B as the MFMA's first operand, accumulator r
    // of the 32 x 32 tile (i, j) holds C row i * 32 + lane mod 32, column
    // j * 32 + (r mod 4) + 8 (r / 4) + 4 h (h = lane / 32): register quad q holds four
    // consecutive columns 8 q + 4 h.
    uint32_t tbm, tbn;
    g_tile_coords(g, tile, tbm, tbn);
    const int64_t m0 = (int64_t)tbm * kGBM, n0 = (int64_t)tbn * kGBN;
    if (g.vec_c) {
      // Buffer stores through a resource over C from (m0, n0) on; masked elements use an
      // offset past it (dropped by the hardware).
      constexpr int kElt = kBf16Out ? 2 : 4;
      const int64_t rem = ((g.M - m0) * g.N - n0) * kElt;
      const __amdgpu_buffer_rsrc_t rc =
          g_rsrc((uint8_t*)g.C + (m0 * g.N + n0) * kElt,
                 (uint32_t)(rem < 0x7FFFFFF0 ? rem : 0x7FFFFFF0));
      const int h = lane >> 5;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rl = wm * 128 + i * 32 + (lane & 31);
        const bool row_ok = m0 + rl < g.M;
        const uint32_t rbase = (uint32_t)(rl * g.N) * kElt;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // one 32 x 32 tile at a time: keeps the accumulator reads from being hoisted
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (kBf16Out) {
            // quads 2 p and 2 p + 1 of the lane pair (l, l + 32) are exchanged so that
            // lane l holds columns 16 p .. + 7 and lane l + 32 columns 16 p + 8 .. + 15
#pragma unroll
            for (int p = 0; p < 2; ++p) {
              const uint32_t x0 = pack_bf16_rne(acc[i][j][8 * p] * s, acc[i][j][8 * p + 1] * s);
              const uint32_t x1 = pack_bf16_rne(acc[i][j][8 * p + 2] * s, acc[i][j][8 * p + 3] * s);
              const uint32_t y0 = pack_bf16_rne(acc[i][j][8 * p + 4] * s, acc[i][j][8 * p + 5] * s);
              const uint32_t y1 = pack_bf16_rne(acc[i][j][8 * p + 6] * s, acc[i][j][8 * p + 7] * s);
              const auto w0 = __builtin_amdgcn_permlane32_swap(x0, y0, false, false);
              const auto w1 = __builtin_amdgcn_permlane32_swap(x1, y1, false, false);
              const int cl = wn * 128 + j * 32 + 16 * p + 8 * h;
              const bool ok = row_ok && n0 + cl < g.N;
              const uint32_t voff = ok ? rbase + (uint32_t)cl * 2 : 0x80000000u;
              __builtin_amdgcn_raw_buffer_store_b128(
                  g_u32x4{(uint32_t)w0[0], (uint32_t)w1[0], (uint32_t)w0[1], (uint32_t)w1[1]}, rc,
                  voff, 0, kGStAux);
            }
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int cl = wn * 128 + j * 32 + 8 * q + 4 * h;
              const bool ok = row_ok && n0 + cl < g.N;
              const uint32_t voff = ok ? rbase + (uint32_t)cl * 4 : 0x80000000u;
              __builtin_amdgcn_raw_buffer_store_b128(
                  g_u32x4{__float_as_uint(acc[i][j][4 * q] * s),
                        __float_as_uint(acc[i][j][4 * q + 1] * s),
                        __float_as_uint(acc[i][j][4 * q + 2] * s),
                        __float_as_uint(acc[i][j][4 * q + 3] * s)},
                  rc, voff, 0, kGStAux);
            }
          }
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t row = m0 + wm * 128 + i * 32 + (lane & 31);
        if (row < g.M) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int64_t col = n0 + wn * 128 + j * 32 + 8 * q + 4 * (lane >> 5);
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (col + e < g.N) {
                  const float v = acc[i][j][4 * q + e] * s;
                  if constexpr (kBf16Out)
                    ((uint16_t*)g.C)[row * g.N + col + e] =
                        (uint16_t)(pack_bf16_rne(v, 0.0f) & 0xFFFFu);
                  else
                    ((float*)g.C)[row * g.N + col + e] = v;
                }
            }
        }
      }
    }
    tile = next;
    ra = rna;
    rb = rnb;
  }
  // no LDS DMA may still be in flight when the block exits
  G_WAIT_VMCNT(0);
}

template <int kFa, int kFb>
static int gemm_launch(const GemmArgs& g, bool bf16_out, hipStream_t stream) {
  const void* fn = bf16_out ? (const void*)fp8_gemm_kernel<kFa, kFb, true>
                            : (const void*)fp8_gemm_kernel<kFa, kFb, false>;
  int cus = 0;
  const int rc = current_device_cus(&cus);
  if (rc != FP8Q_OK) return rc;
  // Persistent blocks, twice as many as compute units: the 128 KB ring and 512 registers
  // per lane let one block reside per CU, and the second half of the grid starts on each
  // CU as the first half finishes.  Measured against one block per CU (medians of 5 x 10
  // launches, interleaved): 8192 x 16384 x 4096 440 -> 402 us, 8192 x 49152 x 12288
  // 3959 -> 3844 us, no change on 8192 x 4096 x 16384 and 4096^3; four per CU 456 us and
  // one tile per block 517 us on the first.
  const int64_t want = 2 * (int64_t)cus;
  const int64_t blocks = (int64_t)g.ntiles < want ? (int64_t)g.ntiles : want;
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
  g.nbm = (uint32_t)nbm;
  g.nbn = (uint32_t)nbn;
  g.ntiles = (uint32_t)(nbm * nbn);
  g.pad2 = 0;
  // vector path: 16-byte stores of 8 bf16 / 4 fp32 columns, tile offsets within 2^31
  const int64_t elt = c_dtype == FP8Q_BF16 ? 2 : 4;
  g.vec_c = N % (16 / elt) == 0 && (uintptr_t)C % 16 == 0 && kGBM * N * elt < ((int64_t)1 << 31);
  g.pad = 0;
  const bool bf16 = c_dtype == FP8Q_BF16;
  const hipStream_t st = (hipStream_t)stream;
  if (a_format == FP8Q_E4M3)
    return b_format == FP8Q_E4M3 ? gemm_launch<0, 0>(g, bf16, st) : gemm_launch<0, 1>(g, bf16, st);
  return b_format == FP8Q_E4M3 ? gemm_launch<1, 0>(g, bf16, st) : gemm_launch<1, 1>(g, bf16, st);
}
