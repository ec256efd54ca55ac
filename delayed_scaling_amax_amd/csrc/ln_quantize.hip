// ln_quantize.hip -- LayerNorm output -> FP8 quantize + amax, the LayerNorm applied in
// registers so its bf16 output is never written.
//
// What it computes: the transformer block of the reproducer in "Fusion of Fp8
// quantization and amax reduction kernels" (test.py: BasicTransformer applies Flax
// nn.LayerNorm() and feeds the result to the MLP's first dense, whose FP8 dot
// quantizes it).  Per row of length H:
//   mu = mean(x), V = mean((x - mu)^2), rstd = 1 / sqrt(V + eps),
//   y = RN_bf16(gamma * (x - mu) * rstd + beta),
// then code = FP8(saturate(RN32(y / scale))) and amax = max(amax, max|y|) exactly as
// the plain quantize does ("User Guide on Native XLA-FP8", section "JAX").
//
// Design (gfx950; HBM-bound at 3 bytes/element plus 8 bytes per row of statistics):
//  * One wavefront per row, persistent grid: the row (H <= 16384 bf16 = 32 KB) is
//    loaded as 16-byte units into registers -- the wavefront's next row is loaded
//    while the current one is reduced and written -- so every reduction is a
//    wavefront butterfly, with no LDS round trip and no block barrier per row.
//  * gamma and beta are staged once per block into LDS (zero-padded to the unit
//    grid), read back per element.
//  * Statistics in binary32 with tree sums (depth log2(8 kV) per lane, the squares of
//    rows over 512 long 8 + log2(kV), + 6 across the wavefront, the latter on the DPP
//    network; at most ceil(log2 H) + 6 in all) and a corrected second pass:
//    mu' = RN(S/H); d' = RN(x - mu');
//    e' = sum(d')/H and V' = sum(d'^2)/H - e'^2 remove the first mean's rounding
//    error from both the deviations and the variance (rows whose mean is large
//    against their spread lose no accuracy); y' = RN(fma(d' - e', RN(gamma rstd'),
//    beta)).
//  * Rows with inf/NaN inputs (or V + eps = 0) produce NaN, written as the positive
//    default NaN 0x7FC0; its code is 0x7F.
//  * The quantize of y' is the shared element math (corrected division by the scale,
//    saturate, native OCP convert, fixed codes for huge quotients).  The amax goes
//    lane max -> wavefront -> LDS -> one global atomic per block.  Rows that give no
//    NaN take the lane max as a float max3 of |y|; other rows take the packed bf16
//    magnitude max.
#include "device_common.h"
#include "host_common.h"
#include "quant_math.h"
#include "fp8q.h"

namespace fp8q {

constexpr int kLBlock = 256;       // 4 wavefronts, one row each at a time
// Rows of 24 or 32 units per lane (hidden 8200-16384) are split over kSplit wavefronts
// (4: 6 or 8 units each): a row's sums are combined through LDS, and the smaller register
// need lets more wavefronts share one block's 96 or 128 KB of gamma/beta (24 units on one
// wavefront took 232-240 registers, 32 units more than 256; 8 units take 106-111).
template <int kV, int kSplit>
constexpr int ln_block() { return kSplit == 1 ? kLBlock : (kV * kSplit == 32 && kSplit == 2 ? 512 : 1024); }
template <int kV, int kSplit>
constexpr int ln_rows_per_block() { return ln_block<kV, kSplit>() / (64 * kSplit); }
constexpr int kLMaxH = 16384;      // 64 lanes x 32 units x 8 elements
#ifndef FP8Q_LN_BLOCKS_PER_CU
#define FP8Q_LN_BLOCKS_PER_CU 4
#endif
// A scheduling barrier after each unit of the last pass (below): measured slower once
// the next unit's gamma/beta are read during the current unit (8192 x 12288 75.2 vs 74.1
// us, 4096 x 16384 54.6 vs 52.6), so off.
#ifndef FP8Q_LN_UNIT_BARRIER
#define FP8Q_LN_UNIT_BARRIER 0
#endif
constexpr int kLBlocksPerCU = FP8Q_LN_BLOCKS_PER_CU;
// Wavefronts per row for 24 and 32 units per lane (hidden 8200-12288, 12296-16384).
// Measured (µs; one wavefront per row before the split): 4096 x 16384: 92 -> 2 parts 59-61,
// 4 parts 53-55; 8192 x 12288: 78.5 -> 76.7-77.7 / 74.4; 8192 x 10000: 72-75 / 67.7-69.2.
#ifndef FP8Q_LN_SPLIT24
#define FP8Q_LN_SPLIT24 4
#endif
#ifndef FP8Q_LN_SPLIT32
#define FP8Q_LN_SPLIT32 4
#endif
constexpr int kLSplit24 = FP8Q_LN_SPLIT24;
constexpr int kLSplit32 = FP8Q_LN_SPLIT32;

struct LnArgs {
  const uint16_t* x;
  const float* gamma;  // may be null: 1
  const float* beta;   // may be null: 0
  uint8_t* dst;
  const float* scale;
  uint32_t* amax;
  float* mean_out;  // may be null
  float* rstd_out;  // may be null
  int64_t rows;
  int32_t H;
  int32_t nunits;  // H / 8
  float eps;
  int32_t vec_affine;  // gamma and beta (where given) are 16-byte aligned
  float inv_h;         // RN(1/H)
  int32_t pad;
};

typedef uint32_t ln_u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t ln_u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t ln_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// Units u = lane + 64 k of one row; a unit past the row's end reads zeros (the
// resource covers exactly the row).
template <int kV>
__device__ __forceinline__ void ln_load_row(uint4 (&w)[kV], __amdgpu_buffer_rsrc_t rs,
                                            int lane) {
#pragma unroll
  for (int k = 0; k < kV; ++k) {
    const ln_u32x4 v = __builtin_bit_cast(
        ln_u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)(lane + 64 * k) * 16u, 0, 2));
    w[k] = make_uint4(v[0], v[1], v[2], v[3]);
  }
}

constexpr int ln_pow2_ceil(int n) { return n <= 1 ? 1 : 2 * ln_pow2_ceil((n + 1) / 2); }

// Pairwise (tree) sum of N values, depth ceil(log2 N): a count that is not a power of two
// is padded with exact zeros.
template <int N>
__device__ __forceinline__ float tree_sum(float (&v)[N]) {
  constexpr int P = ln_pow2_ceil(N);
  if constexpr (P == N) {
#pragma unroll
    for (int w = N / 2; w >= 1; w /= 2) {
#pragma unroll
      for (int i = 0; i < w; ++i) v[i] = v[i] + v[i + w];
    }
    return v[0];
  } else {
    float t[P];
#pragma unroll
    for (int i = 0; i < P; ++i) t[i] = i < N ? v[i] : 0.0f;
    return tree_sum(t);
  }
}

// Sum over the 64 lanes of a wavefront as a pairwise tree on the DPP network (no LDS
// round trips): xor-1 and xor-2 within quads, rotations by 4 and 8 within each 16-lane
// row, then row 0 + row 1 and row 2 + row 3 (row_bcast15), and their sum (row_bcast31)
// into lane 63, whose value is returned to every lane through a scalar register.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ float dpp_add(float v) {
  // lanes of rows outside kRowMask read 0 and keep v
  const float t = __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, kRowMask, 0xF,
                                         false));
  return v + t;
}

__device__ __forceinline__ float wave_sum(float v) {
  v = dpp_add<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v = dpp_add<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v = dpp_add<0x124, 0xF>(v);  // row_ror:4
  v = dpp_add<0x128, 0xF>(v);  // row_ror:8
  v = dpp_add<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v = dpp_add<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

__device__ __forceinline__ void wave_sum2(float& a, float& b) {
  a = dpp_add<0xB1, 0xF>(a);
  b = dpp_add<0xB1, 0xF>(b);
  a = dpp_add<0x4E, 0xF>(a);
  b = dpp_add<0x4E, 0xF>(b);
  a = dpp_add<0x124, 0xF>(a);
  b = dpp_add<0x124, 0xF>(b);
  a = dpp_add<0x128, 0xF>(a);
  b = dpp_add<0x128, 0xF>(b);
  a = dpp_add<0x142, 0xA>(a);
  b = dpp_add<0x142, 0xA>(b);
  a = dpp_add<0x143, 0xC>(a);
  b = dpp_add<0x143, 0xC>(b);
  a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, a), 63));
  b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, b), 63));
}

__device__ __forceinline__ float lo_f32(uint32_t w) { return as_float(w << 16); }
__device__ __forceinline__ float hi_f32(uint32_t w) { return as_float(w & 0xFFFF0000u); }

struct LnQuant {
  float s, r;
  uint32_t xlim;
  uint32_t clim;  // sat_limit_bf16(s): units whose |y| stay within need no saturation
  bool win;
  float gmax;     // max |gamma| of the block's staged gamma
  bool gb_fin;    // every staged gamma and beta is finite
};

// y rounded to bf16 (nearest even), returned as the binary32 of the same value: the
// packed convert puts RN_bf16(y) in the high half and RN_bf16(0) = 0 in the low one.
__device__ __forceinline__ float round_bf16(float y) {
  return as_float(pack_bf16_rne(0.0f, y));
}

// max(|v0|, ..., |v7|) of non-NaN values: four max3 with |.| source modifiers.
__device__ __forceinline__ float max3_abs(float a, float b, float c) {
  float m;
  __asm__("v_max3_f32 %0, |%1|, |%2|, |%3|" : "=v"(m) : "v"(a), "v"(b), "v"(c));
  return m;
}
__device__ __forceinline__ float max8_abs(const float (&v)[8]) {
  float m = max3_abs(v[0], v[1], v[2]);
  m = max3_abs(m, v[3], v[4]);
  m = max3_abs(m, v[5], v[6]);
  return max3_abs(m, v[7], v[7]);
}

// The codes of 8 bf16-valued binary32 y (the corrected division, saturated or, where
// the caller has checked that no quotient can exceed FP8_MAX, not), as codes8_bf16 and
// codes8_bf16_unsaturated give them for the packed values.
template <int kFmt, bool kSat>
__device__ __forceinline__ uint2 codes8_vals(const float (&x)[8], float s, float r) {
  float c[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float qk = div_corrected1(x[k], s, r);
    c[k] = kSat ? saturate<kFmt>(qk) : qk;
  }
  return make_uint2(pack4<kFmt>(c[0], c[1], c[2], c[3]), pack4<kFmt>(c[4], c[5], c[6], c[7]));
}

// 8 bf16-valued binary32 back to packed bf16 (exact).
__device__ __forceinline__ uint4 pack8_bf16(const float (&v)[8]) {
  return make_uint4(pack_bf16_rne(v[0], v[1]), pack_bf16_rne(v[2], v[3]),
                    pack_bf16_rne(v[4], v[5]), pack_bf16_rne(v[6], v[7]));
}

// Make the packed row opaque to the compiler between passes (an empty asm that
// rebinds the registers, emitting nothing): values derived from it are recomputed
// rather than merged with, and kept live from, an earlier pass.
template <int kV>
__device__ __forceinline__ void rebind(uint4 (&w)[kV]) {
#pragma unroll
  for (int k = 0; k < kV; ++k)
    __asm__ volatile("" : "+v"(w[k].x), "+v"(w[k].y), "+v"(w[k].z), "+v"(w[k].w));
}

// The 8 elements of a unit as binary32.
__device__ __forceinline__ void unpack8(const uint4& w, float (&x)[8]) {
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[2 * j] = lo_f32(u[j]);
    x[2 * j + 1] = hi_f32(u[j]);
  }
}

// Normalize, quantize and store one row held in w[] (units lane + 64 k).  The row
// stays packed; each pass re-derives x (and d = RN(x - mu'), bit-identical every time)
// unit by unit, so only the packed row and a few partial sums stay live.  Sums are
// trees: 8 elements of a unit (depth 3), then the kV units (depth log2 kV), then the
// wavefront (depth 6); for rows longer than 512, the squares of a unit are summed as a
// chain of fmas (depth 8 instead of 3, 8 instructions instead of 15).
// Sums of a row split over kSplit wavefronts (2 or 4): each part's wavefront sum goes to
// LDS and every lane adds the parts as the same tree ((p0 + p1) + (p2 + p3)), so all
// parts hold the identical value.  `xch` holds 3 floats per part of each row slot: the
// mean's partial, then the two deviation sums; one block barrier each.  (The next row's
// mean partial is written only after every wavefront has passed the deviation sums'
// barrier, i.e. has read this row's mean, and likewise for the deviation sums.)
template <int kSplit>
__device__ __forceinline__ float parts_sum(const float* xch, int i) {
  if constexpr (kSplit == 2) return xch[i] + xch[3 + i];
  else return (xch[i] + xch[3 + i]) + (xch[6 + i] + xch[9 + i]);
}

template <int kSplit>
__device__ __forceinline__ float row_total(float v, float* xch, int part, int lane) {
  if constexpr (kSplit == 1) {
    return v;
  } else {
    if (lane == 0) xch[3 * part] = v;
    __syncthreads();
    return parts_sum<kSplit>(xch, 0);
  }
}

template <int kSplit>
__device__ __forceinline__ void row_total2(float& a, float& b, float* xch, int part, int lane) {
  if constexpr (kSplit > 1) {
    if (lane == 0) {
      xch[3 * part + 1] = a;
      xch[3 * part + 2] = b;
    }
    __syncthreads();
    a = parts_sum<kSplit>(xch, 1);
    b = parts_sum<kSplit>(xch, 2);
  }
}

// Rows of up to 8 units per lane, one wavefront per row, keep the unpacked row (then
// its deviations d') in registers, 8 kV of them, instead of unpacking it again in each
// pass (3 fewer instructions per element); the packed registers are then free after the
// first pass and take the wavefront's next row, whose load overlaps this row's last two
// passes.  Longer rows stay packed (the registers would halve the resident wavefronts).
template <int kV, int kSplit>
constexpr bool ln_keep() { return kSplit == 1 && kV <= 8; }
// Measured (us, events; the row packed in every pass before): 8192 x 4096 28.2 -> kept
// 26.3, kept with the next row's load after the first pass (3 wavefronts per SIMD at 8
// units: the next row's registers do not fit under 4) 26.3; 16384 x 2048 28.3 -> 25.1
// -> 23.7, 32768 x 1024 30.2 -> 27.3 -> 24.6.
// Squares summed as fma chains (below); measured on 8192 x 4096 against the tree of
// products: 25.8 vs 26.3 us, one chain of 8: 26.0 us.
#ifndef FP8Q_LN_SQ_CHAIN
#define FP8Q_LN_SQ_CHAIN 1
#endif
// the next row's load inside ln_row (below), after the first pass (issued before it, so
// that the registers of both rows are live through the first pass, the 8-unit instance
// spills: 67 us on 8192 x 4096); FP8Q_LN_KEEP8_WAVES: wavefronts per SIMD the 8-unit
// instance is compiled for
// The next unit's gamma/beta read from LDS during the current unit of the last pass:
// with FP8Q_LN_UNIT_BARRIER off, 8192 x 4096 26.0 -> 25.4 us, 8192 x 12288 78.4 -> 74.1,
// 4096 x 16384 55.6 -> 52.6 (one box, one run).
#ifndef FP8Q_LN_GB_PREFETCH
#define FP8Q_LN_GB_PREFETCH 1
#endif
// Rows known to give no NaN skip the per-unit NaN test (below): 0.8 % on 8192 x 4096.
#ifndef FP8Q_LN_ROWFIN
#define FP8Q_LN_ROWFIN 1
#endif
#ifndef FP8Q_LN_PREFETCH
#define FP8Q_LN_PREFETCH 1
#endif
// The wavefront's first row loaded during the gamma/beta staging: 1 for the kept-row
// instances, 2 for all, 0 for none.  Measured (us, medians; none / kept / all): 8192 x
// 4096 24.6 / 24.5 / 24.4, 16384 x 2048 24.0 / 23.4 / 23.4, 8192 x 8192 50.9 / 50.9 /
// 53.2, 4096 x 16384 54.3 / 54.1 / 55.8 (the instances that hold a row per wavefront
// without keeping it lose when its registers are live through the staging).
#ifndef FP8Q_LN_EARLY_ROW
#define FP8Q_LN_EARLY_ROW 1
#endif
#ifndef FP8Q_LN_KEEP8_WAVES
#define FP8Q_LN_KEEP8_WAVES 3
#endif

// `half`: which part of the row's units this wavefront holds (units lane + 64 k +
// 64 kV half); `row_ok`: false for the padding rows of split blocks (no memory access,
// nothing accumulated), which still take part in the barriers.  With ln_keep, w[] holds
// the row `next_rs` covers on return (the next row's load issued after the first pass).
template <int kFmt, int kV, bool kMasked, int kSplit>
__device__ __forceinline__ void ln_row(uint4 (&w)[kV], const LnArgs& a, int64_t row,
                                       bool row_ok, int lane, int half, float* xch,
                                       const float* __restrict__ lg,
                                       const float* __restrict__ lb, const LnQuant& q,
                                       uint32_t& acc, __amdgpu_buffer_rsrc_t next_rs) {
  const float invH = a.inv_h;  // RN(1/H), exact for a power-of-two H
  const int ubase = 64 * kV * half;  // first unit of this wavefront's half
  constexpr bool kKeep = ln_keep<kV, kSplit>();
  float xs[kKeep ? kV : 1][8];
  // pass 1: mean (units past the row read as zeros)
  float p1[kV];
#pragma unroll
  for (int k = 0; k < kV; ++k) {
    float x[8];
    unpack8(w[k], x);
    if constexpr (kKeep) {
#pragma unroll
      for (int j = 0; j < 8; ++j) xs[k][j] = x[j];
    }
    p1[k] = tree_sum(x);
  }
  if constexpr (kKeep && FP8Q_LN_PREFETCH) {
    // the row is unpacked: its registers take the next row (kept below the unpacking)
    __builtin_amdgcn_sched_barrier(0);
    ln_load_row<kV>(w, next_rs, lane);
  }
  const float mu = row_total<kSplit>(wave_sum(tree_sum(p1)), xch, half, lane) * invH;
  // pass 2: deviations from mu', their sum and sum of squares
  if constexpr (!kKeep) rebind(w);
  float s1[kV], s2[kV];
#pragma unroll
  for (int k = 0; k < kV; ++k) {
    float x[8], sq[8];
    if constexpr (kKeep) {
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = xs[k][j];
    } else {
      unpack8(w[k], x);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = x[j] - mu;
    if constexpr (kKeep) {
#pragma unroll
      for (int j = 0; j < 8; ++j) xs[k][j] = x[j];
    }
    if constexpr (kV * kSplit >= 2 && FP8Q_LN_SQ_CHAIN) {
      // the unit's squares as two chains of 4 fmas (one rounding per element) and their
      // sum: depth 5 instead of 3, which rows over 512 long have room for under the
      // depth bound ceil(log2 H) + 6; 9 instructions instead of 15
      float qa = x[0] * x[0], qb = x[1] * x[1];
#pragma unroll
      for (int j = 2; j < 8; j += 2) {
        qa = __builtin_fmaf(x[j], x[j], qa);
        qb = __builtin_fmaf(x[j + 1], x[j + 1], qb);
      }
      s2[k] = qa + qb;
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) sq[j] = x[j] * x[j];
      s2[k] = tree_sum(sq);
    }
    s1[k] = tree_sum(x);
    if (kMasked && ubase + lane + 64 * k >= a.nunits) s1[k] = s2[k] = 0.0f;
  }
  float t1 = tree_sum(s1), t2 = tree_sum(s2);
  wave_sum2(t1, t2);
  row_total2<kSplit>(t1, t2, xch, half, lane);
  const float e = t1 * invH;
  float var = __builtin_fmaf(-e, e, t2 * invH);
  var = var < 0.0f ? 0.0f : var;  // rounding can dip below 0; a NaN stays NaN
  const float ve = var + a.eps;
  // hardware reciprocal square root (1 ulp) where its input is normal; the IEEE
  // square root and divide for a subnormal (or zero) V + eps
  const float rstd = ve >= 0x1p-126f ? __builtin_amdgcn_rsqf(ve) : 1.0f / __builtin_sqrtf(ve);
  // A row whose mean is finite (every x finite), whose rstd is finite and positive (every
  // d' and e' finite) and whose gamma rstd products stay finite, with finite gamma and
  // beta, gives no NaN y (an fma of finite operands is finite or overflows to an
  // infinity): its units skip the NaN test.  Wave-uniform (mu, rstd are).
  const bool row_fin = FP8Q_LN_ROWFIN && q.gb_fin && (as_uint(mu) & 0x7FFFFFFFu) < 0x7F800000u &&
                       rstd > 0.0f && q.gmax * rstd < __builtin_inff();
  if (lane == 0 && half == 0 && row_ok) {
    if (a.mean_out) a.mean_out[row] = mu + e;
    if (a.rstd_out) a.rstd_out[row] = rstd;
  }
  // pass 3: y, its bf16 rounding, the codes and the amax
  if constexpr (!kKeep) rebind(w);
  const __amdgpu_buffer_rsrc_t out =
      ln_rsrc(a.dst + (row_ok ? row * (int64_t)a.H : 0), row_ok ? (uint32_t)a.H : 0u);
  // gamma/beta of a unit's first 4 and last 4 columns (two planes: consecutive lanes
  // read consecutive 16 bytes)
  constexpr int kPlane = 64 * kV * kSplit;  // units, i.e. float4s per plane
  const float4* g4 = (const float4*)lg;
  const float4* b4 = (const float4*)lb;
  // Two forms of a unit's rounding, amax and codes, chosen per row by a scalar branch:
  // rows that give no NaN (row_fin) with the scale inside the division window round each
  // y to a bf16-valued binary32 in one instruction and take the magnitude max as a float
  // max3 with |.| modifiers, which for non-NaN values orders exactly as the bit patterns
  // do; other rows keep y packed, canonicalize NaNs and take the packed 16-bit magnitude
  // max.  Both give the same codes and amax.  The branch is per unit, after y: with a
  // whole unit loop per form the compiler hoists the y arithmetic the two loops share
  // above the branch, and the 8-unit instances spill.  Measured against the packed form
  // alone (us, medians of 5 x 20 launches, one box): 8192 x 4096 25.7 -> 25.0,
  // 8192 x 4000 25.4 -> 24.6, 16384 x 2048 24.8 -> 23.9, 8192 x 8192 54.6 -> 52.2,
  // 4096 x 16384 53.7 -> 54.1; 8 fewer VALU instructions per unit of 8 elements.
  uint32_t fast = uniform((uint32_t)(row_fin && q.win));
  // held in an SGPR (otherwise the compiler re-derives it, through a VGPR and a
  // readfirstlane, at every unit's branch)
  __asm__ volatile("" : "+s"(fast));
  {
    uint32_t acc32 = 0;  // fast rows: max |y| as binary32 bits (low 16 bits zero)
    float4 gb_next[4];
    if constexpr (FP8Q_LN_GB_PREFETCH) {
      const int u0 = ubase + lane;
      gb_next[0] = g4[u0];
      gb_next[1] = g4[kPlane + u0];
      gb_next[2] = b4[u0];
      gb_next[3] = b4[kPlane + u0];
    }
#pragma unroll
    for (int k = 0; k < kV; ++k) {
      const int unit = ubase + lane + 64 * k;
      float4 g0, g1, b0, b1;
      if constexpr (FP8Q_LN_GB_PREFETCH) {
        // this unit's values were read during the previous unit; read the next unit's now
        g0 = gb_next[0];
        g1 = gb_next[1];
        b0 = gb_next[2];
        b1 = gb_next[3];
        if (k + 1 < kV) {
          gb_next[0] = g4[unit + 64];
          gb_next[1] = g4[kPlane + unit + 64];
          gb_next[2] = b4[unit + 64];
          gb_next[3] = b4[kPlane + unit + 64];
        }
      } else {
        g0 = g4[unit];
        g1 = g4[kPlane + unit];
        b0 = b4[unit];
        b1 = b4[kPlane + unit];
      }
      const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
      const float bv[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
      float y[8];
      if constexpr (kKeep) {
#pragma unroll
        for (int j = 0; j < 8; ++j) y[j] = __builtin_fmaf(xs[k][j] - e, gv[j] * rstd, bv[j]);
      } else {
        float x[8];
        unpack8(w[k], x);
#pragma unroll
        for (int j = 0; j < 8; ++j) y[j] = __builtin_fmaf((x[j] - mu) - e, gv[j] * rstd, bv[j]);
      }
      const bool valid = row_ok && (!kMasked || unit < a.nunits);
      uint2 c;
      // a fresh scalar compare per unit: a compare shared by all units crosses blocks as
      // a lane mask, rebuilt with two VALU instructions at each branch
      uint32_t fast_u = fast;
      __asm__ volatile("" : "+s"(fast_u));
      if (fast_u) {
        float yb[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) yb[j] = round_bf16(y[j]);
        const uint32_t mb = as_uint(max8_abs(yb));
        acc32 = max(acc32, valid ? mb : 0u);
        // no saturation step where no quotient of the unit (across the wavefront) can
        // exceed FP8_MAX
        if (__builtin_amdgcn_ballot_w64(mb > q.clim << 16) == 0)
          c = codes8_vals<kFmt, false>(yb, q.s, q.r);
        else
          c = codes8_vals<kFmt, true>(yb, q.s, q.r);
        if (mb >= q.xlim << 16) c = patch8_bf16<kFmt>(c, pack8_bf16(yb), q.xlim);
      } else {
        uint4 yw = make_uint4(pack_bf16_rne(y[0], y[1]), pack_bf16_rne(y[2], y[3]),
                              pack_bf16_rne(y[4], y[5]), pack_bf16_rne(y[6], y[7]));
        uint32_t mg = mag8_bf16(yw);
        if (__builtin_amdgcn_ballot_w64(halves_nan(mg) != 0) != 0) {  // NaNs in the unit
          uint32_t o[4] = {yw.x, yw.y, yw.z, yw.w};
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            const uint32_t l = (o[h] & 0x7FFFu) > 0x7F80u ? 0x7FC0u : (o[h] & 0xFFFFu);
            const uint32_t u = ((o[h] >> 16) & 0x7FFFu) > 0x7F80u ? 0x7FC0u : (o[h] >> 16);
            o[h] = l | (u << 16);
          }
          yw = make_uint4(o[0], o[1], o[2], o[3]);
          mg = mag8_bf16(yw);
        }
        acc = pk_max_u16(acc, valid ? mg : 0u);
        if (q.win) {
          if (__builtin_amdgcn_ballot_w64(max_halves(mg) > q.clim) == 0)
            c = codes8_bf16_unsaturated<kFmt>(yw, q.s, q.r);
          else
            c = codes8_bf16<kFmt>(yw, q.s, q.r);
          if (max_halves(mg) >= q.xlim) c = patch8_bf16<kFmt>(c, yw, q.xlim);
        } else {
          const uint32_t u[4] = {yw.x, yw.y, yw.z, yw.w};
          uint32_t cw[2] = {0, 0};
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float v = (j & 1) ? hi_f32(u[j >> 1]) : lo_f32(u[j >> 1]);
            cw[j >> 2] |= code_ieee<kFmt>(v, q.s) << (8 * (j & 3));
          }
          c = make_uint2(cw[0], cw[1]);
        }
      }
      __builtin_amdgcn_raw_buffer_store_b64(ln_u32x2{c.x, c.y}, out, (uint32_t)unit * 8u, 0, 0);
#if FP8Q_LN_UNIT_BARRIER
      // keep each unit's work (LDS reads, arithmetic) from being hoisted into the
      // previous one's, which would hold every unit's temporaries at once
      __builtin_amdgcn_sched_barrier(0);
#endif
    }
    acc = pk_max_u16(acc, acc32 >> 16);
  }
}

// The resource of row r's part `half` (units from 64 kV half on) in split blocks: the
// part's bytes of the row, empty for a padding row past the end.
template <int kV, int kSplit>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t ln_split_rsrc(const LnArgs& a, int64_t r,
                                                               int half, uint32_t row_bytes) {
  // this half's units start 64 kV units (1024 kV bytes) into the row
  return r < a.rows ? ln_rsrc(a.x + r * a.H + 512 * kV * half,
                              row_bytes > 1024u * kV * half ? row_bytes - 1024u * kV * half : 0u)
                    : ln_rsrc(a.x, 0u);
}

// Rows kept unpacked (ln_keep) are held to the register count at which kLBlocksPerCU
// blocks of 4 wavefronts fit each CU (one wavefront of each block per SIMD).
template <int kV, int kSplit>
constexpr int ln_waves_per_eu() {
  return !ln_keep<kV, kSplit>() ? 1 : kV == 8 ? FP8Q_LN_KEEP8_WAVES : kLBlocksPerCU;
}

template <int kFmt, int kV, bool kMasked, int kSplit>
__global__ __launch_bounds__((ln_block<kV, kSplit>()))
__attribute__((amdgpu_waves_per_eu(ln_waves_per_eu<kV, kSplit>())))
void ln_quantize_kernel(const LnArgs a) {
  constexpr int kBlk = ln_block<kV, kSplit>();
  // gamma then beta, each 512 kV kSplit floats, zero-padded; 16-byte aligned for the
  // b128 reads.  Each is stored as two planes, columns 8u..8u+3 of every unit u, then
  // columns 8u+4..8u+7, so that a wavefront's reads of one plane (lane l: unit base + l)
  // are 64 consecutive 16-byte pieces, free of bank conflicts (unit-major order puts
  // lanes 32 bytes apart: 2-way conflicts).
  extern __shared__ __attribute__((aligned(16))) float lds[];
  __shared__ uint32_t block_amax;
  __shared__ float xch_all[kSplit > 1 ? 3 * kSplit * ln_rows_per_block<kV, kSplit>() : 1];
  constexpr int kPad = 512 * kV * kSplit;
  float* lg = lds;
  float* lb = lds + kPad;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: SGPR
  const int64_t nwaves = (int64_t)gridDim.x * (kBlk / 64);
  int64_t row = (int64_t)blockIdx.x * (kBlk / 64) + wave;  // (kSplit == 1)
  const uint32_t row_bytes = (uint32_t)a.H * 2u;
  // The wavefront's first row (or row part) is loaded while gamma/beta are staged:
  // issued after the gamma/beta loads, so the staging waits for those alone.
  uint4 w[kV];
  constexpr bool kEarly = FP8Q_LN_EARLY_ROW == 2 || (FP8Q_LN_EARLY_ROW == 1 && ln_keep<kV, kSplit>());
  const auto load_first = [&]() {
    if constexpr (!kEarly) {
    } else if constexpr (kSplit == 1) {
      ln_load_row<kV>(w, row < a.rows ? ln_rsrc(a.x + row * a.H, row_bytes) : ln_rsrc(a.x, 0u),
                      lane);
    } else {
      const int64_t r = (int64_t)blockIdx.x * ln_rows_per_block<kV, kSplit>() + wave / kSplit;
      ln_load_row<kV>(w, ln_split_rsrc<kV, kSplit>(a, r, wave % kSplit, row_bytes), lane);
    }
  };
  // stage gamma/beta: 16-byte loads, all issued before any is used.  Unconditional
  // buffer loads whose resources cover exactly gamma and beta (none for an absent one):
  // the pieces past H, and a missing gamma or beta, read zeros (a load under a branch
  // whose other side fills the same registers waits for the load before the next is
  // issued, one round trip per piece).
  if (a.vec_affine) {
    float4 gs[kPad / 4 / kBlk > 0 ? kPad / 4 / kBlk : 1];
    float4 bs[kPad / 4 / kBlk > 0 ? kPad / 4 / kBlk : 1];
    constexpr int kIt = (kPad / 4 + kBlk - 1) / kBlk;
    const __amdgpu_buffer_rsrc_t rg = ln_rsrc(a.gamma, a.gamma ? (uint32_t)a.H * 4u : 0u);
    const __amdgpu_buffer_rsrc_t rb = ln_rsrc(a.beta, a.beta ? (uint32_t)a.H * 4u : 0u);
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
      const uint32_t off = (uint32_t)(threadIdx.x + it * kBlk) * 16u;  // float4 index * 16
      gs[it] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rg, off, 0, 0));
      bs[it] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rb, off, 0, 0));
    }
    load_first();
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
      const int i4 = threadIdx.x + it * kBlk;
      if (4 * i4 < kPad) {
        const int p4 = (i4 & 1) * (kPad / 8) + (i4 >> 1);  // plane, unit
        float4 g = gs[it];
        if (!a.gamma) {  // gamma 1 inside the row, 0 in the padding
          const float one = 4 * i4 < a.H ? 1.0f : 0.0f;
          g = make_float4(one, one, one, one);
        }
        ((float4*)lg)[p4] = g;
        ((float4*)lb)[p4] = bs[it];
      }
    }
  } else {
    load_first();
    for (int i = threadIdx.x; i < kPad; i += kBlk) {
      const bool in = i < a.H;
      const int p = ((i >> 2) & 1) * (kPad / 2) + (i >> 3) * 4 + (i & 3);  // plane, unit, column
      lg[p] = in ? (a.gamma ? a.gamma[i] : 1.0f) : 0.0f;
      lb[p] = in ? (a.beta ? a.beta[i] : 0.0f) : 0.0f;
    }
  }
  if (threadIdx.x == 0) block_amax = 0;
  __shared__ uint32_t gb_gmax, gb_bmax;  // max |gamma|, max |beta| bits
  if (threadIdx.x == 0) gb_gmax = gb_bmax = 0;

  LnQuant q;
  q.s = uniform(*a.scale);
  q.r = 1.0f / q.s;
  q.win = (q.s >= 0x1p-80f) && (q.s <= 0x1p125f);
  q.xlim = min(as_uint(q.s * 0x1p126f) >> 16, 0x7F80u);
  q.clim = sat_limit_bf16<kFmt>(q.s);
  __syncthreads();
  // the staged gamma's largest magnitude and whether gamma and beta are all finite
  // (magnitude bits: unsigned order is magnitude order; inf and NaN lie at or above
  // 0x7F800000)
  {
    uint32_t gm = 0, bm = 0;
    for (int i = threadIdx.x; i < kPad / 4; i += kBlk) {
      const uint4 g4 = ((const uint4*)lg)[i], b4 = ((const uint4*)lb)[i];
      gm = max(max(max(gm, g4.x & 0x7FFFFFFFu), max(g4.y & 0x7FFFFFFFu, g4.z & 0x7FFFFFFFu)),
               g4.w & 0x7FFFFFFFu);
      bm = max(max(max(bm, b4.x & 0x7FFFFFFFu), max(b4.y & 0x7FFFFFFFu, b4.z & 0x7FFFFFFFu)),
               b4.w & 0x7FFFFFFFu);
    }
    gm = wave_max_u32(gm);
    bm = wave_max_u32(bm);
    if ((threadIdx.x & 63) == 0) {
      atomicMax(&gb_gmax, gm);
      atomicMax(&gb_bmax, bm);
    }
    __syncthreads();
    q.gmax = as_float(gb_gmax);
    q.gb_fin = gb_gmax < 0x7F800000u && gb_bmax < 0x7F800000u;
  }

  uint32_t acc = 0;
  if constexpr (kSplit == 1) {
    if constexpr (ln_keep<kV, kSplit>() && FP8Q_LN_PREFETCH) {
      // the next row is loaded inside ln_row, after the current row's first pass (a
      // row past the end has an empty resource and reads zeros)
      if constexpr (!kEarly) {
        if (row < a.rows) ln_load_row<kV>(w, ln_rsrc(a.x + row * a.H, row_bytes), lane);
      }
      for (; row < a.rows; row += nwaves) {
        const int64_t nx = row + nwaves;
        const __amdgpu_buffer_rsrc_t nrs =
            nx < a.rows ? ln_rsrc(a.x + nx * a.H, row_bytes) : ln_rsrc(a.x, 0u);
        ln_row<kFmt, kV, kMasked, 1>(w, a, row, true, lane, 0, nullptr, lg, lb, q, acc, nrs);
      }
    } else {
      // one row at a time: latency is hidden by the other resident wavefronts
      for (bool first = true; row < a.rows; row += nwaves, first = false) {
        if (!first || !kEarly) ln_load_row<kV>(w, ln_rsrc(a.x + row * a.H, row_bytes), lane);
        ln_row<kFmt, kV, kMasked, 1>(w, a, row, true, lane, 0, nullptr, lg, lb, q, acc,
                                     ln_rsrc(a.x, 0u));
      }
    }
  } else {
    // wavefronts kSplit r .. kSplit r + kSplit - 1 hold the parts of row slot r; every
    // wavefront of the block runs the same iterations (the barriers), padding rows past
    // the end
    constexpr int kRows = ln_rows_per_block<kV, kSplit>();
    const int slot = wave / kSplit, half = wave % kSplit;
    float* xch = xch_all + 3 * kSplit * slot;
    bool first = true;
    for (int64_t base = (int64_t)blockIdx.x * kRows; base < a.rows;
         base += (int64_t)gridDim.x * kRows, first = false) {
      const int64_t r = base + slot;
      const bool ok = r < a.rows;
      if (!first || !kEarly) ln_load_row<kV>(w, ln_split_rsrc<kV, kSplit>(a, r, half, row_bytes), lane);
      ln_row<kFmt, kV, kMasked, kSplit>(w, a, r, ok, lane, half, xch, lg, lb, q, acc,
                                        ln_rsrc(a.x, 0u));
    }
  }
  // block amax: packed halves -> wavefront -> LDS -> one global atomic
  uint32_t m = max_halves(acc) << 16;
  m = wave_max_u32(m);
  if (lane == 0 && m != 0) atomicMax(&block_amax, m);
  __syncthreads();
  if (threadIdx.x == 0 && block_amax != 0) amax_accumulate(a.amax, block_amax);
}

// ---------------------------------------------------------------- host side
template <int kFmt, int kV, bool kMasked, int kSplit = 1>
static int ln_launch(const LnArgs& a, hipStream_t stream) {
  constexpr int kBlk = ln_block<kV, kSplit>();
  const void* fn = (const void*)ln_quantize_kernel<kFmt, kV, kMasked, kSplit>;
  const size_t smem = (size_t)2 * 512 * kV * kSplit * sizeof(float);
  static std::atomic<int> fit[64];  // per device (the LDS attribute is set on each one)
  const int dev = current_device_index();
  if (dev < 0) return FP8Q_EHIP;
  int per_cu = fit[dev].load(std::memory_order_relaxed);
  if (per_cu <= 0) {
    // gamma/beta staging beyond 64 KB (24 and 32 units per lane: 96 and 128 KB)
    if (smem > 65536 &&
        hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem) !=
            hipSuccess)
      return FP8Q_EHIP;
    int occ = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, fn, kBlk, smem) != hipSuccess)
      return FP8Q_EHIP;
    per_cu = occ < kLBlocksPerCU ? (occ > 0 ? occ : 1) : kLBlocksPerCU;
    fit[dev].store(per_cu, std::memory_order_relaxed);
  }
  int cus = 0;
  const int st = current_device_cus(&cus);
  if (st != FP8Q_OK) return st;
  constexpr int kRowsPerBlock = kBlk / (64 * kSplit);
  int64_t blocks = (a.rows + kRowsPerBlock - 1) / kRowsPerBlock;
  const int64_t cap = (int64_t)cus * per_cu;
  if (blocks > cap) blocks = cap;
  void* args[] = {(void*)&a};
  return launch_status(
      hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(kBlk), args, smem, stream));
}

template <int kFmt>
static int ln_dispatch(const LnArgs& a, hipStream_t stream) {
  const int need = (a.nunits + 63) / 64;  // units per lane
  const int kv = need <= 1 ? 1 : need <= 2 ? 2 : need <= 4 ? 4 : need <= 8 ? 8 : need <= 16 ? 16
                 : need <= 24 ? 24 : 32;
  const bool masked = a.nunits != 64 * kv;
  switch (kv) {
    case 1: return masked ? ln_launch<kFmt, 1, true>(a, stream) : ln_launch<kFmt, 1, false>(a, stream);
    case 2: return masked ? ln_launch<kFmt, 2, true>(a, stream) : ln_launch<kFmt, 2, false>(a, stream);
    case 4: return masked ? ln_launch<kFmt, 4, true>(a, stream) : ln_launch<kFmt, 4, false>(a, stream);
    case 8: return masked ? ln_launch<kFmt, 8, true>(a, stream) : ln_launch<kFmt, 8, false>(a, stream);
    case 16: return masked ? ln_launch<kFmt, 16, true>(a, stream) : ln_launch<kFmt, 16, false>(a, stream);
    // hidden 8200 .. 12288 (12288: the hidden-12288 MLP) and 12296 .. 16384
    case 24:
      return masked ? ln_launch<kFmt, 24 / kLSplit24, true, kLSplit24>(a, stream)
                    : ln_launch<kFmt, 24 / kLSplit24, false, kLSplit24>(a, stream);
    default:
      return masked ? ln_launch<kFmt, 32 / kLSplit32, true, kLSplit32>(a, stream)
                    : ln_launch<kFmt, 32 / kLSplit32, false, kLSplit32>(a, stream);
  }
}

}  // namespace fp8q

using namespace fp8q;

extern "C" int fp8_layernorm_quantize_amax(const void* x, int x_dtype, const float* gamma,
                                           const float* beta, float eps, int64_t rows,
                                           int64_t hidden, uint8_t* dst, int format,
                                           const float* scale, float* amax, float* mean,
                                           float* rstd, void* stream) {
  if (rows < 0 || hidden < 0) return FP8Q_EINVAL;
  if (format != FP8Q_E4M3 && format != FP8Q_E5M2) return FP8Q_EINVAL;
  if (x_dtype != FP8Q_BF16 && x_dtype != FP8Q_F32) return FP8Q_EINVAL;
  if (scale == nullptr || amax == nullptr) return FP8Q_EINVAL;
  if (!(eps >= 0.0f) || eps > 3.4e38f) return FP8Q_EINVAL;  // NaN, negative or inf
  if (x_dtype != FP8Q_BF16) return FP8Q_EUNSUPPORTED;
  if (rows == 0 || hidden == 0) return FP8Q_OK;
  if (x == nullptr || dst == nullptr) return FP8Q_EINVAL;
  if (hidden % 8 != 0 || hidden > kLMaxH) return FP8Q_EUNSUPPORTED;
  if ((uintptr_t)x % 16 != 0 || (uintptr_t)dst % 8 != 0) return FP8Q_EUNSUPPORTED;
  if (rows > INT64_MAX / hidden) return FP8Q_EINVAL;
  LnArgs a;
  a.x = (const uint16_t*)x;
  a.gamma = gamma;
  a.beta = beta;
  a.dst = dst;
  a.scale = scale;
  a.amax = (uint32_t*)amax;
  a.mean_out = mean;
  a.rstd_out = rstd;
  a.rows = rows;
  a.H = (int32_t)hidden;
  a.nunits = (int32_t)(hidden / 8);
  a.eps = eps;
  a.vec_affine = ((uintptr_t)gamma % 16 == 0) && ((uintptr_t)beta % 16 == 0);
  a.inv_h = 1.0f / (float)hidden;
  a.pad = 0;
  return format == FP8Q_E4M3 ? ln_dispatch<FP8Q_E4M3>(a, (hipStream_t)stream)
                             : ln_dispatch<FP8Q_E5M2>(a, (hipStream_t)stream);
}
