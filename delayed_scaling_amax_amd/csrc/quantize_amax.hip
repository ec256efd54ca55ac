// quantize_amax.hip -- fused FP8 quantize + amax over one or many tensors, one launch.
//
// What it computes ("User Guide on Native XLA-FP8", section "JAX"; "Fusion of Fp8
// quantization and amax reduction kernels", openxla/xla issue 7432): for every element
// x of a tensor, code = FP8(saturate(RN32(x / scale))) with the scale of the previous
// step, and in the same pass amax = max(amax, max|x|).
//
// Design (gfx950, HBM-bound at 3 bytes/element for bf16 -> fp8):
//  * A unit is 8 elements.  A tensor's units are its aligned body, read as 16-byte
//    bf16x8 loads, a lane taking two adjacent units per 16-byte code store, then its
//    unaligned head/tail elements ("scalar units").  Units are grouped into chunks of kQChunk that never straddle tensors;
//    all tensors' chunks form one chunk space.  The grid is persistent (a few blocks
//    per CU) and walks that space grid-stride, so at any moment the whole chip streams
//    one contiguous window of memory; a block issues one amax atomic per tensor.
//  * amax is an integer max: |x| is the bit pattern with the sign cleared (bf16: two
//    halves at once with v_pk_max_u16), reduced lane -> wavefront -> block, then one
//    atomicMax on the binary32 bit pattern (skipped when amax already holds as much).
//    Non-negative floats order like their bits, NaN above inf, so the result does not
//    depend on atomic order.
//  * Division.  r = RN(1/scale) once per tensor (IEEE).  Per element the quotient is
//    q0 = RN(x*r) corrected by Markstein's step (q = q0 - (q0*s - x)*r as two FMAs;
//    twice for fp32 sources), which equals the IEEE quotient while scale is in
//    [2^-80, 2^125] and |x| < scale*2^126 -- the host sweep in the tests covers every
//    bf16 mantissa against every scale mantissa.  A group of 8 with any element
//    outside that window (or inf/NaN) takes the IEEE divide per element.
//  * Saturation with v_med3_f32 against +-FP8_MAX, then the native OCP convert
//    v_cvt_pk_fp8_f32 / v_cvt_pk_bf8_f32 (round to nearest even).  NaN quotients
//    (only possible on the IEEE path) are written as 0x7F with the sign of x.
#include <hip/hip_ext.h>
#include <string.h>

#include <mutex>

#include "device_common.h"
#include "host_common.h"
#include "quant_math.h"

namespace fp8q {

// Launch shape (measured on MI355X; overridable at build time for tuning sweeps).
#ifndef FP8Q_Q_BLOCK
#define FP8Q_Q_BLOCK 256
#endif
// Chunks of 8 units per thread with one pass in flight ahead and one block (four
// wavefronts) per CU.  With the waits covering only the pass being converted, a wavefront
// keeps a whole pass of loads in flight, and one block per CU is the fastest measured at
// every size: against two, 701 vs 734 us on a 4 GB step, 89.3 vs 90.3 us on 0.5 GB, 6.75
// vs 6.95 us on 3 x 1M elements (two blocks with the waits that also covered the
// look-ahead: 708, 90.9 and 6.8 us).  16 units per thread were slower at every size.
#ifndef FP8Q_Q_UNROLL
#define FP8Q_Q_UNROLL 8
#endif
#ifndef FP8Q_Q_BLOCKS_PER_CU
#define FP8Q_Q_BLOCKS_PER_CU 1
#endif
// Cache policy of the streaming body (gfx950 buffer-op aux bits: 1 = sc0, 2 = nt,
// 16 = sc1).  Measured on the read-16B/write-8B shape of this kernel: non-temporal
// loads and sc1 (device-scope, write-through) stores reach ~87% of HBM peak, against
// ~70% with default policies.
#ifndef FP8Q_Q_LD_AUX
#define FP8Q_Q_LD_AUX 2
#endif
#ifndef FP8Q_Q_ST_AUX
#define FP8Q_Q_ST_AUX 16
#endif
// Launches whose codes are larger than the 256 MB Infinity Cache in front of HBM store
// them non-temporally as well (nt | sc1): they could not stay in the cache for the
// consumer, and on the 4.08 GB hidden-12288 step (1.36 GB of codes) this is 1.4-2 %
// faster (685 against 695-699 us, interleaved in one process).  Smaller launches keep
// sc1 stores, which leave the codes in the cache for the GEMM that reads them next (on
// a 0.5 GB step quantized repeatedly, nt stores were 8 % slower: 83.6 against 76.9 us).
#ifndef FP8Q_Q_ST_STREAM_AUX
#define FP8Q_Q_ST_STREAM_AUX 18
#endif
#ifndef FP8Q_Q_STREAM_BYTES
#define FP8Q_Q_STREAM_BYTES (256LL << 20)
#endif
constexpr int64_t kQStreamBytes = FP8Q_Q_STREAM_BYTES;
constexpr int kQBlock = FP8Q_Q_BLOCK;             // threads per block
constexpr int kQUnroll = FP8Q_Q_UNROLL;           // 8-element groups per thread per chunk
constexpr int kQMaxEntries = 32;                  // tensors per launch (kernel-argument table)
constexpr int kQPlanMaxEntries = 2048;            // tensors per launch (planned table in device memory)
constexpr int kQBlocksPerCU = FP8Q_Q_BLOCKS_PER_CU;  // persistent grid size per CU
#ifndef FP8Q_Q_GELU_BLOCKS_PER_CU
#define FP8Q_Q_GELU_BLOCKS_PER_CU 6
#endif
// the evaluated gelu instance (FP8Q_Q_GELU_TABLE 0) is arithmetic-bound: more resident
// waves hide exp/rcp latency (on 8192 x 16384 bf16 with the direct form: 6 blocks per CU
// 75-80 us, 5 76-80, 4 79-86, 3 79-89; its 79 registers leave room for six).  With the
// table its 128 KB of LDS leave room for one block per CU, which the occupancy query at
// launch applies.
constexpr int kQGeluBlocksPerCU = FP8Q_Q_GELU_BLOCKS_PER_CU;
constexpr int kQChunk = kQBlock * kQUnroll;       // units (8-element groups) per chunk
#ifndef FP8Q_Q_DEPTH
#define FP8Q_Q_DEPTH 1
#endif
#ifndef FP8Q_Q_PASS
#define FP8Q_Q_PASS 4
#endif
// Unit-to-lane layout of a pass: 0 = lane l takes unit l of each 256-unit row of the
// pass, so each 16-byte load instruction reads one contiguous 4 KB span (bf16; fp32: two
// instructions per unit, 32-byte stride) and each lane writes 8 code bytes; 1 = a lane
// takes two adjacent units (32 contiguous bytes of bf16, 64 of fp32: each load
// instruction then reads every second or fourth 16-byte piece of its span) and writes
// their 16 code bytes with one store.  With the waits covering only the pass being
// converted and one block per CU, 0 is faster at every size measured: 0.5 GB bf16 step
// 83.0 vs 89.4 us, 4 GB 694 vs 702 us, fp32 134M elements 115.5 vs 160.7 us, gelu 97.7
// vs 99.0 us.  (1 was adopted when the waits also covered the look-ahead pass.)
#ifndef FP8Q_Q_PAIR
#define FP8Q_Q_PAIR 0
#endif
constexpr bool kQPair = FP8Q_Q_PAIR != 0;
// Chunk split over the grid: 1 = grid-stride, 0 = contiguous ranges per block (kernel-
// argument tables); planned tables: FP8Q_Q_PLAN_CONTIG (1 = contiguous ranges).
#ifndef FP8Q_Q_SCHEDULE
#define FP8Q_Q_SCHEDULE 1
#endif
#ifndef FP8Q_Q_PLAN_CONTIG
#define FP8Q_Q_PLAN_CONTIG 0
#endif
// Passes in flight ahead of the one being converted.  One is enough for every instance
// (the gelu one included) once the waits cover only the pass being converted: two were
// 1-2% slower on the plain quantize of a 0.5 GB step and 2% on the gelu one.
constexpr int kQDepth = FP8Q_Q_DEPTH;
// Planned tables of many small tensors move to another tensor on nearly every chunk, and
// finding it costs two dependent scalar loads (the chunk's entry, then its fields) that
// stall the wavefront before the next loads can be issued.  More resident wavefronts
// hide the stalls: on the 1152-tensor list (402.7 M elements), 1 block per CU 308 us, 2
// 241, 3 229-230, 4 with two passes ahead 227; two passes ahead add 1-2 % (one block
// per CU: 308 / 302 / 309 us for one, two, three).
#ifndef FP8Q_Q_PLAN_DEPTH
#define FP8Q_Q_PLAN_DEPTH 2
#endif
constexpr int kQPlanDepth = FP8Q_Q_PLAN_DEPTH;
#ifndef FP8Q_Q_PLAN_BLOCKS_PER_CU
#define FP8Q_Q_PLAN_BLOCKS_PER_CU 3
#endif
constexpr int kQPlanBlocksPerCU = FP8Q_Q_PLAN_BLOCKS_PER_CU;
constexpr int kQPass = FP8Q_Q_PASS;    // bf16 groups per pass (fp32: half)
// The gelu instance (table in LDS, one block per CU) converts whole chunks as one pass of
// 8 groups: more bytes in flight per wavefront against the LDS gathers' latency.  On the
// (2048,4,16384) pre-activation (us, best of 3 x 20 launches, 4 rounds): passes of 2
// groups 83.8-85.2, 4 69.2-72.8, 8 65.0-68.3, 8 with two passes ahead 65.7-68.9.
#ifndef FP8Q_Q_GELU_PASS
#define FP8Q_Q_GELU_PASS 8
#endif
constexpr int kQGeluPass = FP8Q_Q_GELU_PASS;  // groups per pass, gelu instance

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// s_waitcnt immediate for vmcnt(0) alone (gfx9 encoding: expcnt and lgkmcnt at their
// maxima, so only vector memory operations are waited for).
constexpr int kVmcnt0 = 0x0F70;

// Buffer resource over [base, base + bytes) (raw, dword-granular, no swizzle).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// voff: per-lane byte offset (VGPR); soff: wave-uniform byte offset (SGPR/constant).
__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                               uint32_t soff) {
  const u32x4 v = __builtin_bit_cast(
      u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, FP8Q_Q_LD_AUX));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

template <int kAux = FP8Q_Q_ST_AUX>
__device__ __forceinline__ void buffer_store8(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                              uint32_t soff, uint2 o) {
  __builtin_amdgcn_raw_buffer_store_b64(u32x2{o.x, o.y}, r, voff, soff, kAux);
}

template <int kAux = FP8Q_Q_ST_AUX>
__device__ __forceinline__ void buffer_store16(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                               uint32_t soff, uint2 a, uint2 b) {
  __builtin_amdgcn_raw_buffer_store_b128(u32x4{a.x, a.y, b.x, b.y}, r, voff, soff, kAux);
}

__device__ __forceinline__ uint4 load16(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ void store8(uint2* p, uint2 o) { *(u32x2*)p = u32x2{o.x, o.y}; }

struct QEntry {
  const void* src;
  uint8_t* dst;
  const float* scale;
  uint32_t* amax;
  int64_t fbegin;   // first full chunk of this tensor in the launch's full-chunk space
  int64_t nfull;    // full chunks of the aligned body: n_vec / kQChunk
  int64_t n_units;  // vector groups + scalar units
  int64_t n_vec;    // 8-element groups at [head, head + 8*n_vec), 16B/8B aligned
  int64_t head;     // elements before the first vector group
  int64_t numel;
  int32_t dtype;
  int32_t fmt;
  int32_t gelu;     // producer prologue: quantize RN_bf16(gelu(x)) instead of x (bf16 only)
  int32_t pad;
};

// Kinds: dtype * 2 + fmt for plain entries (0..3), 4 + fmt for gelu-prologue entries.
constexpr int kQKinds = 6;
__host__ __device__ __forceinline__ int entry_kind(const QEntry& e) {
  return e.gelu ? 4 + e.fmt : e.dtype * 2 + e.fmt;
}

// The batched amax_and_scale_update appended to a quantize launch
// (fp8_quantize_amax_and_update): the history roll by the block that finishes its
// quantize work first, the rest by the block that finishes last, over n <= kQUpdMaxCols
// tensors with history[H][n], H * n <= kQUpdMaxElems.
constexpr int64_t kQUpdMaxCols = 256;
constexpr int64_t kQUpdMaxElems = 65536;
static_assert(kQUpdMaxCols <= kQBlock, "the appended update gives each column a thread");
struct QUpdate {
  float* amax;
  float* hist;
  float* scale;
  float* scale_inv;
  const uint8_t* formats;
  uint32_t* counter;  // blocks finished (+1 for the roll); 0 at launch, left 0
  int64_t n;
  int64_t H;
  int32_t algo;
  int32_t margin;
  int32_t reset;
  int32_t pad;
};

// Entries are sorted by kind: kind k occupies [run_end[k-1], run_end[k]).
struct QTable {
  static constexpr bool kPlanned = false;
  static constexpr bool kContig = FP8Q_Q_SCHEDULE == 0;
  QEntry e[kQMaxEntries];
  int64_t total_full;
  int32_t n;
  int32_t run_end[kQKinds];
  QUpdate upd;  // used by the kUpd kernel instances only
};
static_assert(sizeof(QTable) <= 4096, "the table travels as the kernel argument");

// A planned table (fp8_multi_quantize_plan): up to kQPlanMaxEntries entries in device
// memory, laid out and sorted as in QTable, and the entry holding each full chunk (so a
// block that moves on to a chunk of another tensor finds it with one load, where a
// search over the entries would cost a chain of dependent loads per move); the header
// travels as the kernel argument.
struct QPlanTable {
  static constexpr bool kPlanned = true;
  static constexpr bool kContig = FP8Q_Q_PLAN_CONTIG != 0;
  const QEntry* __restrict__ e;
  const int32_t* __restrict__ chunk_entry;  // [total_full]
  int64_t total_full;
  int32_t n;
  int32_t run_end[kQKinds];
};

// ---------------------------------------------------------------- gelu prologue
// y = RN_bf16(gelu(x)) for bf16 x, tanh form, in binary32 through its exact identity
// gelu(x) = x / (1 + 2^t), t = -2 log2(e) u, u = sqrt(2/pi) * (x + 0.044715 x^3).
// With h = t/2 and m = 2^-|h| (never below 2^-126 where it matters, so the exp unit's
// lack of subnormal results is harmless), m^2 = 2^-|t| and
//   t <= 0:  y = x / (1 + 2^t)          = x * d
//   t >  0:  y = x 2^-t / (1 + 2^-t)    = ((x * d) * m) * m,   d = 1 / (1 + m^2),
// the last product rounding once into the subnormal range for the tiny tails.  No
// branches: one exp2, one reciprocal.  Error of the binary32 value before the bf16
// rounding: h carries 3 roundings (constants folded so 1 + 0.044715 x^2 is one fma),
// amplified by |2u| through the exponential, plus a few ulps from exp2, the reciprocal
// and the products -- below (3|2u| + 10) * 2^-24 relative.  (Checked exhaustively:
// every bf16 input, against the double-precision value and its error window.)
// Non-finite inputs: +inf gives +inf by itself; -inf and NaN give NaN and are patched
// (gelu(-inf) = -0, gelu(NaN) = the default NaN with the input's sign).
__device__ __forceinline__ float gelu_f32(float x) {
  constexpr float kH = (float)(-0.7978845608028654 * 1.4426950408889634);
  constexpr float kH3 = (float)(-0.7978845608028654 * 1.4426950408889634 * 0.044715);
  const float h = x * __builtin_fmaf(kH3, x * x, kH);
  const float m = __builtin_amdgcn_exp2f(-__builtin_fabsf(h));
  const float d = __builtin_amdgcn_rcpf(__builtin_fmaf(m, m, 1.0f));
  const float p = x * d;
  return h > 0.0f ? (p * m) * m : p;
}

// The direct form for inputs above -9 (where 2^t < 2^104, far from overflow, and the
// quotient stays a normal binary32): t = -2 log2(e) u folded into two constants,
// y = x * rcp(1 + 2^t) -- one exp2, one reciprocal, five other operations (the form
// above takes nine).  Error before the bf16 rounding: t carries 3 roundings amplified by
// |2u| through the exponential, plus the exp2, the sum, the reciprocal and the product:
// below (4|2u| + 5) * 2^-24 relative.  +inf gives +inf, NaN gives NaN (patched).
__device__ __forceinline__ float gelu_f32_direct(float x) {
  constexpr float kT = (float)(-2.0 * 0.7978845608028654 * 1.4426950408889634);
  constexpr float kT3 = (float)(-2.0 * 0.7978845608028654 * 1.4426950408889634 * 0.044715);
  const float t = x * __builtin_fmaf(kT3, x * x, kT);
  return x * __builtin_amdgcn_rcpf(__builtin_amdgcn_exp2f(t) + 1.0f);
}

// Raw bf16 bits at or above this (as unsigned 16-bit values): x <= -9, -inf or a NaN with
// the sign bit set -- the inputs the direct form is not used for.
constexpr uint32_t kGeluDirectLimit = 0xC110u;

// gelu of a non-finite bf16 input h (exponent all ones).
__device__ __forceinline__ uint32_t gelu_special(uint32_t h) {
  if ((h & 0x7FFFu) > 0x7F80u) return (h & 0x8000u) | 0x7FC0u;  // NaN
  return (h & 0x8000u) ? 0x8000u : 0x7F80u;                        // -inf -> -0, +inf
}

// One bf16 pre-activation (low 16 bits of h) -> bf16 bits of its gelu.
__device__ __forceinline__ uint32_t gelu_bf16(uint32_t h) {
  if ((h & 0x7F80u) == 0x7F80u) return gelu_special(h);
  return pack_bf16_rne(gelu_f32(as_float(h << 16)), 0.0f) & 0xFFFFu;
}

// Eight bf16 pre-activations -> eight bf16 gelu outputs (same packing), before the
// patch of non-finite inputs: a NaN output comes from a NaN or -inf input, nothing else.
__device__ __forceinline__ uint4 gelu8_unpatched(uint4 w) {
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
  uint32_t o[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
    o[k] = pack_bf16_rne(gelu_f32(as_float(u[k] << 16)), gelu_f32(as_float(u[k] & 0xFFFF0000u)));
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// Eight bf16 inputs, all above -9 (or +inf, or positive NaN), through the direct form.
__device__ __forceinline__ uint4 gelu8_direct(uint4 w) {
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
  uint32_t o[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
    o[k] = pack_bf16_rne(gelu_f32_direct(as_float(u[k] << 16)),
                         gelu_f32_direct(as_float(u[k] & 0xFFFF0000u)));
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// Replace the outputs of non-finite inputs in y = gelu8_unpatched(w).
__device__ __forceinline__ uint4 gelu8_patch(uint4 w, uint4 y) {
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
  uint32_t o[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t lo = u[k] & 0xFFFFu, hi = u[k] >> 16;
    const uint32_t ol = (lo & 0x7F80u) == 0x7F80u ? gelu_special(lo) : (o[k] & 0xFFFFu);
    const uint32_t oh = (hi & 0x7F80u) == 0x7F80u ? gelu_special(hi) : (o[k] >> 16);
    o[k] = ol | (oh << 16);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// gelu of eight packed bf16 values, patched; the wave tests for NaN outputs once.
__device__ __forceinline__ uint4 gelu8_bf16(uint4 w) {
  const uint4 y = gelu8_unpatched(w);
  const uint32_t mg = pk_max_u16(pk_max_u16(y.x & 0x7FFF7FFFu, y.y & 0x7FFF7FFFu),
                                 pk_max_u16(y.z & 0x7FFF7FFFu, y.w & 0x7FFF7FFFu));
  if (__builtin_amdgcn_ballot_w64(halves_nan(mg) != 0) != 0) return gelu8_patch(w, y);
  return y;
}

// ---------------------------------------------------------------- gelu table
// A bf16 input has 65536 bit patterns, so the full-chunk passes of the gelu instance
// look its output up instead of evaluating it: gelu_bf16 of every pattern, built on each
// device by gelu_table_kernel (the same arithmetic as above, run once per device before
// its first gelu launch), copied into each block's LDS at kernel start (128 KB: the
// instance runs one block per CU) and read with 16-bit gathers -- one LDS read and about
// one address instruction per element instead of ten instructions, two of them
// transcendental.  The remainders (phase 2) still evaluate per element, with the same
// gelu_bf16.  FP8Q_Q_GELU_TABLE 0 keeps the evaluated form everywhere.
#ifndef FP8Q_Q_GELU_TABLE
#define FP8Q_Q_GELU_TABLE 1
#endif
constexpr bool kQGeluTable = FP8Q_Q_GELU_TABLE != 0;
constexpr int kQGeluTableBytes = 65536 * 2;
static __device__ __attribute__((aligned(16))) uint16_t g_gelu_table[65536];

__global__ __launch_bounds__(256) void gelu_table_kernel() {
  const uint32_t h = blockIdx.x * 256u + threadIdx.x;  // grid of 256 blocks: every pattern
  g_gelu_table[h] = (uint16_t)gelu_bf16(h);
}

// the gelu instance's dynamic LDS: the table
extern __shared__ __attribute__((aligned(16))) uint16_t q_gelu_lds[];

// Copy the table into this block's LDS by LDS DMA (16 bytes per lane, 1 KB per
// wavefront instruction, no registers), then wait for it and publish it to the block.
__device__ __forceinline__ void gelu_table_to_lds() {
  typedef __attribute__((address_space(3))) uint8_t lds_u8;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)g_gelu_table, (short)0, kQGeluTableBytes, 0x00020000);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t lane = threadIdx.x & 63;
  constexpr int kPieces = kQGeluTableBytes / 1024 / (kQBlock / 64);  // 1 KB pieces per wave
#pragma unroll
  for (int j = 0; j < kPieces; ++j) {
    const uint32_t piece = (uint32_t)(wave * kPieces + j);  // wave-uniform
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (__attribute__((address_space(3))) void*)((lds_u8*)q_gelu_lds + 1024 * piece), 16,
        piece * 1024u + lane * 16u, 0, 0, 0);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

// gelu of the two bf16 values of w, from the LDS table
__device__ __forceinline__ uint32_t gelu2_lds(uint32_t w) {
  return (uint32_t)q_gelu_lds[w & 0xFFFFu] | ((uint32_t)q_gelu_lds[w >> 16] << 16);
}

// ---------------------------------------------------------------- per-tensor constants
// Filled once per block at kernel start (one thread per tensor) so that switching to
// the next tensor costs an LDS read, not a dependent global load.
template <int kCap>
struct QSharedT {
  float scale[kCap];
  float rcp[kCap];      // RN(1/scale)
  uint32_t xlim[kCap];  // magnitude bits at which the fixed-code path starts
  uint32_t win[kCap];   // scale inside the Markstein window
  uint32_t amax[kCap];  // this block's amax bits per tensor
  uint32_t last;        // kUpd: the finished-block count before this block's
  uint32_t any_out;     // planned tables: some tensor's scale is outside the window
};
using QShared = QSharedT<kQMaxEntries>;

// Fold a thread's accumulator into the block's amax slot of tensor t: wavefront max,
// then one LDS atomic max per wavefront (no barrier).
template <bool kBF16, class Sh>
__device__ __forceinline__ void flush_amax(uint32_t acc, Sh& sh, int t) {
  if constexpr (kBF16) {
    const uint32_t lo = acc & 0xFFFFu, hi = acc >> 16;
    acc = (lo > hi ? lo : hi) << 16;
  }
  acc = wave_max_u32(acc);
  if ((threadIdx.x & 63) == 0 && acc != 0) atomicMax(&sh.amax[t], acc);
}

// The per-tensor constants of entry t (one thread per tensor).
template <class Tab, class Sh>
__device__ __forceinline__ void setup_entry(const Tab& tab, Sh& sh, int t) {
  const float s = *tab.e[t].scale;
  sh.scale[t] = s;
  sh.rcp[t] = 1.0f / s;
  // the window needs r normal and every residual exact (see the division notes)
  sh.win[t] = (s >= 0x1p-80f) && (s <= 0x1p125f);
  const uint32_t lim = as_uint(s * 0x1p126f);  // +inf when s >= 4
  sh.xlim[t] = tab.e[t].dtype == FP8Q_BF16 ? min(lim >> 16, 0x7F80u) : min(lim, 0x7F800000u);
  sh.amax[t] = 0;
}

// Fill the per-tensor constants and zero the block's amax slots; for a planned table
// also note whether any tensor's scale lies outside the window.  Contains a barrier:
// every thread of the block calls it exactly once.
template <class Tab, class Sh>
__device__ __forceinline__ void setup_shared(const Tab& tab, Sh& sh) {
  const int tid = threadIdx.x;
  if constexpr (Tab::kPlanned) {
    uint32_t out = 0;
    for (int t = tid; t < tab.n; t += kQBlock) {
      setup_entry(tab, sh, t);
      out |= sh.win[t] ^ 1u;
    }
    sh.any_out = __syncthreads_or(out) != 0;
  } else {
    if (tid < tab.n) setup_entry(tab, sh, tid);
  }
  __syncthreads();
}

// ---------------------------------------------------------------- chunk ownership
// The full chunks of one run of same-kind tensors, [f0, f1), are split over the grid:
// grid-stride (block b owns f0' + b + kG, the whole grid streams one window of memory)
// or contiguous ranges (block b owns [f0 + (f1-f0)*b/G, f0 + (f1-f0)*(b+1)/G)).
// Both table forms use the grid-stride split: for the 1152-tensor list of 4-64-chunk
// tensors, contiguous ranges per block (a block then changes tensor only at tensor
// boundaries) ran 460 us against 360 us, as for large tensors the chip streaming one
// window of memory at a time wins.
struct Owned {
  int64_t first;  // first owned chunk (>= limit: none)
  int64_t limit;  // owned chunks are < limit
  int64_t step;
};

template <bool kContig>
__device__ __forceinline__ Owned owned_chunks(int64_t f0, int64_t f1) {
  const int64_t G = gridDim.x, b = blockIdx.x;
  Owned o;
  if constexpr (!kContig) {
    o.first = f0 + ((b - f0 % G) % G + G) % G;
    o.limit = f1;
    o.step = G;
  } else {
    o.first = f0 + (f1 - f0) * b / G;
    o.limit = f0 + (f1 - f0) * (b + 1) / G;
    o.step = 1;
  }
  return o;
}

// Full-chunk range [f0, f1) of the run (same-kind tensors) holding table entry t.
template <class Tab>
__device__ __forceinline__ void run_bounds(const Tab& tab, int t, int64_t& f0, int64_t& f1) {
  const int kind = entry_kind(tab.e[t]);
  const int tb = kind > 0 ? tab.run_end[kind - 1] : 0;
  const int te = tab.run_end[kind];
  f0 = tab.e[tb].fbegin;
  f1 = tab.e[te - 1].fbegin + tab.e[te - 1].nfull;
}

// ---------------------------------------------------------------- element-wise units
// Units [g0, g1) of a tensor, one element at a time through the IEEE divide.  Vector
// unit g holds elements head + 8g .. head + 8g + 7; scalar element j (unit n_vec +
// j/8) is tensor element j (head part) or j + 8*n_vec (tail part).
template <bool kBF16, int kFmt, bool kGelu>
__device__ __forceinline__ void elementwise_units(const void* __restrict__ src,
                                                  uint8_t* __restrict__ dst, int64_t head,
                                                  int64_t n_vec, int64_t numel, int64_t g0,
                                                  int64_t g1, float s, uint32_t& acc) {
  const int64_t n_scalar = numel - 8 * n_vec;
  for (int64_t g = g0 + threadIdx.x; g < g1; g += kQBlock) {
    for (int q = 0; q < 8; ++q) {
      int64_t i;
      if (g < n_vec) {
        i = head + 8 * g + q;
      } else {
        const int64_t j = (g - n_vec) * 8 + q;
        if (j >= n_scalar) break;
        i = j < head ? j : j + 8 * n_vec;
      }
      float x;
      if constexpr (kBF16) {
        uint32_t b = ((const uint16_t*)src)[i];
        if constexpr (kGelu) b = gelu_bf16(b);
        x = as_float(b << 16);
        acc = pk_max_u16(acc, b & 0x7FFFu);  // low half of the packed accumulator
      } else {
        x = ((const float*)src)[i];
        const uint32_t mag = as_uint(x) & 0x7FFFFFFFu;
        acc = acc > mag ? acc : mag;
      }
      dst[i] = (uint8_t)code_ieee<kFmt>(x, s);
    }
  }
}

// ---------------------------------------------------------------- phase 1: full chunks
// A chunk is kQChunk consecutive units of one tensor; the full chunks of every tensor
// form one space, and block b owns chunks b, b+G, b+2G, ... (grid-stride: the whole
// grid streams one window of memory at a time).  A chunk is read as passes of kU*kL
// 16-byte loads per thread (one pass per bf16 chunk, two per fp32 chunk) through
// buffer resources based at the chunk.  The next pass's loads -- same chunk, next
// chunk, or the next tensor of the same kind -- are issued before the current pass is
// converted, so a wave's HBM requests stay in flight while it computes and across
// tensor boundaries.  Tensors whose scale is outside the Markstein window are skipped
// here and done element-wise in phase 2.
//
// With `setup`, this is the block's first run: the loads of its first pass are issued
// speculatively (assuming that tensor's scale is in the window) before the per-tensor
// constants are set up, so the block's first HBM requests do not wait for the scale
// loads, the reciprocals and the barrier.
template <bool kBF16, int kFmt, bool kGelu, int kStAux, class Tab, class Sh>
__device__ __forceinline__ void run_full_chunks(const Tab& tab, Sh& sh, int t_begin,
                                                int t_end, bool setup) {
  constexpr int kD = Tab::kPlanned ? kQPlanDepth : kQDepth;  // passes in flight ahead
  constexpr int kL = kBF16 ? 1 : 2;                // 16-byte loads per group
  constexpr int kU = kGelu ? kQGeluPass : kBF16 ? kQPass : kQPass / 2;  // groups per pass
  constexpr int kP = kQUnroll / kU;                // passes per chunk
  static_assert(kQUnroll % kU == 0, "a chunk is a whole number of passes");
  constexpr int esz = kBF16 ? 2 : 4;
  const uint32_t tid = threadIdx.x;

  // first chunk of this block in the run, and the tensor holding it
  int64_t f0, f1;
  run_bounds(tab, t_begin, f0, f1);
  const Owned own = owned_chunks<Tab::kContig>(f0, f1);
  int64_t j = own.first;
  int t = t_begin;
  auto settle = [&](int& tt, int64_t& jj) __attribute__((always_inline)) {  // move (tt, jj) to a chunk this phase does
    while (tt < t_end) {
      const int64_t end = tab.e[tt].fbegin + tab.e[tt].nfull;
      if (jj >= own.limit) {
        tt = t_end;
      } else if (jj >= end) {
        if constexpr (Tab::kPlanned) {
          tt = tab.chunk_entry[jj];  // jj < own.limit <= the run's end: a chunk of the run
        } else {
          ++tt;
        }
      } else if (!sh.win[tt]) {  // skip the tensor: next owned chunk at or after its end
        jj += (end - jj + own.step - 1) / own.step * own.step;
        ++tt;
      } else {
        break;
      }
    }
  };
  // Fields of a tensor the pipeline touches, kept in registers: re-read from the
  // table only when the pipeline moves to another tensor.
  struct TensorView {
    const uint4* in;    // aligned body, 16-byte units
    uint2* out;         // aligned body codes, 8-byte units
    int64_t fbegin;     // first full chunk
    int64_t fend;       // one past the last full chunk
  };
  auto view = [&](int tt) __attribute__((always_inline)) {
    TensorView v;
    v.in = (const uint4*)((const char*)tab.e[tt].src + tab.e[tt].head * esz);
    v.out = (uint2*)(tab.e[tt].dst + tab.e[tt].head);
    v.fbegin = tab.e[tt].fbegin;
    v.fend = v.fbegin + tab.e[tt].nfull;
    return v;
  };

  struct Pass {
    uint4 w[kU][kL];
  };
  // live == false: the same loads through an empty descriptor (no memory access, zeros
  // returned), for a slot past the end of the run.
  auto load_pass = [&](Pass& P, const TensorView& v, int64_t jj, int pp,
                       bool live) __attribute__((always_inline)) {
    const int64_t unit0 = (jj - v.fbegin) * kQChunk + pp * kU * kQBlock;
    const __amdgpu_buffer_rsrc_t rin =
        buffer_rsrc(v.in + unit0 * kL, live ? kU * kQBlock * kL * 16 : 0);
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int l = 0; l < kL; ++l) {
        if constexpr (kQPair)  // unit 2 kQBlock (u / 2) + 2 tid + (u mod 2) of the pass
          P.w[u][l] = buffer_load16(rin, ((2 * tid + (u & 1)) * kL + l) * 16,
                                    (u >> 1) * 2 * kQBlock * kL * 16);
        else  // unit kQBlock u + tid
          P.w[u][l] = buffer_load16(rin, (tid * kL + l) * 16, u * kQBlock * kL * 16);
      }
  };

  // A pipeline slot: a pass position and the view of its tensor.
  struct Slot {
    int t;
    int64_t j;
    int p;
    TensorView v;
  };
  auto advance = [&](const Slot& a) __attribute__((always_inline)) {  // the pass after a (t == t_end: none)
    Slot n = a;
    if (++n.p == kP) {
      n.p = 0;
      n.j += own.step;
      if (n.j >= a.v.fend || n.j >= own.limit) {  // leaving the tensor or the range (rare)
        settle(n.t, n.j);
        if (n.t < t_end) n.v = view(n.t);
      }
    }
    return n;
  };

  // kD passes are in flight ahead of the one being converted, in a ring of kD + 1 pass
  // buffers that the loop below walks with constant indexes (no register copies).  Every
  // pass issues the same loads and stores -- the loads of a slot past the end go through
  // an empty descriptor, and the set-up issues empty stand-ins for the stores of the
  // passes it loads -- so the vmcnt wait the compiler places before each group is the
  // same on every path into it and covers that group's loads only.  (A load under a
  // branch, or a copy of a buffer still being loaded, makes it wait for the passes
  // behind as well.)
  constexpr int kR = kD + 1;
  constexpr int kS = kQPair ? kU / 2 : kU;  // stores per pass
  auto stand_in_stores = [&](const TensorView& v) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t rnull = buffer_rsrc(v.out, 0);
#pragma unroll
    for (int q = 0; q < kS; ++q) {
      if constexpr (kQPair)
        buffer_store16<kStAux>(rnull, tid * 16, q * kQBlock * 16, make_uint2(0, 0), make_uint2(0, 0));
      else
        buffer_store8<kStAux>(rnull, tid * 8, q * kQBlock * 8, make_uint2(0, 0));
    }
  };
  Pass buf[kR];
  Slot pos[kR];
  int ts = t_begin;  // speculative first position: chunk ranges only
  int64_t js = j;
  if (setup) {
    if constexpr (Tab::kPlanned) {
      if (js < own.limit) ts = tab.chunk_entry[js];
    } else {
      while (ts < t_end && js < own.limit && js >= tab.e[ts].fbegin + tab.e[ts].nfull) ++ts;
    }
    if (js >= own.limit) ts = t_end;
    if (ts < t_end) load_pass(buf[0], view(ts), js, 0, true);
    setup_shared(tab, sh);
  }
  settle(t, j);
  if (t >= t_end) return;
  pos[0] = Slot{t, j, 0, view(t)};
  if (!setup) {
    load_pass(buf[0], pos[0].v, pos[0].j, pos[0].p, true);
  } else if (ts != t || js != j) {  // rare: the speculative pass is not this block's first
    // Let the speculative loads land before the reload, so that no path reaches the loop
    // with them in flight (the waits in the loop would then cover them too).
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
    load_pass(buf[0], pos[0].v, pos[0].j, pos[0].p, true);
  }
  stand_in_stores(pos[0].v);
#pragma unroll
  for (int d = 1; d < kD; ++d) {
    pos[d] = pos[d - 1].t < t_end ? advance(pos[d - 1]) : pos[d - 1];
    load_pass(buf[d], pos[d].v, pos[d].j, pos[d].p, pos[d].t < t_end);
    stand_in_stores(pos[d].v);
  }
  float s = uniform(sh.scale[t]), r = uniform(sh.rcp[t]);
  uint32_t xlim = uniform(sh.xlim[t]);
  uint32_t clim = kGelu ? sat_limit_bf16<kFmt>(s) : 0u;
  uint32_t acc = 0;
  // The loop leaves only at the end of the ring.  When a run ends partway round, the
  // rest of the ring runs as dead passes: their loads are empty (zeros), they do no
  // arithmetic, their stores go through an empty descriptor and are dropped, and they
  // flush no amax.  An exit from
  // within the ring would give the loop head a second way in, with that pass's
  // look-ahead loads in flight, and the waits in the loop would have to cover it.
  for (;;) {
    bool more = false;
#pragma unroll
    for (int k = 0; k < kR; ++k) {
      const Slot& c = pos[k];
      const bool real = k == 0 || c.t < t_end;  // the head of the ring is always real
      const Slot& last = pos[(k + kD - 1) % kR];
      Slot& ahead = pos[(k + kD) % kR];
      ahead = last.t < t_end ? advance(last) : last;
      load_pass(buf[(k + kD) % kR], ahead.v, ahead.j, ahead.p, ahead.t < t_end);
      // the next passes' loads are issued; keep them ahead of this pass's arithmetic
      __builtin_amdgcn_sched_barrier(0);
      Pass& cur = buf[k];
      const __amdgpu_buffer_rsrc_t rout =
          buffer_rsrc(c.v.out + (c.j - c.v.fbegin) * kQChunk + c.p * kU * kQBlock,
                      real ? kU * kQBlock * 8 : 0);
      // A dead pass skips the arithmetic (vector ALU only: the memory operations are the
      // same on both sides of this branch) and stores its zero codes through the empty
      // descriptor.
      uint2 o[kU] = {};
      if (real) {
        uint32_t pm = 0;  // pass magnitude max
        if constexpr (kGelu && kQGeluTable) {
          // table lookups; the table holds the patched outputs of non-finite inputs
#pragma unroll
          for (int u = 0; u < kU; ++u) {
            const uint4 x = cur.w[u][0];
            cur.w[u][0] = make_uint4(gelu2_lds(x.x), gelu2_lds(x.y), gelu2_lds(x.z),
                                     gelu2_lds(x.w));
            pm = pk_max_u16(pm, mag8_bf16(cur.w[u][0]));
          }
          // no saturation needed when no |y| of the pass exceeds clim (<= FP8_MAX * s)
          const bool nosat = __builtin_amdgcn_ballot_w64(max_halves(pm) > clim) == 0;
#pragma unroll
          for (int u = 0; u < kU; ++u)
            o[u] = nosat ? codes8_bf16_unsaturated<kFmt>(cur.w[u][0], s, r)
                         : codes8_bf16<kFmt>(cur.w[u][0], s, r);
        } else if constexpr (kGelu) {
          // the direct gelu form unless some input of the pass is <= -9 (wave-uniform)
          uint32_t raw = 0;
#pragma unroll
          for (int u = 0; u < kU; ++u)
            raw = pk_max_u16(raw, pk_max_u16(pk_max_u16(cur.w[u][0].x, cur.w[u][0].y),
                                             pk_max_u16(cur.w[u][0].z, cur.w[u][0].w)));
          const bool direct =
              __builtin_amdgcn_ballot_w64(max_halves(raw) >= kGeluDirectLimit) == 0;
#pragma unroll
          for (int u = 0; u < kU; ++u) {
            // the magnitude max feeds both the amax and the test for NaN outputs
            const uint4 x = cur.w[u][0];
            cur.w[u][0] = direct ? gelu8_direct(x) : gelu8_unpatched(x);
            uint32_t mg = mag8_bf16(cur.w[u][0]);
            if (__builtin_amdgcn_ballot_w64(halves_nan(mg) != 0) != 0) {
              cur.w[u][0] = gelu8_patch(x, cur.w[u][0]);
              mg = mag8_bf16(cur.w[u][0]);
            }
            pm = pk_max_u16(pm, mg);
          }
          // no saturation needed when no |y| of the pass exceeds clim (<= FP8_MAX * s)
          const bool nosat = __builtin_amdgcn_ballot_w64(max_halves(pm) > clim) == 0;
#pragma unroll
          for (int u = 0; u < kU; ++u)
            o[u] = nosat ? codes8_bf16_unsaturated<kFmt>(cur.w[u][0], s, r)
                         : codes8_bf16<kFmt>(cur.w[u][0], s, r);
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          if constexpr (kGelu) {
            // done above
          } else if constexpr (kBF16) {
            const uint32_t mg = mag8_bf16(cur.w[u][0]);
            pm = pk_max_u16(pm, mg);
            o[u] = codes8_bf16<kFmt>(cur.w[u][0], s, r);
          } else {
            const uint32_t m = mag8_f32(cur.w[u][0], cur.w[u][kL - 1]);
            pm = pm > m ? pm : m;
            o[u] = codes8_f32<kFmt>(cur.w[u][0], cur.w[u][kL - 1], s, r);
          }
        }
        if constexpr (kBF16) {
          acc = pk_max_u16(acc, pm);
          if (max_halves(pm) >= xlim) {  // rare: inf/NaN or a quotient far beyond FP8
#pragma unroll
            for (int u = 0; u < kU; ++u)
              if (max_halves(mag8_bf16(cur.w[u][0])) >= xlim)
                o[u] = patch8_bf16<kFmt>(o[u], cur.w[u][0], xlim);
          }
        } else {
          acc = acc > pm ? acc : pm;
          if (pm >= xlim) {
#pragma unroll
            for (int u = 0; u < kU; ++u)
              if (mag8_f32(cur.w[u][0], cur.w[u][kL - 1]) >= xlim)
                o[u] = patch8_f32<kFmt>(o[u], cur.w[u][0], cur.w[u][kL - 1], xlim);
          }
        }
      }
      if constexpr (kQPair) {
        static_assert(kU % 2 == 0, "units pair up within a pass");
#pragma unroll
        for (int q = 0; q < kU / 2; ++q)
          buffer_store16<kStAux>(rout, tid * 16, q * kQBlock * 16, o[2 * q], o[2 * q + 1]);
      } else {
#pragma unroll
        for (int u = 0; u < kU; ++u) buffer_store8<kStAux>(rout, tid * 8, u * kQBlock * 8, o[u]);
      }
      const Slot& nx = pos[(k + 1) % kR];
      more = nx.t < t_end;  // uniform
      if (real && (!more || nx.t != c.t)) {
        flush_amax<kBF16>(acc, sh, c.t);
        acc = 0;
        if (more) {
          s = uniform(sh.scale[nx.t]);
          r = uniform(sh.rcp[nx.t]);
          xlim = uniform(sh.xlim[nx.t]);
          if constexpr (kGelu) clim = sat_limit_bf16<kFmt>(s);
        }
      }
    }
    if (!more) return;
  }
}

// ---------------------------------------------------------------- phase 2
// Per tensor t: this block's full chunks if the scale is outside the window (all
// element-wise), and the tensor's remainder -- the units past its last full chunk:
// aligned groups, then the scalar head/tail -- done by block t mod G.
template <bool kBF16, int kFmt, bool kGelu, class Tab, class Sh>
__device__ __forceinline__ void tensor_rest(const Tab& tab, Sh& sh, int t, bool full = true,
                                            bool rest = true) {
  const QEntry& e = tab.e[t];
  const int64_t G = gridDim.x, b = blockIdx.x;
  const float s = uniform(sh.scale[t]);
  const bool win = uniform(sh.win[t]) != 0;
  uint32_t acc = 0;
  bool touched = false;
  if (full && !win) {
    int64_t f0, f1;
    run_bounds(tab, t, f0, f1);
    const Owned own = owned_chunks<Tab::kContig>(f0, f1);
    // this block's chunks of tensor t, in the same ownership as phase 1
    int64_t jj = own.first;
    if (jj < e.fbegin) jj += (e.fbegin - jj + own.step - 1) / own.step * own.step;
    const int64_t stop = min(own.limit, e.fbegin + e.nfull);
    for (; jj < stop; jj += own.step) {
      const int64_t k = jj - e.fbegin;
      elementwise_units<kBF16, kFmt, kGelu>(e.src, e.dst, e.head, e.n_vec, e.numel,
                                            k * kQChunk, (k + 1) * kQChunk, s, acc);
      touched = true;
    }
  }
  const int64_t u0 = e.nfull * kQChunk;
  if (rest && u0 < e.n_units && t % G == b) {
    touched = true;
    if (win) {
      constexpr int esz = kBF16 ? 2 : 4;
      const uint4* in = (const uint4*)((const char*)e.src + e.head * esz);
      uint2* out = (uint2*)(e.dst + e.head);
      const float r = uniform(sh.rcp[t]);
      const uint32_t xlim = uniform(sh.xlim[t]);
      for (int64_t g = u0 + threadIdx.x; g < e.n_vec; g += kQBlock) {
        uint2 o;
        if constexpr (kBF16) {
          uint4 w = load16(in + g);
          if constexpr (kGelu) w = gelu8_bf16(w);
          o = quant8_bf16<kFmt>(w, s, r, xlim, acc);
        } else {
          o = quant8_f32<kFmt>(load16(in + 2 * g), load16(in + 2 * g + 1), s, r, xlim, acc);
        }
        store8(out + g, o);
      }
      elementwise_units<kBF16, kFmt, kGelu>(e.src, e.dst, e.head, e.n_vec, e.numel,
                                            u0 > e.n_vec ? u0 : e.n_vec, e.n_units, s, acc);
    } else {
      elementwise_units<kBF16, kFmt, kGelu>(e.src, e.dst, e.head, e.n_vec, e.numel, u0,
                                            e.n_units, s, acc);
    }
  }
  if (touched) flush_amax<kBF16>(acc, sh, t);
}

// kSrc: bit 0 = the table holds plain bf16 sources, bit 1 = fp32 sources, bit 2 = bf16
// sources with the gelu prologue.  Each instance keeps its register budget to the
// paths it can meet (the bf16-only one is the common case).
template <int kKind>
struct KindTraits {
  static constexpr bool kGelu = kKind >= 4;
  static constexpr bool kBF16 = kKind != 2 && kKind != 3;
  static constexpr int kFmt = kKind & 1;
  static constexpr int kSrcBit = kGelu ? 4 : kBF16 ? 1 : 2;
};

// Phase 1 for the run of kind kKind, if the instance handles that kind.
template <int kSrc, int kKind, int kStAux, class Tab, class Sh>
__device__ __forceinline__ void phase1_run(const Tab& tab, Sh& sh, int& tb, bool& ready) {
  using T = KindTraits<kKind>;
  const int te = tab.run_end[kKind];
  if constexpr ((kSrc & T::kSrcBit) != 0) {
    if (te > tb) {
      run_full_chunks<T::kBF16, T::kFmt, T::kGelu, kStAux>(tab, sh, tb, te, !ready);
      ready = true;
    }
  }
  tb = te;
}

// Phase 2 for table entry t if its kind is kKind.
template <int kSrc, int kKind, class Tab, class Sh>
__device__ __forceinline__ void phase2_entry(const Tab& tab, Sh& sh, int t, int kind,
                                             bool full = true, bool rest = true) {
  using T = KindTraits<kKind>;
  if constexpr ((kSrc & T::kSrcBit) != 0)
    if (kind == kKind) tensor_rest<T::kBF16, T::kFmt, T::kGelu>(tab, sh, t, full, rest);
}

template <int kSrc, class Tab, class Sh>
__device__ __forceinline__ void phase2_dispatch(const Tab& tab, Sh& sh, int t, bool full,
                                                bool rest) {
  const int kind = entry_kind(tab.e[t]);  // uniform
  phase2_entry<kSrc, 0>(tab, sh, t, kind, full, rest);
  phase2_entry<kSrc, 1>(tab, sh, t, kind, full, rest);
  phase2_entry<kSrc, 2>(tab, sh, t, kind, full, rest);
  phase2_entry<kSrc, 3>(tab, sh, t, kind, full, rest);
  phase2_entry<kSrc, 4>(tab, sh, t, kind, full, rest);
  phase2_entry<kSrc, 5>(tab, sh, t, kind, full, rest);
}

// ---------------------------------------------------------------- appended update
// Counts this block as finished and returns the count before it (block-uniform).  Every
// thread's global writes and atomics -- the amax maxima, and the roll's stores in the
// block that rolls -- are performed before the block counts itself.  kRelease (the block
// that rolled the history, once) also writes the roll back past its XCD's L2 with a
// device-scope release; the block that sees the full count (gridDim.x, the extra count
// coming from that release) acquires at device scope, so its loads of row 0 see the
// roll.  The other blocks order device-scope atomics only, for which waiting for them to
// complete is enough: a device-scope fence would write back and invalidate the XCD's L2
// in every block.  Contains barriers: every thread of the block calls it.
template <bool kRelease, class Sh>
__device__ __forceinline__ uint32_t arrive(uint32_t* counter, Sh& sh) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old =
        kRelease ? __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT)
                 : __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old == gridDim.x) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    sh.last = old;
  }
  __syncthreads();
  return sh.last;
}

// The batched update of u.n tensors ("Implement fused kernel for FP8 scale update": roll
// the history, insert the new amax, select, new scale; the same results as
// amax_and_scale_update_kernel) split in two so that only one memory round trip follows
// the launch's last quantize block.  The roll does not depend on this step's amax: the
// first block to finish its quantize work moves rows [0, H-1) to [1, H) in place and
// leaves each column's maximum over them in row 0, which the roll has freed.  The block
// that finishes last then needs row 0 and the amaxes only.

// The roll, by one block.  Thread t owns column t mod n and every (kQBlock / n)-th
// history row, so consecutive threads touch consecutive columns of a row and each keeps
// its column maximum in a register (one LDS atomic per thread at the end: per-element
// atomics on n slots would serialize).  Destination rows [1, H) are walked from the top
// in chunks of (kQBlock / n) * 32 rows (history 1024 of up to 64 tensors in one chunk,
// one load round trip): a chunk loads its source rows (one row up), a barrier, then
// stores; rows below the chunk are read only by later chunks, so no row is overwritten
// before it is read.  Row 0 then takes the column maxima as amax bits (0 when H == 1).
__device__ void roll_in_block(const QUpdate& u, uint32_t* colmax) {
  constexpr int kR = 32;  // rows per thread per chunk
  const int tid = threadIdx.x;
  const int n = (int)u.n;  // 1 .. kQUpdMaxCols (= kQBlock)
  const int groups = kQBlock / n;
  const int c = tid % n, g = tid / n;
  const bool active = g < groups;
  const int64_t H = u.H, span = (int64_t)groups * kR;
  uint32_t* hist = (uint32_t*)u.hist;
  if (tid < n) colmax[tid] = 0u;
  uint32_t m = 0u;
  for (int64_t d_hi = H; d_hi > 1; d_hi -= span) {
    const int64_t d_lo = d_hi - span > 1 ? d_hi - span : 1;
    // every lane loads (rows outside the chunk read element 0, always present) and the
    // maxima come after all loads are issued: one round trip, no per-load wait
    uint32_t v[kR];
#pragma unroll
    for (int k = 0; k < kR; ++k) {
      const int64_t d = d_lo + g + (int64_t)k * groups;
      v[k] = hist[active && d < d_hi ? (d - 1) * n + c : 0];
    }
#pragma unroll
    for (int k = 0; k < kR; ++k) {
      const int64_t d = d_lo + g + (int64_t)k * groups;
      if (active && d < d_hi) m = m > v[k] ? m : v[k];
    }
    __syncthreads();  // every load of the chunk before any store
#pragma unroll
    for (int k = 0; k < kR; ++k) {
      const int64_t d = d_lo + g + (int64_t)k * groups;
      if (active && d < d_hi) hist[d * n + c] = v[k];
    }
  }
  __syncthreads();  // colmax zeroed (and every chunk's loads done) before the maxima go in
  if (active && m != 0u) atomicMax(&colmax[c], m);
  __syncthreads();
  if (tid < n) hist[tid] = colmax[tid];
}

// The rest, by the block that finishes last (after the roll and every block's amax
// atomics): thread t < n selects from row 0's column maximum and the new amax (read with
// device-scope atomic loads), writes the amax into row 0, the new scale and its inverse,
// and resets the amax if asked.
__device__ void finish_in_block(const QUpdate& u) {
  const int tid = threadIdx.x;
  if (tid < (int)u.n) {
    // each loading wavefront acquires for itself: its L1 and L2 lines of the history
    // are dropped before row 0 is read
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    uint32_t* hist = (uint32_t*)u.hist;
    const uint32_t hm = hist[tid];
    const uint32_t ab =
        __hip_atomic_load((uint32_t*)u.amax + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const float s_old = u.scale[tid];
    const uint32_t fmt = u.formats[tid];
    uint32_t sel_bits = hm > ab ? hm : ab;
    if (u.algo == FP8Q_AMAX_MOST_RECENT) sel_bits = ab;
    hist[tid] = ab;
    const float s = next_scale(sel_bits, fmt, s_old, u.margin);
    u.scale[tid] = s;
    u.scale_inv[tid] = 1.0f / s;
    if (u.reset) u.amax[tid] = 0.0f;
  }
  if (tid == 0) __hip_atomic_store(u.counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Phases 1 and 2 of a launch and the block's amax atomics.
template <int kSrc, int kStAux, class Tab, class Sh>
__device__ __forceinline__ void quantize_body(const Tab& tab, Sh& sh) {
  const int n = tab.n;
  const int tid = threadIdx.x;

  // phase 1, one run of same-kind tensors at a time; the first run also sets up sh
  bool ready = false;
  int tb = 0;
  phase1_run<kSrc, 0, kStAux>(tab, sh, tb, ready);
  phase1_run<kSrc, 1, kStAux>(tab, sh, tb, ready);
  phase1_run<kSrc, 2, kStAux>(tab, sh, tb, ready);
  phase1_run<kSrc, 3, kStAux>(tab, sh, tb, ready);
  phase1_run<kSrc, 4, kStAux>(tab, sh, tb, ready);
  phase1_run<kSrc, 5, kStAux>(tab, sh, tb, ready);
  if (!ready) setup_shared(tab, sh);
  // phase 2
  if constexpr (Tab::kPlanned) {
    // many entries: the remainders of tensors b, b + G, ..., and only when some scale is
    // outside the window (rare) a pass over every entry for their full chunks
    for (int t = blockIdx.x; t < n; t += gridDim.x) phase2_dispatch<kSrc>(tab, sh, t, false, true);
    if (sh.any_out)
      for (int t = 0; t < n; ++t)
        if (!uniform(sh.win[t])) phase2_dispatch<kSrc>(tab, sh, t, true, false);
    __syncthreads();
    // one global atomic per tensor this block saw a non-zero |x| in
    for (int t = tid; t < n; t += kQBlock)
      if (sh.amax[t] != 0) amax_accumulate(tab.e[t].amax, sh.amax[t]);
  } else {
    for (int t = 0; t < n; ++t) phase2_dispatch<kSrc>(tab, sh, t, true, true);
    __syncthreads();
    // one global atomic per tensor this block saw a non-zero |x| in
    if (tid < n && sh.amax[tid] != 0) amax_accumulate(tab.e[tid].amax, sh.amax[tid]);
  }
}

template <int kSrc, bool kUpd, bool kStream = false>
__global__ __launch_bounds__(kQBlock) void quantize_amax_kernel(const QTable tab) {
  __shared__ QShared sh;
  if constexpr (kSrc == 4 && kQGeluTable) gelu_table_to_lds();
  quantize_body<kSrc, kStream ? FP8Q_Q_ST_STREAM_AUX : FP8Q_Q_ST_AUX>(tab, sh);
  if constexpr (kUpd) {
    __shared__ uint32_t colmax[kQUpdMaxCols];
    // every block counts once, the one that rolls the history (the first) twice
    uint32_t k = arrive<false>(tab.upd.counter, sh);
    if (k == 0) {
      roll_in_block(tab.upd, colmax);
      k = arrive<true>(tab.upd.counter, sh);
    }
    if (k == gridDim.x) finish_in_block(tab.upd);
  }
}

// A planned table of up to kQPlanMaxEntries tensors (fp8_multi_quantize_amax_planned).
template <int kSrc, bool kStream = false>
__global__ __launch_bounds__(kQBlock) void quantize_amax_planned_kernel(const QPlanTable tab) {
  __shared__ QSharedT<kQPlanMaxEntries> sh;
  quantize_body<kSrc, kStream ? FP8Q_Q_ST_STREAM_AUX : FP8Q_Q_ST_AUX>(tab, sh);
}

// ---------------------------------------------------------------- host side
static int validate_entry(const fp8q_tensor& t) {
  if (t.numel < 0) return FP8Q_EINVAL;
  if (t.src_dtype != FP8Q_BF16 && t.src_dtype != FP8Q_F32) return FP8Q_EINVAL;
  if (t.format != FP8Q_E4M3 && t.format != FP8Q_E5M2) return FP8Q_EINVAL;
  if (t.scale == nullptr || t.amax == nullptr) return FP8Q_EINVAL;
  if (t.numel > 0 && (t.src == nullptr || t.dst == nullptr)) return FP8Q_EINVAL;
  return FP8Q_OK;
}

// Split one tensor into aligned body and scalar head/tail.
static void plan_entry(const fp8q_tensor& t, bool gelu, QEntry* e) {
  const int64_t esz = t.src_dtype == FP8Q_BF16 ? 2 : 4;
  const uintptr_t s = (uintptr_t)t.src, d = (uintptr_t)t.dst;
  int64_t head = -1;
  for (int64_t h = 0; h < 8; ++h)
    if ((s + h * esz) % 16 == 0 && (d + h) % 8 == 0) {
      head = h;
      break;
    }
  e->src = t.src;
  e->dst = t.dst;
  e->scale = t.scale;
  e->amax = (uint32_t*)t.amax;
  e->numel = t.numel;
  e->dtype = t.src_dtype;
  e->fmt = t.format;
  e->gelu = gelu ? 1 : 0;
  e->pad = 0;
  if (head < 0 || t.numel < head + 8) {  // no aligned body: all elements scalar
    e->head = t.numel;
    e->n_vec = 0;
  } else {
    e->head = head;
    e->n_vec = (t.numel - head) / 8;
  }
  e->n_units = e->n_vec + ceil_div(t.numel - 8 * e->n_vec, 8);
  e->nfull = e->n_vec / kQChunk;
}

// Build the gelu table on the current device before its first gelu launch: one small
// kernel on `stream`, then a synchronisation of `stream` (once per device and process),
// so that launches on any stream find it complete.
static int ensure_gelu_table(hipStream_t stream) {
  static std::atomic<bool> ready[64];
  static std::mutex lock;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return FP8Q_EHIP;
  if (ready[dev].load(std::memory_order_acquire)) return FP8Q_OK;
  std::lock_guard<std::mutex> g(lock);
  if (ready[dev].load(std::memory_order_relaxed)) return FP8Q_OK;
  hipLaunchKernelGGL(gelu_table_kernel, dim3(256), dim3(256), 0, stream);
  if (hipGetLastError() != hipSuccess) return FP8Q_EHIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return FP8Q_EHIP;
  ready[dev].store(true, std::memory_order_release);
  return FP8Q_OK;
}

// Launch one table.  `start`/`stop` (may be null): events that take the start and stop
// time of this kernel's own dispatch (hipExtLaunchKernel), for profiling.  *launched
// tells whether a kernel was enqueued (a table of empty tensors enqueues nothing).
static int launch_table(QTable* tab, bool upd, hipStream_t stream, hipEvent_t start,
                        hipEvent_t stop, bool* launched) {
  *launched = false;
  int64_t units = 0;
  for (int i = 0; i < tab->n; ++i) units += tab->e[i].n_units;
  if (units == 0) return FP8Q_OK;
  int cus = 0;
  int st = current_device_cus(&cus);
  if (st != FP8Q_OK) return st;
  int src_kinds = 0;
  for (int i = 0; i < tab->n; ++i)
    src_kinds |= tab->e[i].gelu ? 4 : tab->e[i].dtype == FP8Q_BF16 ? 1 : 2;
  // tables hold either plain entries (any mix of bf16 and fp32) or gelu entries only
  // codes beyond the Infinity Cache's size are stored non-temporally (plain entries)
  const bool nt = src_kinds != 4 && units * 8 >= kQStreamBytes;
  const void* fn = nullptr;
  if (!upd && !nt)
    fn = src_kinds == 1   ? (const void*)quantize_amax_kernel<1, false>
         : src_kinds == 2 ? (const void*)quantize_amax_kernel<2, false>
         : src_kinds == 3 ? (const void*)quantize_amax_kernel<3, false>
         : src_kinds == 4 ? (const void*)quantize_amax_kernel<4, false>
                          : nullptr;
  else if (!upd)
    fn = src_kinds == 1   ? (const void*)quantize_amax_kernel<1, false, true>
         : src_kinds == 2 ? (const void*)quantize_amax_kernel<2, false, true>
         : src_kinds == 3 ? (const void*)quantize_amax_kernel<3, false, true>
                          : nullptr;
  else if (!nt)
    fn = src_kinds == 1   ? (const void*)quantize_amax_kernel<1, true>
         : src_kinds == 2 ? (const void*)quantize_amax_kernel<2, true>
         : src_kinds == 3 ? (const void*)quantize_amax_kernel<3, true>
                          : nullptr;
  else
    fn = src_kinds == 1   ? (const void*)quantize_amax_kernel<1, true, true>
         : src_kinds == 2 ? (const void*)quantize_amax_kernel<2, true, true>
         : src_kinds == 3 ? (const void*)quantize_amax_kernel<3, true, true>
                          : nullptr;
  if (fn == nullptr) return FP8Q_EINVAL;
  // the gelu instance reads its table from dynamic LDS
  const bool table = src_kinds == 4 && kQGeluTable;
  const size_t smem = table ? (size_t)kQGeluTableBytes : 0;
  if (table) {
    st = ensure_gelu_table(stream);
    if (st != FP8Q_OK) return st;
  }
  // The grid-stride schedule needs every block resident at once: cap the blocks per
  // CU at what the instance's register and LDS use allow.  Per device: the dynamic-LDS
  // attribute is set on each device the instance runs on.
  static std::atomic<int> fit[64][32];
  const int dev = current_device_index();
  if (dev < 0) return FP8Q_EHIP;
  const int inst = src_kinds + (upd ? 8 : 0) + (nt ? 16 : 0);
  int per_cu = fit[dev][inst].load(std::memory_order_relaxed);
  if (per_cu <= 0) {
    if (table && hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)smem) != hipSuccess)
      return FP8Q_EHIP;
    int occ = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, fn, kQBlock, smem) != hipSuccess)
      return FP8Q_EHIP;
    const int want = src_kinds == 4 ? kQGeluBlocksPerCU : kQBlocksPerCU;
    per_cu = occ < want ? (occ > 0 ? occ : 1) : want;
    fit[dev][inst].store(per_cu, std::memory_order_relaxed);
  }
  const int64_t max_blocks = (int64_t)cus * per_cu;
  int64_t blocks = tab->total_full > tab->n ? tab->total_full : tab->n;
  if (blocks > max_blocks) blocks = max_blocks;
  if (blocks < 1) blocks = 1;
  void* args[] = {tab};
  *launched = true;
  if (start == nullptr && stop == nullptr)
    return launch_status(
        hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(kQBlock), args, smem, stream));
  return launch_status(hipExtLaunchKernel(fn, dim3((unsigned)blocks), dim3(kQBlock), args,
                                          smem, stream, start, stop, 0));
}

// Quantize n tensors (with the gelu prologue on every one if `gelu`), at most
// kQMaxEntries per launch.  Optional profiling events: `start` takes the start time of
// the first kernel launched, `stop` the stop time of the last; when no kernel is
// launched both are recorded on the stream, so they still form a valid (empty) interval.
static int validate_entries(const fp8q_tensor* tensors, int n, bool gelu) {
  if (n < 0 || (n > 0 && tensors == nullptr)) return FP8Q_EINVAL;
  for (int i = 0; i < n; ++i) {
    int st = validate_entry(tensors[i]);
    if (st != FP8Q_OK) return st;
    if (gelu && tensors[i].src_dtype != FP8Q_BF16) return FP8Q_EUNSUPPORTED;
  }
  return FP8Q_OK;
}

// With `upd` (validated entries, at most kQMaxEntries, at least one non-empty), the
// single launch also carries the appended update.
static int quantize_entries(const fp8q_tensor* tensors, int n, bool gelu, hipStream_t stream,
                            hipEvent_t start = nullptr, hipEvent_t stop = nullptr,
                            const QUpdate* upd = nullptr) {
  int vst = validate_entries(tensors, n, gelu);
  if (vst != FP8Q_OK) return vst;
  // the stop event goes to the last launch: find the last block of entries with work
  int last_base = -1;
  for (int i = 0; i < n; ++i)
    if (tensors[i].numel > 0) last_base = i / kQMaxEntries * kQMaxEntries;
  bool started = false;
  for (int base = 0; base < n; base += kQMaxEntries) {
    QTable tab;
    tab.n = 0;
    tab.total_full = 0;
    const int end = n < base + kQMaxEntries ? n : base + kQMaxEntries;
    // entries grouped by kind, stable within a kind
    for (int kind = 0; kind < kQKinds; ++kind) {
      for (int i = base; i < end; ++i) {
        const int k = gelu ? 4 + tensors[i].format : tensors[i].src_dtype * 2 + tensors[i].format;
        if (k != kind) continue;
        QEntry& e = tab.e[tab.n++];
        plan_entry(tensors[i], gelu, &e);
        e.fbegin = tab.total_full;
        tab.total_full += e.nfull;
      }
      tab.run_end[kind] = tab.n;
    }
    tab.upd = upd != nullptr ? *upd : QUpdate{};
    bool launched = false;
    int st = launch_table(&tab, upd != nullptr, stream, started ? nullptr : start,
                          base == last_base ? stop : nullptr, &launched);
    if (st != FP8Q_OK) return st;
    started = started || launched;
  }
  if (last_base < 0) {  // nothing launched
    if (start != nullptr && hipEventRecord(start, stream) != hipSuccess) return FP8Q_EHIP;
    if (stop != nullptr && hipEventRecord(stop, stream) != hipSuccess) return FP8Q_EHIP;
  }
  return FP8Q_OK;
}

// ---------------------------------------------------------------- planned tables
// What fp8_multi_quantize_plan records in the caller's fp8q_plan (opaque to the caller).
struct PlanRec {
  const QEntry* table;  // the planned entries, in the caller's device workspace
  const int32_t* chunk_entry;  // after them: the entry of every full chunk
  int64_t total_full;
  int64_t units;        // all units of all entries (0: nothing to launch)
  int32_t n;
  int32_t src_kinds;    // bit 0: bf16 sources, bit 1: fp32 sources
  int32_t run_end[kQKinds];
  uint32_t magic;
};
static_assert(sizeof(PlanRec) <= sizeof(fp8q_plan), "the plan record fits the descriptor");
constexpr uint32_t kPlanMagic = 0x51385046u;
constexpr int kPlanChunk = 128;  // entries staged on the host per copy
constexpr int kMapChunk = 4096;  // chunk-map words staged on the host per copy

static int64_t entries_bytes(int n) { return ((int64_t)n * (int64_t)sizeof(QEntry) + 15) / 16 * 16; }

// Workspace bytes of a plan of these (validated) entries: the entries, then one int32
// per full chunk.
static int64_t plan_bytes(const fp8q_tensor* tensors, int n) {
  if (n <= 0) return 0;
  int64_t full = 0;
  for (int i = 0; i < n; ++i) {
    QEntry e;
    plan_entry(tensors[i], false, &e);
    full += e.nfull;
  }
  return entries_bytes(n) + 4 * full;
}

// Validate and plan n entries (grouped by kind, stable within a kind, as in QTable), copy
// the planned entries into the device workspace and fill *rec.  The copies come from host
// memory (staged kPlanChunk entries at a time on the stack), which HIP performs
// synchronously: the call returns with the table in place.
static int build_plan(const fp8q_tensor* tensors, int n, void* workspace, int64_t bytes,
                      PlanRec* rec, hipStream_t stream) {
  int st = validate_entries(tensors, n, false);
  if (st != FP8Q_OK) return st;
  if (n > kQPlanMaxEntries) return FP8Q_EUNSUPPORTED;
  if (n > 0 && (workspace == nullptr || (uintptr_t)workspace % 16 != 0 ||
                bytes < plan_bytes(tensors, n)))
    return FP8Q_EINVAL;
  int16_t order[kQPlanMaxEntries];  // output position -> input index
  int32_t count[kQKinds] = {};
  for (int i = 0; i < n; ++i) ++count[tensors[i].src_dtype * 2 + tensors[i].format];
  int32_t pos[kQKinds];
  for (int k = 0, at = 0; k < kQKinds; ++k) {
    pos[k] = at;
    at += count[k];
    rec->run_end[k] = at;
  }
  for (int i = 0; i < n; ++i) order[pos[tensors[i].src_dtype * 2 + tensors[i].format]++] = (int16_t)i;
  QEntry stage[kPlanChunk];
  rec->total_full = 0;
  rec->units = 0;
  rec->src_kinds = 0;
  for (int p0 = 0; p0 < n; p0 += kPlanChunk) {
    const int m = n - p0 < kPlanChunk ? n - p0 : kPlanChunk;
    for (int j = 0; j < m; ++j) {
      const fp8q_tensor& t = tensors[order[p0 + j]];
      plan_entry(t, false, &stage[j]);
      stage[j].fbegin = rec->total_full;
      rec->total_full += stage[j].nfull;
      rec->units += stage[j].n_units;
      rec->src_kinds |= t.src_dtype == FP8Q_BF16 ? 1 : 2;
    }
    if (hipMemcpyAsync((QEntry*)workspace + p0, stage, m * sizeof(QEntry),
                       hipMemcpyHostToDevice, stream) != hipSuccess)
      return FP8Q_EHIP;
  }
  // the entry of every full chunk, in the planned order
  int32_t* map = (int32_t*)((char*)workspace + entries_bytes(n));
  int32_t words[kMapChunk];
  int m = 0;
  int64_t at = 0;
  for (int p = 0; p < n; ++p) {
    QEntry e;
    plan_entry(tensors[order[p]], false, &e);
    for (int64_t c = 0; c < e.nfull; ++c) {
      words[m++] = p;
      if (m == kMapChunk) {
        if (hipMemcpyAsync(map + at, words, m * 4, hipMemcpyHostToDevice, stream) != hipSuccess)
          return FP8Q_EHIP;
        at += m;
        m = 0;
      }
    }
  }
  if (m > 0 &&
      hipMemcpyAsync(map + at, words, m * 4, hipMemcpyHostToDevice, stream) != hipSuccess)
    return FP8Q_EHIP;
  rec->table = (const QEntry*)workspace;
  rec->chunk_entry = map;
  rec->n = n;
  rec->magic = kPlanMagic;
  return FP8Q_OK;
}

// One launch of the planned kernel over every entry of the plan.
static int launch_planned(const PlanRec& rec, hipStream_t stream) {
  if (rec.units == 0) return FP8Q_OK;
  int cus = 0;
  int st = current_device_cus(&cus);
  if (st != FP8Q_OK) return st;
  // codes beyond the Infinity Cache's size are stored non-temporally (as for argument
  // tables; on the 1152-tensor list, 402 MB of codes: 228.5 -> 220.4 us)
  const bool nt = rec.units * 8 >= kQStreamBytes;
  const void* fn =
      nt ? (rec.src_kinds == 1   ? (const void*)quantize_amax_planned_kernel<1, true>
            : rec.src_kinds == 2 ? (const void*)quantize_amax_planned_kernel<2, true>
                                 : (const void*)quantize_amax_planned_kernel<3, true>)
         : (rec.src_kinds == 1   ? (const void*)quantize_amax_planned_kernel<1>
            : rec.src_kinds == 2 ? (const void*)quantize_amax_planned_kernel<2>
                                 : (const void*)quantize_amax_planned_kernel<3>);
  static std::atomic<int> fit[64][8];
  const int dev = current_device_index();
  if (dev < 0) return FP8Q_EHIP;
  const int inst = (rec.src_kinds & 3) + (nt ? 4 : 0);
  int per_cu = fit[dev][inst].load(std::memory_order_relaxed);
  if (per_cu <= 0) {
    int occ = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, fn, kQBlock, 0) != hipSuccess)
      return FP8Q_EHIP;
    per_cu = occ < kQPlanBlocksPerCU ? (occ > 0 ? occ : 1) : kQPlanBlocksPerCU;
    fit[dev][inst].store(per_cu, std::memory_order_relaxed);
  }
  const int64_t max_blocks = (int64_t)cus * per_cu;
  int64_t blocks = rec.total_full > rec.n ? rec.total_full : rec.n;
  if (blocks > max_blocks) blocks = max_blocks;
  if (blocks < 1) blocks = 1;
  QPlanTable tab;
  tab.e = rec.table;
  tab.chunk_entry = rec.chunk_entry;
  tab.total_full = rec.total_full;
  tab.n = rec.n;
  for (int k = 0; k < kQKinds; ++k) tab.run_end[k] = rec.run_end[k];
  void* args[] = {&tab};
  return launch_status(hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(kQBlock), args, 0, stream));
}

// ---------------------------------------------------------------- allocation-free plans
// fp8_multi_quantize_amax_noalloc keeps its plan in this file-scope device array instead
// of a caller's workspace: up to kQPlanMaxEntries entries and kScratchMapWords full chunks
// (2^18 chunks of 16384 elements: 4.3 G elements).  Each device holds its own copy for the
// life of the process; host code reaches it only through the address hipGetSymbolAddress
// returns for the current device (the array's name in host code is not a device address).
constexpr int64_t kScratchMapWords = (int64_t)1 << 18;
constexpr int64_t kScratchBytes =
    ((int64_t)kQPlanMaxEntries * (int64_t)sizeof(QEntry) + 15) / 16 * 16 + 4 * kScratchMapWords;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// The current device's address of `scratch`, looked up once per device.
static int scratch_address(void** out) {
  static std::atomic<void*> cache[64];
  static std::mutex lock;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return FP8Q_EHIP;
  void* p = cache[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> g(lock);
    p = cache[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
        return FP8Q_EHIP;
      cache[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return FP8Q_OK;
}

}  // namespace fp8q

using namespace fp8q;

extern "C" int fp8_multi_quantize_amax_noalloc(const fp8q_tensor* tensors, int n,
                                               void* stream) {
  int st = validate_entries(tensors, n, false);
  if (st != FP8Q_OK) return st;
  if (n > kQPlanMaxEntries) return FP8Q_EUNSUPPORTED;
  if (n == 0) return FP8Q_OK;
  if ((plan_bytes(tensors, n) - entries_bytes(n)) / 4 > kScratchMapWords) return FP8Q_EUNSUPPORTED;
  void* ptr = nullptr;
  st = scratch_address(&ptr);
  if (st != FP8Q_OK) return st;
  PlanRec rec{};
  st = build_plan(tensors, n, ptr, kScratchBytes, &rec, (hipStream_t)stream);
  if (st != FP8Q_OK) return st;
  return launch_planned(rec, (hipStream_t)stream);
}

extern "C" int fp8_multi_quantize_amax(const fp8q_tensor* tensors, int n, void* stream) {
  return quantize_entries(tensors, n, false, (hipStream_t)stream);
}

extern "C" int64_t fp8_multi_quantize_plan_bytes(const fp8q_tensor* tensors, int n) {
  const int st = validate_entries(tensors, n, false);
  if (st != FP8Q_OK) return st;
  if (n > kQPlanMaxEntries) return FP8Q_EUNSUPPORTED;
  return plan_bytes(tensors, n);
}

extern "C" int fp8_multi_quantize_plan(const fp8q_tensor* tensors, int n, void* workspace,
                                       int64_t workspace_bytes, fp8q_plan* plan, void* stream) {
  if (plan == nullptr) return FP8Q_EINVAL;
  PlanRec rec{};
  const int st = build_plan(tensors, n, workspace, workspace_bytes, &rec, (hipStream_t)stream);
  if (st != FP8Q_OK) return st;
  *plan = fp8q_plan{};
  memcpy(plan, &rec, sizeof(rec));
  return FP8Q_OK;
}

extern "C" int fp8_multi_quantize_amax_planned(const fp8q_plan* plan, void* stream) {
  if (plan == nullptr) return FP8Q_EINVAL;
  PlanRec rec;
  memcpy(&rec, plan, sizeof(rec));
  if (rec.magic != kPlanMagic || rec.n < 0 || rec.n > kQPlanMaxEntries ||
      (rec.n > 0 && rec.table == nullptr))
    return FP8Q_EINVAL;
  return launch_planned(rec, (hipStream_t)stream);
}

extern "C" int fp8_multi_quantize_amax_timed(const fp8q_tensor* tensors, int n, void* stream,
                                             void* start_event, void* stop_event) {
  return quantize_entries(tensors, n, false, (hipStream_t)stream, (hipEvent_t)start_event,
                          (hipEvent_t)stop_event);
}

extern "C" int fp8_quantize_amax_and_update(const fp8q_tensor* tensors, int n_tensors,
                                            float* amax, float* amax_history, float* scale,
                                            float* scale_inv, const uint8_t* formats, int64_t n,
                                            int64_t history_len, int algo, int margin,
                                            int reset_amax, uint32_t* workspace, void* stream,
                                            void* start_event, void* stop_event) {
  // everything is validated before anything is enqueued
  int st = validate_entries(tensors, n_tensors, false);
  if (st != FP8Q_OK) return st;
  st = validate_update(amax, amax_history, scale, scale_inv, formats, n, history_len, algo,
                       margin);
  if (st != FP8Q_OK) return st;
  if (workspace == nullptr) return FP8Q_EINVAL;
  bool any = false;
  for (int i = 0; i < n_tensors; ++i) any = any || tensors[i].numel > 0;
  const bool fuse = n > 0 && any && n_tensors <= kQMaxEntries && n <= kQUpdMaxCols &&
                    history_len <= kQUpdMaxElems / n;
  hipStream_t s = (hipStream_t)stream;
  if (fuse) {
    QUpdate u{amax, amax_history, scale, scale_inv, formats, workspace, n, history_len,
              algo, margin, reset_amax ? 1 : 0, 0};
    return quantize_entries(tensors, n_tensors, false, s, (hipEvent_t)start_event,
                            (hipEvent_t)stop_event, &u);
  }
  // the same results as two launches
  st = quantize_entries(tensors, n_tensors, false, s, (hipEvent_t)start_event,
                        (hipEvent_t)stop_event);
  if (st != FP8Q_OK) return st;
  return fp8_amax_and_scale_update(amax, amax_history, scale, scale_inv, formats, n,
                                   history_len, algo, margin, reset_amax, stream);
}

static fp8q_tensor single_entry(const void* src, int src_dtype, uint8_t* dst, int64_t numel,
                                int format, const float* scale, float* amax) {
  fp8q_tensor t;
  t.src = src;
  t.dst = dst;
  t.numel = numel;
  t.src_dtype = src_dtype;
  t.format = format;
  t.scale = scale;
  t.amax = amax;
  return t;
}

extern "C" int fp8_quantize_amax(const void* src, int src_dtype, uint8_t* dst, int64_t numel,
                                 int format, const float* scale, float* amax, void* stream) {
  const fp8q_tensor t = single_entry(src, src_dtype, dst, numel, format, scale, amax);
  return quantize_entries(&t, 1, false, (hipStream_t)stream);
}

extern "C" int fp8_gelu_quantize_amax(const void* src, int src_dtype, uint8_t* dst,
                                      int64_t numel, int format, const float* scale,
                                      float* amax, void* stream) {
  const fp8q_tensor t = single_entry(src, src_dtype, dst, numel, format, scale, amax);
  return quantize_entries(&t, 1, true, (hipStream_t)stream);
}
