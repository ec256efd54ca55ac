/*
 * fp8q.h -- C ABI of the MI355X (gfx950) FP8 delayed-scaling library libfp8q.so.
 *
 * The library implements the memory-bound hot path of FP8 training with delayed
 * scaling:
 *   - quantize: each element of a wide (bf16 or fp32) tensor is divided by the
 *     scale of the previous step, saturated to the FP8 range and cast to E4M3 or
 *     E5M2, while max|x| of the same tensor is reduced in the same pass
 *     ("Fusion of Fp8 quantization and amax reduction kernels", openxla/xla issue
 *     7432: the quantize and the amax passes read the same tensor and are fused);
 *   - the amax-history scale update for many tensors in one launch ("Implement
 *     fused kernel for FP8 scale update", TransformerEngine PR 593: roll the amax
 *     history in place, take the amax from it, compute the new scale);
 *   - dequantize (FP8 code times scale);
 *   - the quantize fused into the kernel that produces the tensor, for the MLP's gelu
 *     activation and the LayerNorm in front of it (the reproducer's transformer block
 *     in that issue), so the bf16 activation is never written;
 *   - the consumer: an FP8 matrix product with per-tensor scales on the matrix cores.
 * The formulas are those of "User Guide on Native XLA-FP8" (NVIDIA JAX-Toolbox),
 * section "JAX": quantize A_fp8 = cast(A / A_scale); dequantize cast_up(a_fp8) *
 * a_scale; delayed scaling A_scale = max|A| / E4M3_MAX.
 *
 * Conventions shared by every entry point
 *   Pointers.   Every pointer except `tensors` of fp8_multi_quantize_amax is a
 *               DEVICE pointer on the current HIP device.  The caller owns all
 *               memory; the library allocates nothing, frees nothing and keeps no
 *               per-call state, so calls are reentrant and thread-safe.
 *   Streams.    `stream` is a hipStream_t (NULL = the null stream).  Every call only
 *               enqueues work on it and returns; nothing synchronises and nothing is
 *               copied device-to-host.
 *   Errors.     Arguments are validated on the host before anything is enqueued; a
 *               negative status is returned and nothing is enqueued.  A failed
 *               launch returns FP8Q_EHIP.  Faults during kernel execution surface at
 *               the caller's next synchronisation, as in HIP.
 *   Layout.     Tensors are dense and contiguous, element i at byte offset
 *               i * sizeof(element).  The quantize, dequantize and update entry points
 *               accept any alignment: when source and destination are aligned alike
 *               the body runs with 16-byte vector loads, otherwise (or for the few
 *               head/tail elements) element-wise.  The LayerNorm-fused quantize and
 *               the GEMM state their alignment requirements.
 *   Aliasing.   Sources and destinations of one call must not overlap.
 *   Numerics.   Binary32 throughout: the quotient x/scale is one IEEE division
 *               rounded to nearest even, then saturated to +-FP8_MAX (448 for E4M3,
 *               57344 for E5M2), then rounded to nearest even into the FP8 format,
 *               FP8 subnormals and the sign of zero kept.  A NaN quotient becomes
 *               0x7F (E4M3 and E5M2 NaN) with the sign bit of x.  +-inf saturates.
 */
#ifndef FP8Q_H
#define FP8Q_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* FP8 formats ("User Guide on Native XLA-FP8", opening paragraphs: E4M3 for the
 * forward pass, E5M2 for gradients).  OCP encodings: E4M3 = float8_e4m3fn (bias 7,
 * no inf, max 448), E5M2 = float8_e5m2 (bias 15, inf, max 57344). */
enum { FP8Q_E4M3 = 0, FP8Q_E5M2 = 1 };

/* Wide element types (quantize source, dequantize destination). */
enum { FP8Q_BF16 = 0, FP8Q_F32 = 1 };

/* How the scale update picks the amax ("Implement fused kernel for FP8 scale
 * update": the amax comes from the history).  MAX: the largest entry of the rolled
 * history window; MOST_RECENT: the amax just inserted. */
enum { FP8Q_AMAX_MAX = 0, FP8Q_AMAX_MOST_RECENT = 1 };

/* Status codes. */
enum {
  FP8Q_OK = 0,
  FP8Q_EINVAL = -1,       /* invalid argument; nothing was enqueued            */
  FP8Q_EUNSUPPORTED = -2, /* valid request this library cannot serve            */
  FP8Q_EHIP = -3          /* a HIP runtime call or kernel launch failed          */
};

/* One entry of a multi-tensor quantize call. */
typedef struct fp8q_tensor {
  const void* src;    /* device; numel elements of src_dtype                          */
  uint8_t* dst;       /* device; numel FP8 codes                                      */
  int64_t numel;      /* >= 0; 0 is a no-op for this entry (amax left unchanged)      */
  int32_t src_dtype;  /* FP8Q_BF16 | FP8Q_F32                                         */
  int32_t format;     /* FP8Q_E4M3 | FP8Q_E5M2                                        */
  const float* scale; /* device, 1 float: the previous step's scale (the divisor)    */
  float* amax;        /* device, 1 float: max-accumulated with max|src|; entries may
                         share one amax                                               */
} fp8q_tensor;

/*
 * fp8_quantize_amax -- fused quantize + amax of one tensor.
 *   dst[i]  = FP8(saturate(RN32(src[i] / *scale)))            for i in [0, numel)
 *   *amax   = max(*amax, max_i |src[i]|)
 * ("User Guide on Native XLA-FP8", section "JAX": quantization divides by the scale
 * of the previous step and casts; the amax is max|A| of the unscaled tensor.
 * "Fusion of Fp8 quantization and amax reduction kernels": both in one pass.)
 * The amax is max-accumulated ("Gradient accumulation of FP8 params": FP8 meta
 * combines with max): it is compared by bit pattern with the sign cleared, so a NaN
 * input propagates into amax, and the caller zeroes *amax before the first call of a
 * step (or lets fp8_amax_and_scale_update with reset_amax do it).  *amax must hold a
 * non-negative value or NaN.
 *   src_dtype  FP8Q_BF16 or FP8Q_F32.   format  FP8Q_E4M3 or FP8Q_E5M2.
 *   numel      >= 0; 0 enqueues nothing.  src, dst non-NULL when numel > 0; scale and
 *              amax non-NULL always.
 * Returns FP8Q_OK, FP8Q_EINVAL or FP8Q_EHIP.
 */
int fp8_quantize_amax(const void* src, int src_dtype, uint8_t* dst, int64_t numel,
                      int format, const float* scale, float* amax, void* stream);

/*
 * fp8_multi_quantize_amax -- fp8_quantize_amax over a list of tensors in one
 * kernel launch per 32 entries (the per-op launch overhead of many small GPU ops is
 * what "Implement fused kernel for FP8 scale update" profiles; batching across
 * layers is the remedy it names).  Each entry follows fp8_quantize_amax exactly;
 * entries may mix dtypes and formats and may share an amax.
 *   tensors    HOST array of n entries, read during the call only.
 *   n          >= 0; 0 enqueues nothing.
 * Every entry is validated before anything is enqueued.
 * Returns FP8Q_OK, FP8Q_EINVAL or FP8Q_EHIP.
 */
int fp8_multi_quantize_amax(const fp8q_tensor* tensors, int n, void* stream);

/*
 * A plan: a list of up to 2048 quantize entries laid out once in a caller-owned device
 * workspace, so that every later call quantizes the whole list in ONE kernel launch with
 * no per-call host work beyond the launch (the per-call launches of many small ops are
 * what "Implement fused kernel for FP8 scale update" profiles; a list longer than the 32
 * entries one launch of fp8_multi_quantize_amax takes would otherwise need several
 * launches).  The plan holds the entries' pointers and sizes; the tensors' contents and
 * their scales and amaxes are read when the planned launch runs, so one plan serves
 * every step while the buffers stay in place.  Opaque to the caller; filled by
 * fp8_multi_quantize_plan.
 */
typedef struct fp8q_plan {
  uint64_t opaque[16];
} fp8q_plan;

/* Bytes of device workspace the plan of these n entries needs: 96 per entry (rounded
 * up to a multiple of 16) plus 4 per full chunk of 16384 aligned elements (0 for n ==
 * 0).  Negative: the status the plan call would return for this list (FP8Q_EINVAL,
 * FP8Q_EUNSUPPORTED). */
int64_t fp8_multi_quantize_plan_bytes(const fp8q_tensor* tensors, int n);

/*
 * fp8_multi_quantize_plan -- validate a list of n quantize entries (as
 * fp8_multi_quantize_amax) and lay it out in `workspace` for
 * fp8_multi_quantize_amax_planned.  The layout is copied from host memory with
 * hipMemcpyAsync on `stream`, which HIP performs synchronously for host memory that is
 * not page-locked: the call returns with the workspace written, after the work enqueued
 * before it on the stream.  A set-up call, not one per step; not for graph capture.
 *   tensors    HOST array of n entries (bf16 or fp32 sources; no gelu), read during the
 *              call only.
 *   n          0 .. 2048 (more: FP8Q_EUNSUPPORTED).
 *   workspace  DEVICE memory of at least fp8_multi_quantize_plan_bytes(tensors, n) bytes,
 *              16-byte aligned, caller-owned; it must stay allocated and unchanged while
 *              the plan is in use, and not be rewritten while a planned launch reading
 *              it may still run.  (NULL allowed when n == 0.)
 *   plan       HOST descriptor, filled on success.
 * Returns FP8Q_OK, FP8Q_EINVAL, FP8Q_EUNSUPPORTED or FP8Q_EHIP.
 */
int fp8_multi_quantize_plan(const fp8q_tensor* tensors, int n, void* workspace,
                            int64_t workspace_bytes, fp8q_plan* plan, void* stream);

/*
 * fp8_multi_quantize_amax_planned -- fp8_multi_quantize_amax over every entry of a plan,
 * in one kernel launch (none when every entry is empty).  Same results as
 * fp8_multi_quantize_amax on the planned list.  Asynchronous: only enqueues the launch.
 *   plan       HOST descriptor filled by fp8_multi_quantize_plan.
 * Returns FP8Q_OK, FP8Q_EINVAL (a descriptor that no plan call filled) or FP8Q_EHIP.
 */
int fp8_multi_quantize_amax_planned(const fp8q_plan* plan, void* stream);

/*
 * fp8_multi_quantize_amax_noalloc -- for callers that cannot allocate device memory
 * (code under graph capture set-up, tight serving loops, harnesses that forbid
 * hipMalloc): fp8_multi_quantize_plan followed by fp8_multi_quantize_amax_planned, with
 * the plan held in a fixed device array of the library instead of a caller's workspace.
 * Same results as fp8_multi_quantize_amax; one launch.  Allocates nothing: the array
 * (1,245,184 bytes per device: 2048 entries and the entries of 2^18 chunks of 16384
 * elements) is part of the library's device code and each device keeps it until the
 * process ends.  Every call on a device rewrites that device's array, so calls that may
 * overlap on one device (different streams, or threads) race; calls in order on one
 * stream do not.  Like fp8_multi_quantize_plan, the call copies the plan from host
 * memory and returns once it is in place (after the work enqueued before it on the
 * stream); not for graph capture.
 *   tensors, n  as fp8_multi_quantize_amax; n <= 2048 and at most 2^18 full chunks of
 *               16384 aligned elements in all (larger lists: FP8Q_EUNSUPPORTED, nothing
 *               enqueued).
 * Returns FP8Q_OK, FP8Q_EINVAL, FP8Q_EUNSUPPORTED or FP8Q_EHIP.
 */
int fp8_multi_quantize_amax_noalloc(const fp8q_tensor* tensors, int n, void* stream);

/*
 * fp8_multi_quantize_amax_timed -- fp8_multi_quantize_amax with profiling events: the
 * same validation, kernels and results, each kernel launched with hipExtLaunchKernel so
 * that the events take the start and stop time of the kernel's own dispatch rather than
 * of a stream position before it (an event recorded on the stream ahead of a launch also
 * spans the dispatch latency).  For measuring the kernel's duration with HIP events.
 *   start_event  hipEvent_t created by the caller with timing enabled, or NULL: takes
 *                the start of the first kernel launched.
 *   stop_event   likewise, or NULL: takes the end of the last kernel launched.
 * When no kernel is launched (n == 0 or every numel == 0) both events are recorded on
 * the stream, an empty interval.  The events remain the caller's.
 * Returns FP8Q_OK, FP8Q_EINVAL or FP8Q_EHIP.
 */
int fp8_multi_quantize_amax_timed(const fp8q_tensor* tensors, int n, void* stream,
                                  void* start_event, void* stop_event);

/*
 * fp8_gelu_quantize_amax -- the activation between the two dense layers of the MLP,
 * quantized in the kernel that produces it: the bf16 pre-activation x is read, the
 * tanh-form gelu is applied, and the result goes through fp8_quantize_amax's quantize
 * and amax without the bf16 activation tensor ever being written
 * ("Fusion of Fp8 quantization and amax reduction kernels": the reproducer's
 * dense -> gelu -> dense MLP, whose activations are quantized and amax-reduced in
 * passes of their own).
 *   y[i]    = RN_bf16(gelu(src[i])),  gelu(x) = x / (1 + exp(-2u)),
 *             u = sqrt(2/pi) * (x + 0.044715 x^3)      (= 0.5 x (1 + tanh u) exactly)
 *   dst[i]  = FP8(saturate(RN32(y[i] / *scale)))
 *   *amax   = max(*amax, max_i |y[i]|)
 * gelu is evaluated in binary32 (exp2 and reciprocal on the hardware units): y[i] is
 * the bf16 rounding of a value within a relative (16 + 4|2u|) * 2^-24 of the exact
 * gelu, so it is the correctly rounded bf16 of gelu(x) except where that lies within
 * this distance of a bf16 rounding midpoint (then it may be the other neighbour).
 * gelu(+inf) = +inf, gelu(-inf) = -0, gelu(NaN) = NaN with the sign of x.
 * The bulk of the tensor reads y from a table of these values for all 65536 bf16
 * inputs, which the library builds on each device, with the same binary32 arithmetic,
 * before the first call on that device runs: that first call launches one extra small
 * kernel on `stream` and synchronizes `stream` once (so it must not be captured into a
 * graph); every later call is one launch.  The table is device memory of the library
 * (128 KB per device, kept until the process ends).
 *   src_dtype  FP8Q_BF16 (FP8Q_F32 returns FP8Q_EUNSUPPORTED).   format  as above.
 *   numel, pointers, alignment, amax accumulation and errors as fp8_quantize_amax.
 * Returns FP8Q_OK, FP8Q_EINVAL, FP8Q_EUNSUPPORTED or FP8Q_EHIP.
 */
int fp8_gelu_quantize_amax(const void* src, int src_dtype, uint8_t* dst, int64_t numel,
                           int format, const float* scale, float* amax, void* stream);

/*
 * fp8_layernorm_quantize_amax -- the LayerNorm in front of the MLP, quantized in the
 * kernel that normalizes: each row of the bf16 input is normalized in registers and
 * its bf16 result goes through fp8_quantize_amax's quantize and amax without being
 * written ("Fusion of Fp8 quantization and amax reduction kernels": the reproducer's
 * transformer block applies nn.LayerNorm() to its input and feeds the result to the
 * MLP's first FP8 dense).  Per row r of `hidden` elements:
 *   mu = mean(x), V = mean((x - mu)^2) (biased), rstd = 1 / sqrt(V + eps)
 *   y[i]    = RN_bf16(gamma[i] * (x[i] - mu) * rstd + beta[i])
 *   dst[i]  = FP8(saturate(RN32(y[i] / *scale)))
 *   *amax   = max(*amax, max over all rows of |y[i]|)
 *   mean[r] = mu, rstd[r] = rstd           (binary32; for the backward pass)
 * Evaluated in binary32: tree sums and a corrected two-pass variance; y[i] is the bf16
 * rounding of a value within (twice its first-order bound)
 *   2^-23 (|gamma| rstd (|d| (L/2 + 7 + L^2 2^-24 A A_d rstd^2) + L A_d + L^2 2^-24 A) + |y|)
 * of the exact one, L = ceil(log2 hidden) + 10, d = x - mu, A = mean|x|, A_d = mean|d|;
 * so it is the correctly rounded bf16 of the exact LayerNorm except within that
 * distance of a bf16 rounding midpoint.  mean and rstd are within a few ulps of the
 * exact values.  A row containing inf or NaN (or with V + eps = 0) gives NaN outputs,
 * written as the positive default NaN (code 0x7F), and NaN mean/rstd.
 *   x          device, rows x hidden bf16, row-major, 16-byte aligned.
 *   x_dtype    FP8Q_BF16 (FP8Q_F32 returns FP8Q_EUNSUPPORTED).
 *   gamma,beta device, hidden binary32 each, or NULL for 1 / 0.
 *   eps        finite, >= 0 (the layer's default is 1e-6).
 *   rows       >= 0.   hidden: a multiple of 8 in [8, 16384] (else FP8Q_EUNSUPPORTED);
 *              rows == 0 or hidden == 0 enqueues nothing.
 *   dst        device, rows x hidden codes, 8-byte aligned (else FP8Q_EUNSUPPORTED).
 *   format, scale, amax as fp8_quantize_amax.
 *   mean,rstd  device, rows binary32 each, or NULL to skip.
 * Returns FP8Q_OK, FP8Q_EINVAL, FP8Q_EUNSUPPORTED or FP8Q_EHIP.
 */
int fp8_layernorm_quantize_amax(const void* x, int x_dtype, const float* gamma,
                                const float* beta, float eps, int64_t rows, int64_t hidden,
                                uint8_t* dst, int format, const float* scale, float* amax,
                                float* mean, float* rstd, void* stream);

/*
 * fp8_gemm -- the consumer of the quantized tensors: an FP8 matrix product with
 * per-tensor scales on the matrix cores ("User Guide on Native XLA-FP8", section "JAX":
 * the FP8 operands are cast up and multiplied by their scales before the dot; the matmul
 * the page names takes two FP8 tensors and two binary32 scalar scales).
 *   C[m][n] = *a_scale * *b_scale * sum_k decode(A[m][k]) * decode(B[n][k])
 * A is M x K and B is N x K, both row-major (K contiguous: a weight stored K x N is
 * quantized from its transpose); C is M x N row-major.  The FP8 products are exact; the
 * gfx950 matrix core sums each aligned group of 8 consecutive products in fixed point
 * 13 bits below the group's largest (smaller products truncate toward zero; measured)
 * and accumulates the group sums in binary32, so before the final rounding to c_dtype
 * (bf16: round to nearest even)
 *   |C - exact| <= (2^-10 G + 2^-24 (ceil(K/8) + 2) S) |sa sb|,
 *   G = sum over k-groups [8q, 8q+8) of max |a_k b_k|,  S = sum_k |a_k b_k|.
 * NaN operands propagate.  K == 0 gives C = 0.
 *   a_format, b_format  FP8Q_E4M3 or FP8Q_E5M2 (any pairing).
 *   M, N, K     >= 0; M == 0 or N == 0 enqueues nothing.  K a multiple of 16 and at most
 *               2^23 (else FP8Q_EUNSUPPORTED).
 *   A, B        device, 16-byte aligned (else FP8Q_EUNSUPPORTED); non-NULL when K > 0.
 *   a_scale, b_scale  device, 1 float each (the delayed-scaling scales of A and B).
 *   C           device, M x N of c_dtype (FP8Q_BF16 or FP8Q_F32), naturally aligned.
 * Returns FP8Q_OK, FP8Q_EINVAL, FP8Q_EUNSUPPORTED or FP8Q_EHIP.
 */
int fp8_gemm(const uint8_t* A, int a_format, const uint8_t* B, int b_format, int64_t M,
             int64_t N, int64_t K, const float* a_scale, const float* b_scale, void* C,
             int c_dtype, void* stream);

/*
 * fp8_dequantize -- y[i] = RN32(decode(src[i]) * *scale), written as fp32, or
 * rounded to nearest even into bf16 ("User Guide on Native XLA-FP8", section "JAX":
 * dequantization casts up and multiplies by the scale).  A NaN result is written as
 * the quiet NaN 0x7FC00000 (bf16 0x7FC0) carrying the sign bit of the code.
 *   format     FP8Q_E4M3 or FP8Q_E5M2.   dst_dtype  FP8Q_BF16 or FP8Q_F32.
 *   numel      >= 0; src, dst non-NULL when numel > 0; scale non-NULL.
 * Returns FP8Q_OK, FP8Q_EINVAL or FP8Q_EHIP.
 */
int fp8_dequantize(const uint8_t* src, int format, void* dst, int dst_dtype, int64_t numel,
                   const float* scale, void* stream);

/*
 * fp8_amax_and_scale_update -- the delayed-scaling update of n tensors, in place,
 * in one launch ("Implement fused kernel for FP8 scale update": history roll,
 * amax selection and scale computation fused, in place; "User Guide on Native
 * XLA-FP8", section "JAX": scale = amax / FP8_MAX).  For every tensor t:
 *   roll      amax_history[h][t] = old amax_history[h-1][t] for h = H-1 .. 1 (the
 *             oldest row H-1 is dropped), amax_history[0][t] = amax[t];
 *   select    sel = max over h of amax_history[h][t] (algo MAX, compared by bit
 *             pattern) or amax[t] (algo MOST_RECENT);
 *   scale     c = RN32(sel / FP8_MAX(formats[t])) * 2^margin (exact power-of-two
 *             scaling); scale[t] = c if sel and c are finite and > 0, otherwise
 *             scale[t] keeps its previous value;
 *   inverse   scale_inv[t] = RN32(1 / scale[t]);
 *   reset     if reset_amax != 0: amax[t] = 0 after it has been read.
 *   amax           device float[n]   (written only when reset_amax != 0)
 *   amax_history   device float[H][n], row-major, row 0 newest; updated in place
 *   scale          device float[n], in: previous scale, out: new scale
 *   scale_inv      device float[n], out
 *   formats        device uint8[n]: 0 = E4M3 (max 448), any other value = E5M2
 *                  (max 57344)
 *   n >= 0 (0 enqueues nothing); history_len >= 1; algo FP8Q_AMAX_MAX or
 *   FP8Q_AMAX_MOST_RECENT; margin in [-126, 126]; history_len * n below 2^29 (a 2 GiB
 *   history; larger: FP8Q_EUNSUPPORTED).  The five arrays must not overlap.
 * Returns FP8Q_OK, FP8Q_EINVAL, FP8Q_EUNSUPPORTED or FP8Q_EHIP.
 */
int fp8_amax_and_scale_update(float* amax, float* amax_history, float* scale,
                              float* scale_inv, const uint8_t* formats, int64_t n,
                              int64_t history_len, int algo, int margin, int reset_amax,
                              void* stream);

/*
 * fp8_quantize_amax_and_update -- one whole delayed-scaling step: exactly
 *   fp8_multi_quantize_amax(tensors, n_tensors, stream);
 *   fp8_amax_and_scale_update(amax, amax_history, scale, scale_inv, formats, n,
 *                             history_len, algo, margin, reset_amax, stream);
 * (same results, bit for bit) in ONE kernel launch when it fits: the quantize pass of
 * "Fusion of Fp8 quantization and amax reduction kernels" and the fused update of
 * "Implement fused kernel for FP8 scale update" share the launch: the history roll runs
 * in the block that finishes its quantize work first (it needs no amax of this step),
 * the rest of the update in the block that finishes last, after every block's amax is
 * accumulated.  This removes the kernel boundary and the second launch between the two
 * passes.
 * The single launch is used when 1 <= n_tensors <= 32, some tensor is non-empty,
 * 1 <= n <= 256 and history_len * n <= 65536; otherwise the call enqueues the two
 * launches above (same results).  The quantize reads each tensor's scale before the
 * update writes `scale`, so the entries' scale/amax pointers may (and normally do)
 * point into scale[] / amax[].
 *   tensors, n_tensors   as fp8_multi_quantize_amax.
 *   amax ... reset_amax  as fp8_amax_and_scale_update.
 *   workspace   DEVICE pointer to one uint32_t (4 bytes, caller-owned), 0 at the first
 *               call; every call leaves it 0.  It counts the finished blocks, so calls
 *               that may run concurrently (different streams) need separate
 *               workspaces.  Required (non-NULL) even when the two-launch form is used.
 *   start_event, stop_event   optional profiling events as in
 *               fp8_multi_quantize_amax_timed (NULL for none); with the two-launch form
 *               they span the quantize kernels only.
 * Every argument is validated before anything is enqueued.
 * Returns FP8Q_OK, FP8Q_EINVAL, FP8Q_EUNSUPPORTED (history as in
 * fp8_amax_and_scale_update) or FP8Q_EHIP.
 */
int fp8_quantize_amax_and_update(const fp8q_tensor* tensors, int n_tensors, float* amax,
                                 float* amax_history, float* scale, float* scale_inv,
                                 const uint8_t* formats, int64_t n, int64_t history_len,
                                 int algo, int margin, int reset_amax, uint32_t* workspace,
                                 void* stream, void* start_event, void* stop_event);

/* Static, human-readable text for a status code. */
const char* fp8_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FP8Q_H */
