/*
 * fp8_oracle.c -- plain CPU oracle for FP8 delayed scaling.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is compiled into liboracle.so, which only
 * tests/, the smoke check and the CPU-baseline leg of bench.py load.  The GPU
 * library shares no code, header, table or constant with it and never calls it.
 *
 * Everything here is the plain definition, element by element, in IEEE binary32
 * where the method fixes binary32 (the scales and the quotient x/scale) and in
 * exact double arithmetic where only exact values are manipulated (decoding FP8
 * codes, locating the nearest FP8 value).  Build: gcc -O2 -ffp-contract=off, no
 * fast-math, so every binary32 operation below is one correctly rounded IEEE op.
 *
 * Sources (the pages):
 *  [NG-intro]  "User Guide on Native XLA-FP8" (NVIDIA JAX-Toolbox), opening
 *              paragraphs: the two FP8 formats E4M3 (float8_e4m3fn) and E5M2
 *              (float8_e5m2); E4M3 for forward tensors, E5M2 for gradients;
 *              quantization scales wide data into the FP8 range, dequantization
 *              scales it back.
 *  [NG-JAX]    same page, section "JAX", second example: quantize divides by the
 *              scale of the previous step then casts to E4M3; dequantize casts up
 *              and multiplies by the scale; the delayed-scaling update sets
 *              scale = max|A| / E4M3_MAX; scales are held in wider types.
 *  [NG-grad]   same page, section "Gradient accumulation of FP8 params": FP8 meta
 *              (amax history, scale) accumulates with max, not with addition.
 *  [XLA-7432]  "Fusion of Fp8 quantization and amax reduction kernels" (openxla/xla
 *              issue 7432): the quantize pass and the amax reduction read the same
 *              tensor and are the two passes being fused.
 *  [TE-593]    "Implement fused kernel for FP8 scale update" (TransformerEngine
 *              PR 593): one update per call that rolls the amax history in place,
 *              takes the amax from the history and computes the new scale.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *  R1 x/scale is one binary32 IEEE round-to-nearest-even division.
 *  R2 the quotient saturates to +-FP8_MAX before the cast (no NaN/inf on overflow).
 *  R3 the cast rounds to nearest, ties to even, keeps FP8 subnormals and the sign
 *     of zero.
 *  R4 a NaN quotient encodes as 0x7F with the sign bit of x.
 *  R5 amax is the max of the unscaled |x|, taken as an unsigned max over the
 *     binary32 bit patterns with the sign cleared, and max-accumulated into the
 *     caller's amax (also by bit pattern).
 *  R6 history layout hist[H][N] row-major, row 0 newest: the roll moves row h-1 to
 *     row h, drops row H-1 and writes the new amax into row 0; the selection then
 *     runs over the rolled window.
 *  R7 scale = RN32(sel / FP8_MAX) * 2^margin; if sel is not finite or not > 0, or
 *     the result is not finite or not > 0, the previous scale is kept.
 *  R8 scale_inv = RN32(1 / scale).
 *  R9 dequantize y = RN32(decode(q) * scale); a NaN result is the quiet NaN
 *     0x7FC00000 carrying the sign bit of the code; bf16 output rounds y to
 *     nearest even.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

enum { ORC_E4M3 = 0, ORC_E5M2 = 1 };
enum { ORC_BF16 = 0, ORC_F32 = 1 };
enum { ORC_AMAX_MAX = 0, ORC_AMAX_MOST_RECENT = 1 };

static uint32_t f2u(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float u2f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* Format parameters of the two OCP formats named in [NG-intro]:
 *   E4M3 (e4m3fn): 4 exponent bits, bias 7, 3 mantissa bits, no infinity,
 *                  S.1111.111 is NaN, so the largest finite is 1.75 * 2^8 = 448.
 *   E5M2:          5 exponent bits, bias 15, 2 mantissa bits, exponent 31 holds
 *                  inf (mantissa 0) and NaN, largest finite 1.75 * 2^15 = 57344. */
static int fmt_mbits(int fmt) { return fmt == ORC_E4M3 ? 3 : 2; }
static int fmt_bias(int fmt) { return fmt == ORC_E4M3 ? 7 : 15; }
float oracle_fp8_max(int fmt) { return fmt == ORC_E4M3 ? 448.0f : 57344.0f; }

/* Decode one FP8 code to its exact value (closed form of the format). */
float oracle_fp8_decode(int fmt, uint8_t code) {
  int sign = code >> 7;
  int mbits = fmt_mbits(fmt), bias = fmt_bias(fmt);
  int efield = (code & 0x7F) >> mbits;
  int m = code & ((1 << mbits) - 1);
  double v;
  if (fmt == ORC_E4M3 && efield == 15 && m == 7) {
    v = NAN;
  } else if (fmt == ORC_E5M2 && efield == 31) {
    v = (m == 0) ? INFINITY : NAN;
  } else if (efield == 0) {
    v = ldexp((double)m, 1 - bias - mbits);                 /* subnormal */
  } else {
    v = ldexp(1.0 + (double)m / (double)(1 << mbits), efield - bias);
  }
  return (float)(sign ? -v : v);
}

/* Encode v (finite with |v| <= FP8_MAX, or NaN) to the nearest FP8 code, ties to
 * the code with an even mantissa, subnormals kept, sign of zero kept (R3). */
uint8_t oracle_fp8_encode(int fmt, float v) {
  uint8_t sign = signbit(v) ? 0x80 : 0x00;
  if (isnan(v)) return (uint8_t)(0x7F | sign);
  int mbits = fmt_mbits(fmt), bias = fmt_bias(fmt), emin = 1 - bias;
  double a = fabs((double)v);
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e);            /* a = f * 2^e with f in [0.5, 1): binade exponent is e-1 */
  e -= 1;
  if (e < emin) e = emin;  /* below the normal range the spacing stays 2^(emin-mbits) */
  double n = nearbyint(ldexp(a, mbits - e));   /* exact scaling, then RNE to integer */
  int code;
  if (n < (double)(1 << mbits)) {
    code = (int)n;                              /* subnormal (or zero) */
  } else {
    if (n == (double)(2 << mbits)) { n /= 2; e += 1; }  /* rounded up into next binade */
    code = ((e + bias) << mbits) | ((int)n - (1 << mbits));
  }
  return (uint8_t)(code | sign);
}

/* One element of the quantize pass [NG-JAX]: (x / scale) cast to FP8 with R1-R4. */
uint8_t oracle_quantize_element(int fmt, float x, float scale) {
  float v = x / scale;
  if (isnan(v)) return (uint8_t)(0x7F | (signbit(x) ? 0x80 : 0x00));
  float mx = oracle_fp8_max(fmt);
  if (v > mx) v = mx;
  if (v < -mx) v = -mx;
  return oracle_fp8_encode(fmt, v);
}

static float load_wide(const void* src, int src_dtype, int64_t i) {
  if (src_dtype == ORC_BF16) return u2f((uint32_t)((const uint16_t*)src)[i] << 16);
  return ((const float*)src)[i];
}

/* Quantize n elements and max-accumulate amax over the same elements
 * ([XLA-7432] pass pair, [NG-JAX] formulas, R5). */
void oracle_quantize_amax(const void* src, int src_dtype, uint8_t* dst, int64_t n,
                          int fmt, float scale, float* amax) {
  uint32_t acc = f2u(*amax);
  for (int64_t i = 0; i < n; ++i) {
    float x = load_wide(src, src_dtype, i);
    dst[i] = oracle_quantize_element(fmt, x, scale);
    uint32_t mag = f2u(x) & 0x7FFFFFFFu;
    if (mag > acc) acc = mag;
  }
  *amax = u2f(acc);
}

/* The amax-history scale update of [TE-593] for n tensors, out of place
 * (hist_in/hist_out are [H][n] row-major; R6-R8; scale formula [NG-JAX]). */
void oracle_amax_and_scale_update(const float* amax, const float* hist_in, float* hist_out,
                                  const float* scale_in, float* scale_out,
                                  float* scale_inv_out, float* amax_out,
                                  const uint8_t* formats, int64_t n, int64_t H,
                                  int algo, int margin, int reset_amax) {
  for (int64_t t = 0; t < n; ++t) {
    hist_out[t] = amax[t];
    for (int64_t h = 1; h < H; ++h) hist_out[h * n + t] = hist_in[(h - 1) * n + t];

    uint32_t sel_bits;
    if (algo == ORC_AMAX_MOST_RECENT) {
      sel_bits = f2u(amax[t]);
    } else {
      sel_bits = 0;
      for (int64_t h = 0; h < H; ++h) {
        uint32_t b = f2u(hist_out[h * n + t]);
        if (b > sel_bits) sel_bits = b;
      }
    }
    float sel = u2f(sel_bits);
    float mx = oracle_fp8_max(formats[t] ? ORC_E5M2 : ORC_E4M3);
    float s = scale_in[t];
    if (isfinite(sel) && sel > 0.0f) {
      float c = sel / mx;
      c = ldexpf(c, margin);
      if (isfinite(c) && c > 0.0f) s = c;
    }
    scale_out[t] = s;
    scale_inv_out[t] = 1.0f / s;
    amax_out[t] = reset_amax ? 0.0f : amax[t];
  }
}

/* Round a binary32 value to bfloat16 (8 significant bits), nearest-even, with
 * overflow to infinity; returns the bf16 bit pattern.  NaN handled by caller. */
static uint16_t round_to_bf16(float y) {
  uint32_t sign = f2u(y) & 0x80000000u;
  double a = fabs((double)y);
  if (isinf(y) || a == 0.0) return (uint16_t)(f2u(y) >> 16);
  int e;
  frexp(a, &e);
  e -= 1;
  if (e < -126) e = -126;
  double r = ldexp(nearbyint(ldexp(a, 7 - e)), e - 7);   /* nearest multiple of 2^(e-7) */
  if (r >= ldexp(1.0, 128)) return (uint16_t)((sign | 0x7F800000u) >> 16);
  return (uint16_t)((sign | f2u((float)r)) >> 16);       /* r has <= 8 significant bits */
}

/* Dequantize [NG-JAX]: decode, multiply by the scale in binary32 (R9). */
void oracle_dequantize(const uint8_t* src, int fmt, void* dst, int dst_dtype, int64_t n,
                       float scale) {
  for (int64_t i = 0; i < n; ++i) {
    float y = oracle_fp8_decode(fmt, src[i]) * scale;
    uint32_t nan_bits = 0x7FC00000u | ((uint32_t)(src[i] & 0x80) << 24);
    if (dst_dtype == ORC_F32) {
      ((float*)dst)[i] = isnan(y) ? u2f(nan_bits) : y;
    } else {
      ((uint16_t*)dst)[i] = isnan(y) ? (uint16_t)(nan_bits >> 16) : round_to_bf16(y);
    }
  }
}

/* Count of elements whose quotient lands beyond +-FP8_MAX (saturated by R2). */
int64_t oracle_count_saturated(const void* src, int src_dtype, int64_t n, int fmt,
                               float scale) {
  int64_t c = 0;
  float mx = oracle_fp8_max(fmt);
  for (int64_t i = 0; i < n; ++i) {
    float v = load_wide(src, src_dtype, i) / scale;
    if (v > mx || v < -mx) ++c;
  }
  return c;
}

/* ------------------------------------------------------------------------------
 * Producer-fused quantize: the FFN activation of the reproducer in "Fusion of Fp8
 * quantization and amax reduction kernels" (test.py: Dense wi -> nn.gelu -> Dense wo,
 * the wo input quantized to FP8).  Readings (pages silent):
 *  G1 gelu is the tanh form 0.5*x*(1 + tanh(sqrt(2/pi)*(x + 0.044715*x^3))) (the default
 *     of the reproducer's nn.gelu), evaluated here in double precision;
 *  G2 the activation tensor is bf16 (the model's dtype): y = RN_bf16(gelu(x)), one
 *     rounding of the double value; gelu(+inf) = +inf, gelu(-inf) = -0, gelu(NaN) = NaN;
 *  G3 y is then quantized and reduced exactly as a bf16 tensor (R1-R5).
 * A single-precision evaluation of gelu carries a small relative error, growing with
 * |2u| through exp (u = sqrt(2/pi)*(x + 0.044715 x^3)); where the double value lies so
 * close to a bf16 rounding midpoint that such an evaluation may round either way, the
 * other neighbour is returned too (`alt`), so a check can accept either. */
static double gelu_tanh_d(double x) {
  if (isnan(x)) return x;
  if (isinf(x)) return x > 0 ? x : -0.0;
  const double c = sqrt(2.0 / 3.14159265358979323846);
  const double u = c * (x + 0.044715 * x * x * x);
  /* 0.5 * (1 + tanh(u)) == 1 / (1 + exp(-2u)) exactly; the right side keeps full
   * relative precision where 1 + tanh(u) would cancel (x below about -5) */
  return x / (1.0 + exp(-2.0 * u));
}

/* Round a double to bf16 (8 significant bits, subnormals, overflow to inf), RNE;
 * returns the bf16 bits.  If `lo`/`hi` are non-NULL they receive the two bf16 values
 * bracketing |v| (equal when v is exactly representable). */
static uint16_t round_d_to_bf16(double v, double* lo_out, double* hi_out) {
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  if (isnan(v)) return (uint16_t)(0x7FC0 | sign);
  if (isinf(v)) return (uint16_t)(0x7F80 | sign);
  if (a == 0.0) {
    if (lo_out) *lo_out = 0.0;
    if (hi_out) *hi_out = 0.0;
    return sign;
  }
  int e;
  frexp(a, &e);
  e -= 1;
  if (e < -126) e = -126;
  double q = ldexp(1.0, e - 7);           /* spacing of bf16 values near a */
  double fl = floor(a / q) * q, ce = ceil(a / q) * q;
  if (lo_out) *lo_out = fl;
  if (hi_out) *hi_out = ce;
  double r = ldexp(nearbyint(ldexp(a, 7 - e)), e - 7);  /* nearest bf16 magnitude */
  if (r >= ldexp(1.0, 128)) return (uint16_t)(0x7F80 | sign);
  return (uint16_t)((f2u((float)r) >> 16) | sign);
}

/* y = RN_bf16(gelu(x)) for one bf16 x; *alt = the other admissible bf16 result when the
 * double value is within the single-precision error window of a rounding midpoint, else
 * *alt = y.  Window (relative to |gelu|): 2^-24 * (16 + 4*|2u|), plus 2^-147 absolute. */
uint16_t oracle_gelu_bf16(uint16_t xb, uint16_t* alt) {
  float xf = u2f((uint32_t)xb << 16);
  double x = (double)xf;
  double g = gelu_tanh_d(x);
  double lo = 0.0, hi = 0.0;
  uint16_t y = round_d_to_bf16(g, &lo, &hi);
  *alt = y;
  if (isnan(g) || isinf(g) || lo == hi) return y;
  const double c = sqrt(2.0 / 3.14159265358979323846);
  double u2 = fabs(2.0 * c * (x + 0.044715 * x * x * x));
  double win = ldexp(16.0 + 4.0 * u2, -24) * fabs(g) + ldexp(1.0, -147);
  double mid = 0.5 * (lo + hi), a = fabs(g);
  if (fabs(a - mid) <= win) {
    /* the neighbour RN did not pick (at an exact tie RN picked the even one) */
    double picked = (double)u2f((uint32_t)(y & 0x7FFF) << 16);
    double other = (picked == lo) ? hi : lo;
    uint16_t sign = signbit(g) ? 0x8000 : 0;
    if (other >= ldexp(1.0, 128)) *alt = (uint16_t)(0x7F80 | sign);
    else *alt = (uint16_t)((f2u((float)other) >> 16) | sign);
  }
  return y;
}

/* Elementwise over n bf16 pre-activations: y (RN), alt (see above). */
void oracle_gelu_bf16_array(const uint16_t* x, uint16_t* y, uint16_t* alt, int64_t n) {
  for (int64_t i = 0; i < n; ++i) y[i] = oracle_gelu_bf16(x[i], &alt[i]);
}

double oracle_gelu_double(double x) { return gelu_tanh_d(x); }

/* ------------------------------------------------------------------------------
 * Producer-fused quantize of the LayerNorm output: the transformer block of the
 * reproducer in "Fusion of Fp8 quantization and amax reduction kernels" (test.py:
 * BasicTransformer applies Flax nn.LayerNorm() to its input and feeds the result to
 * the MLP's first dense, whose FP8 dot quantizes it).  Readings (the pages give only
 * the call):
 *  L1 the defaults of that layer: per row of the last axis (length H), the mean mu
 *     and the biased variance V = mean((x - mu)^2);
 *     y = gamma * (x - mu) / sqrt(V + eps) + beta, with eps = 1e-6 passed as its
 *     binary32 value (the layer works in binary32) and per-feature binary32 gamma
 *     (scale) and beta (bias); no gamma means 1, no beta means 0.
 *  L2 the dense casts its input to the model's dtype: the quantized tensor is
 *     RN_bf16(y) of the exact y (evaluated here in double, sums compensated), then
 *     quantized and reduced as a bf16 tensor (R1-R5).
 *  L3 a row whose normalization is undefined (an inf or NaN input, or V + eps = 0)
 *     gives NaN, and every NaN of y is the positive default NaN 0x7FC0.
 * Admissible alternative.  A binary32 evaluation -- tree sums of depth D <= ceil(log2 H)
 * + 6, mu' = RN(S/H), d' = RN(x - mu'), a corrected second pass e' = sum(d')/H,
 * V' = sum(d'^2)/H - e'^2, r' = 1/sqrt(V' + eps), y' = RN(fma(d' - e', RN(gamma r'),
 * beta)) -- differs from y by at most, to first order in u = 2^-24,
 *   u (|gamma| r (|d| (D/2 + 6 + (D+1)(D+2) u A A_d r^2) + (D+2) A_d + (D+2)^2 u A) + |y|)
 * (d = x - mu, r = 1/sqrt(V + eps), A = mean|x|, A_d = mean|d|): d' - e' is off by
 * 2u|d| plus the residual error of the corrected mean, (D+2) u A_d, plus (D+2)^2 u^2 A
 * left from the first mean; V' is off relatively by (D+4) u plus the cross term
 * 2 (D+1)(D+2) u^2 A A_d / (V + eps), which r' halves and to which sqrt, the
 * divide and gamma r' add 3 ulps.  The window is twice that with L = ceil(log2 H) + 10
 * >= D + 4, plus 2^-147 for a subnormal y:
 *   w = 2^-23 (|gamma| r (|d| (L/2 + 7 + L^2 2^-24 A A_d r^2) + L A_d + L^2 2^-24 A)
 *              + |y|) + 2^-147.
 * Its absolute terms can exceed a bf16 spacing where |y| is small against the row's
 * spread, so the admissible results form a range: every bf16 value from
 * y_lo = RN_bf16(y - w) to y_hi = RN_bf16(y + w) (RN is monotone), which reduces to
 * y alone away from rounding midpoints and holds both neighbours at an exact tie. */
static int ceil_log2_i64(int64_t n) {
  int l = 0;
  while (((int64_t)1 << l) < n) ++l;
  return l;
}

/* Neumaier's compensated sum step: s + c carries the running sum. */
static void comp_add(double* s, double* c, double v) {
  double t = *s + v;
  *c += (fabs(*s) >= fabs(v)) ? (*s - t) + v : (v - t) + *s;
  *s = t;
}

/* rows x H bf16 inputs (row-major) -> y (RN_bf16 of the exact LayerNorm), the
 * admissible range [y_lo, y_hi] (see above), per-row mean and rstd = 1/sqrt(V + eps)
 * in double (NaN for an undefined row).  gamma, beta: H binary32 values each, or NULL. */
void oracle_layernorm_bf16(const uint16_t* x, const float* gamma, const float* beta,
                           float eps, int64_t rows, int64_t H, uint16_t* y, uint16_t* y_lo,
                           uint16_t* y_hi, double* mean_out, double* rstd_out) {
  const double L = (double)ceil_log2_i64(H) + 10.0;
  for (int64_t r = 0; r < rows; ++r) {
    const uint16_t* xr = x + r * H;
    uint16_t* yr = y + r * H;
    uint16_t* lr = y_lo + r * H;
    uint16_t* hr = y_hi + r * H;
    int finite = 1;
    for (int64_t i = 0; i < H; ++i)
      if ((xr[i] & 0x7F80) == 0x7F80) finite = 0;
    if (!finite) {
      for (int64_t i = 0; i < H; ++i) yr[i] = lr[i] = hr[i] = 0x7FC0;
      mean_out[r] = NAN;
      rstd_out[r] = NAN;
      continue;
    }
    double s = 0.0, c = 0.0, sabs = 0.0;
    for (int64_t i = 0; i < H; ++i) {
      double v = (double)u2f((uint32_t)xr[i] << 16);
      comp_add(&s, &c, v);
      sabs += fabs(v);
    }
    const double mu = (s + c) / (double)H;
    double sv = 0.0, cv = 0.0, sad = 0.0;
    for (int64_t i = 0; i < H; ++i) {
      double d = (double)u2f((uint32_t)xr[i] << 16) - mu;
      comp_add(&sv, &cv, d * d);
      sad += fabs(d);
    }
    const double V = (sv + cv) / (double)H;
    const double A = sabs / (double)H, Ad = sad / (double)H;
    const double rr = 1.0 / sqrt(V + (double)eps);
    mean_out[r] = mu;
    rstd_out[r] = rr;
    for (int64_t i = 0; i < H; ++i) {
      const double g = gamma ? (double)gamma[i] : 1.0;
      const double b = beta ? (double)beta[i] : 0.0;
      const double d = (double)u2f((uint32_t)xr[i] << 16) - mu;
      const double v = g * d * rr + b;
      if (isnan(v)) {
        yr[i] = lr[i] = hr[i] = 0x7FC0;
        continue;
      }
      yr[i] = round_d_to_bf16(v, NULL, NULL);
      const double w =
          ldexp(fabs(g) * rr *
                        (fabs(d) * (L / 2 + 7 + L * L * ldexp(A * Ad * rr * rr, -24)) +
                         L * Ad + L * L * ldexp(A, -24)) +
                    fabs(v),
                -23) +
          ldexp(1.0, -147);
      lr[i] = round_d_to_bf16(v - w, NULL, NULL);
      hr[i] = round_d_to_bf16(v + w, NULL, NULL);
    }
  }
}

/* ------------------------------------------------------------------------------
 * FP8 GEMM consumer ("User Guide on Native XLA-FP8", section "JAX": the FP8 operands are
 * cast up and multiplied by their scales, then the dot; the page's matmul takes two FP8
 * tensors and two binary32 scalar scales).  Readings:
 *  M1 C[m][n] = sa * sb * sum_k decode(A[m][k]) * decode(B[n][k]) with both operands
 *     K-contiguous (A: M x K, B: N x K, row-major): the layout FP8 matmuls require.
 *  M2 the sum is the exact value (every FP8 product is an integer times a power of two,
 *     accumulated here exactly in 128-bit fixed point), converted to double (relative
 *     error below 2^-51) and multiplied by the scales in double (sa * sb is exact in
 *     double).  A hardware evaluation is judged against it by the error bound of its
 *     accumulation, so the oracle also returns sum_k |a_k b_k| and, for accumulators
 *     that sum aligned groups of 8 consecutive products with limited precision, the sum
 *     over those groups (k in [8q, 8q + 8)) of the group's largest |a_k b_k|, both times
 *     |sa sb|.
 *  M3 IEEE specials: a NaN operand, inf * 0, or inf - inf gives NaN; an inf operand
 *     times a finite nonzero one gives +-inf (E5M2 codes only; the quantize never
 *     produces inf).
 */
typedef struct { int64_t m; int e; int special; } fp8_parts; /* value = m * 2^e */

static fp8_parts fp8_split(int fmt, uint8_t code) {
  fp8_parts p = {0, 0, 0};
  const int mbits = fmt_mbits(fmt), bias = fmt_bias(fmt);
  const int ebits = 7 - mbits;
  const int sign = code >> 7, ex = (code >> mbits) & ((1 << ebits) - 1);
  const int man = code & ((1 << mbits) - 1);
  double v = oracle_fp8_decode(fmt, code);
  if (isnan(v)) { p.special = 2; return p; }
  if (isinf(v)) { p.special = v > 0 ? 1 : -1; return p; }
  if (ex == 0) { p.m = man; p.e = 1 - bias - mbits; }
  else { p.m = (1 << mbits) | man; p.e = ex - bias - mbits; }
  if (sign) p.m = -p.m;
  return p;
}

/* C_exact[m*N+n], C_abs[m*N+n] and C_gmax[m*N+n] (all including the scales), double. */
void oracle_fp8_gemm(const uint8_t* A, int a_fmt, const uint8_t* B, int b_fmt, int64_t M,
                     int64_t N, int64_t K, float sa, float sb, double* C_exact, double* C_abs,
                     double* C_gmax) {
  /* products m_a m_b 2^(e_a + e_b); every exponent is >= 2 * (1 - 15 - 2) = -32 */
  const int e0 = -40;
  const double s = (double)sa * (double)sb;
  for (int64_t m = 0; m < M; ++m)
    for (int64_t n = 0; n < N; ++n) {
      __int128 acc = 0, acc_abs = 0;
      int nan = 0, pinf = 0, ninf = 0;
      double gsum = 0.0, gmax = 0.0;   /* sum over groups of 8 of the largest |a b| */
      for (int64_t k = 0; k < K; ++k) {
        if (k % 8 == 0) { gsum += gmax; gmax = 0.0; }
        fp8_parts a = fp8_split(a_fmt, A[m * K + k]), b = fp8_split(b_fmt, B[n * K + k]);
        if (a.special == 2 || b.special == 2) { nan = 1; continue; }
        if (a.special || b.special) {
          const int sa_ = a.special ? a.special : (a.m > 0 ? 1 : a.m < 0 ? -1 : 0);
          const int sb_ = b.special ? b.special : (b.m > 0 ? 1 : b.m < 0 ? -1 : 0);
          if (sa_ == 0 || sb_ == 0) nan = 1;            /* inf * 0 */
          else if (sa_ * sb_ > 0) pinf = 1;
          else ninf = 1;
          continue;
        }
        const __int128 t = (__int128)(a.m * b.m) << (a.e + b.e - e0);
        acc += t;
        acc_abs += t < 0 ? -t : t;
        const double pa = fabs(ldexp((double)(a.m * b.m), a.e + b.e));
        if (pa > gmax) gmax = pa;
      }
      gsum += gmax;
      double v, va;
      if (nan || (pinf && ninf)) { v = NAN; va = NAN; }
      else if (pinf) { v = INFINITY; va = INFINITY; }
      else if (ninf) { v = -INFINITY; va = INFINITY; }
      else {
        /* the exact fixed-point sum in double (two roundings at most) */
        const int neg = acc < 0;
        unsigned __int128 u = neg ? (unsigned __int128)(-acc) : (unsigned __int128)acc;
        const double hi = (double)(uint64_t)(u >> 64), lo = (double)(uint64_t)u;
        v = ldexp(ldexp(hi, 64) + lo, e0);
        if (neg) v = -v;
        const unsigned __int128 ua = (unsigned __int128)acc_abs;
        va = ldexp(ldexp((double)(uint64_t)(ua >> 64), 64) + (double)(uint64_t)ua, e0);
      }
      C_exact[m * N + n] = v * s;
      C_abs[m * N + n] = va * fabs(s);
      if (C_gmax) C_gmax[m * N + n] = (isnan(va) || isinf(va)) ? va : gsum * fabs(s);
    }
}
