"""Host proof that the GPU quantize kernel's division sequence is exact where it is used.

The kernel does not run the general IEEE divide per element.  With r = RN(1/s) computed
once per tensor (one IEEE division), each element takes
    bf16 source:  q0 = RN(x*r);  e = fma(q0, s, -x);  q = fma(-e, r, q0)
    fp32 source:  the same correction applied twice (q1 from q0, then q from q1)
(Markstein's correction step: P. Markstein, "Computation of elementary functions on
the IBM RISC System/6000 processor", IBM J. Res. Dev. 34(1), 1990; J.-M. Muller et al.,
"Handbook of Floating-Point Arithmetic", 2nd ed., section 4.7).  It is used only when
s lies in [2^-80, 2^125] and |x| < s * 2^126; other elements take the IEEE divide.

Over that window every binary32 operation above is exact-scaling in the exponents of x
and s (no overflow, no precision lost to underflow when the quotient can reach a
non-zero FP8 code), so the bf16 case is settled by sweeping every bf16 mantissa against
every binary32 mantissa of s (2^7 * 2^23 pairs).  Tiny quotients, where the residual
may underflow, must still give the same FP8 byte (zero of the right sign).  The fp32
case relies on Markstein's theorem (correction of a faithful quotient with a correctly
rounded reciprocal is correctly rounded); it is exercised here on random and
near-tie operands.
"""
import ctypes
import subprocess

import numpy as np
import pytest

C_SRC = r"""
#include <math.h>
#include <stdint.h>
#include <string.h>
static float u2f(uint32_t u){float f;memcpy(&f,&u,4);return f;}
static uint32_t f2u(float f){uint32_t u;memcpy(&u,&f,4);return u;}
/* OPAQUE stops gcc from merging the negated residual into an fnmadd: that rewrite
   computes x - q0*s instead of -(q0*s - x), which differs in the sign of a zero.  The
   GPU code applies the negation as an operand modifier of v_fma_f32, as written. */
#define OPAQUE(v) __asm__("" : "+x"(v))
static float div3(float x, float s, float r){
  float q0 = x * r; float e = fmaf(q0, s, -x); OPAQUE(e); return fmaf(-e, r, q0);
}
static float div5(float x, float s, float r){
  float q0 = x * r; float e0 = fmaf(q0, s, -x); OPAQUE(e0); float q1 = fmaf(-e0, r, q0);
  float e1 = fmaf(q1, s, -x); OPAQUE(e1); return fmaf(-e1, r, q1);
}
/* every bf16 mantissa (x in [1,2)) against s mantissas [s_lo, s_hi) of [1,2) */
int64_t sweep_bf16(uint32_t s_lo, uint32_t s_hi, int use5){
  int64_t bad = 0;
  for (uint32_t sm = s_lo; sm < s_hi; ++sm){
    float s = u2f(0x3F800000u | sm); float r = 1.0f / s;
    for (uint32_t xm = 0; xm < 128; ++xm){
      float x = u2f(0x3F800000u | (xm << 16));
      float q = use5 ? div5(x, s, r) : div3(x, s, r);
      if (f2u(q) != f2u(x / s)) ++bad;
    }
  }
  return bad;
}
/* random pairs (x bits, s bits) given by the caller; count binary32 mismatches */
int64_t check_pairs(const uint32_t* xb, const uint32_t* sb, int64_t n, int use5,
                    uint32_t* bad_idx, int64_t max_bad){
  int64_t bad = 0;
  for (int64_t i = 0; i < n; ++i){
    float x = u2f(xb[i]), s = u2f(sb[i]); float r = 1.0f / s;
    float q = use5 ? div5(x, s, r) : div3(x, s, r);
    if (f2u(q) != f2u(x / s)) { if (bad < max_bad) bad_idx[bad] = (uint32_t)i; ++bad; }
  }
  return bad;
}
void quotients(const uint32_t* xb, const uint32_t* sb, int64_t n, int use5,
               float* fast, float* ieee){
  for (int64_t i = 0; i < n; ++i){
    float x = u2f(xb[i]), s = u2f(sb[i]); float r = 1.0f / s;
    fast[i] = use5 ? div5(x, s, r) : div3(x, s, r); ieee[i] = x / s;
  }
}
"""


@pytest.fixture(scope="module")
def lib(tmp_path_factory):
    d = tmp_path_factory.mktemp("divalg")
    src = d / "divalg.c"
    src.write_text(C_SRC)
    so = d / "divalg.so"
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-mfma", "-fPIC", "-shared", "-o",
                    str(so), str(src), "-lm"], check=True)
    L = ctypes.CDLL(str(so))
    L.sweep_bf16.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_int]
    L.sweep_bf16.restype = ctypes.c_int64
    vp = ctypes.c_void_p
    L.check_pairs.argtypes = [vp, vp, ctypes.c_int64, ctypes.c_int, vp, ctypes.c_int64]
    L.check_pairs.restype = ctypes.c_int64
    L.quotients.argtypes = [vp, vp, ctypes.c_int64, ctypes.c_int, vp, vp]
    return L


def _parallel_sweep(lib, use5):
    from concurrent.futures import ThreadPoolExecutor
    n, k = 1 << 23, 16
    with ThreadPoolExecutor(8) as ex:
        return sum(ex.map(lambda i: lib.sweep_bf16(i * n // k, (i + 1) * n // k, use5),
                          range(k)))


def test_bf16_three_op_exhaustive(lib):
    """All 2^7 bf16 mantissas x all 2^23 binary32 mantissas of s: zero mismatches."""
    assert _parallel_sweep(lib, 0) == 0


def _pairs_window(g, n, x_is_bf16):
    s_exp = g.integers(-80, 126, n)
    s = np.ldexp(1.0 + g.integers(0, 1 << 23, n) / 2.0 ** 23, s_exp).astype(np.float32)
    # quotient exponent spread over the range that can reach a non-zero FP8 code and
    # up to the 2^126 bound of the window
    q_exp = g.integers(-18, 126, n)
    x = (s.astype(np.float64) * np.ldexp(1.0 + g.random(n), q_exp)).astype(np.float32)
    x = np.minimum(x, np.float32(3.38e38))
    xb = x.view(np.uint32)
    if x_is_bf16:
        xb = xb & 0xFFFF0000
    xb = xb | (g.integers(0, 2, n).astype(np.uint32) << 31)
    keep = np.abs(xb.view(np.float32).astype(np.float64)) < s.astype(np.float64) * 2.0 ** 126
    return xb[keep].copy(), s.view(np.uint32)[keep].copy()


@pytest.mark.parametrize("x_is_bf16,use5", [(True, 0), (False, 1)])
def test_window_random(lib, x_is_bf16, use5):
    g = np.random.Generator(np.random.PCG64(41 + use5))
    xb, sb = _pairs_window(g, 2_000_000, x_is_bf16)
    bad = np.zeros(16, np.uint32)
    nbad = lib.check_pairs(xb.ctypes.data, sb.ctypes.data, xb.size, use5, bad.ctypes.data, 16)
    assert nbad == 0, [(hex(xb[i]), hex(sb[i])) for i in bad[:min(nbad, 16)]]


def test_fp32_near_fp8_ties(lib):
    """x = RN(m*s) +- a few ulps for every FP8 midpoint m: the correction must land on
    the same binary32 quotient as IEEE division (the double rounding decides here)."""
    g = np.random.Generator(np.random.PCG64(43))
    mids = []
    for mb, emin, emax in ((3, -6, 8), (2, -14, 15)):
        for e in range(emin - 1, emax + 1):
            for k in range(1 << mb):
                mids.append(np.ldexp(1.0 + (k + 0.5) / (1 << mb), e))
    mids = np.array(mids)
    s = np.ldexp(1.0 + g.integers(0, 1 << 23, 200000) / 2.0 ** 23,
                 g.integers(-40, 40, 200000)).astype(np.float32)
    m = mids[g.integers(0, mids.size, s.size)]
    x = (m * s.astype(np.float64)).astype(np.float32).view(np.uint32)
    xs = np.concatenate([(x.astype(np.int64) + d).astype(np.uint32) for d in (-2, -1, 0, 1, 2)])
    ss = np.tile(s.view(np.uint32), 5)
    bad = np.zeros(16, np.uint32)
    assert lib.check_pairs(xs.ctypes.data, ss.ctypes.data, xs.size, 1, bad.ctypes.data, 16) == 0


def test_tiny_quotients_give_zero_code(lib):
    """Below the window's exactness range (quotients < 2^-18, where the residual may
    underflow) a binary32 mismatch is allowed only if both quotients encode to an FP8
    zero of the same sign (|q| <= 2^-17, the E5M2 round-to-zero bound)."""
    g = np.random.Generator(np.random.PCG64(47))
    n = 1_000_000
    s = np.ldexp(1.0 + g.integers(0, 1 << 23, n) / 2.0 ** 23, g.integers(-80, 126, n))
    s = s.astype(np.float32)
    q = np.ldexp(1.0 + g.random(n), g.integers(-160, -18, n))
    x = (s.astype(np.float64) * q).astype(np.float32).view(np.uint32) & 0xFFFF0000
    x |= g.integers(0, 2, n).astype(np.uint32) << 31
    for use5 in (0, 1):
        fast = np.empty(n, np.float32)
        ieee = np.empty(n, np.float32)
        lib.quotients(x.ctypes.data, s.view(np.uint32).ctypes.data, n, use5,
                      fast.ctypes.data, ieee.ctypes.data)
        diff = fast.view(np.uint32) != ieee.view(np.uint32)
        assert (np.abs(fast[diff]) < 2.0 ** -17).all()
        assert (np.abs(ieee[diff]) < 2.0 ** -17).all()
        assert (np.signbit(fast[diff]) == np.signbit(ieee[diff])).all()
        # zero quotients keep the sign of x
        z = fast == 0
        assert (np.signbit(fast[z]) == (x[z] >> 31).astype(bool)).all()
