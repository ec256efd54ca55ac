"""CPU oracle for FP8 delayed scaling (quantize + amax, amax-history scale update,
dequantize).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``.  The GPU library (``delayed_scaling_amax_amd``)
never imports, links or calls anything here, and this package never imports it.

The arithmetic lives in ``fp8_oracle.c`` (plain serial C, one IEEE binary32 operation
per step).  This module compiles it with gcc and marshals numpy arrays into it.  The
only parallelism added here is splitting an element range into contiguous chunks run
by threads; the chunk amaxes are combined with the same bit-pattern max the oracle
uses, which is exact and order-independent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fp8_oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")

E4M3, E5M2 = 0, 1
BF16, F32 = 0, 1
AMAX_MAX, AMAX_MOST_RECENT = 0, 1

_lib = None


def build(lib_path: str = LIB_PATH, src: str = _SRC, extra_flags=()) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    tmp = lib_path + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-Wall",
           "-fPIC", "-shared", "-o", tmp, src, "-lm", *extra_flags]
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib_path)
    return lib_path


def _declare(lib):
    c = ctypes
    vp, i64, i32, f32p = c.c_void_p, c.c_int64, c.c_int, c.POINTER(c.c_float)
    lib.oracle_fp8_max.argtypes = [i32]
    lib.oracle_fp8_max.restype = c.c_float
    lib.oracle_fp8_decode.argtypes = [i32, c.c_uint8]
    lib.oracle_fp8_decode.restype = c.c_float
    lib.oracle_fp8_encode.argtypes = [i32, c.c_float]
    lib.oracle_fp8_encode.restype = c.c_uint8
    lib.oracle_quantize_element.argtypes = [i32, c.c_float, c.c_float]
    lib.oracle_quantize_element.restype = c.c_uint8
    lib.oracle_quantize_amax.argtypes = [vp, i32, vp, i64, i32, c.c_float, f32p]
    lib.oracle_quantize_amax.restype = None
    lib.oracle_amax_and_scale_update.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64,
                                                 i32, i32, i32]
    lib.oracle_amax_and_scale_update.restype = None
    lib.oracle_dequantize.argtypes = [vp, i32, vp, i32, i64, c.c_float]
    lib.oracle_dequantize.restype = None
    lib.oracle_count_saturated.argtypes = [vp, i32, i64, i32, c.c_float]
    lib.oracle_count_saturated.restype = i64
    lib.oracle_gelu_bf16_array.argtypes = [vp, vp, vp, i64]
    lib.oracle_gelu_bf16_array.restype = None
    lib.oracle_gelu_double.argtypes = [c.c_double]
    lib.oracle_gelu_double.restype = c.c_double
    lib.oracle_layernorm_bf16.argtypes = [vp, vp, vp, c.c_float, i64, i64, vp, vp, vp, vp, vp]
    lib.oracle_layernorm_bf16.restype = None
    lib.oracle_fp8_gemm.argtypes = [vp, c.c_int, vp, c.c_int, i64, i64, i64, c.c_float, c.c_float,
                                    vp, vp, vp]
    lib.oracle_fp8_gemm.restype = None
    return lib


class Oracle:
    """ctypes view of one compiled oracle library (the real one, or a test mutant)."""

    def __init__(self, lib_path: str):
        self.path = lib_path
        self.lib = _declare(ctypes.CDLL(lib_path))

    # -- scalar entry points -------------------------------------------------
    def fp8_max(self, fmt: int) -> float:
        return float(self.lib.oracle_fp8_max(fmt))

    def decode(self, fmt: int, code: int) -> float:
        return float(self.lib.oracle_fp8_decode(fmt, code))

    def encode(self, fmt: int, v: float) -> int:
        return int(self.lib.oracle_fp8_encode(fmt, v))

    def quantize_element(self, fmt: int, x: float, scale: float) -> int:
        return int(self.lib.oracle_quantize_element(fmt, x, scale))

    # -- array entry points --------------------------------------------------
    @staticmethod
    def _src(x: np.ndarray):
        x = np.ascontiguousarray(x)
        if x.dtype == np.uint16:
            return x, BF16
        if x.dtype == np.float32:
            return x, F32
        raise TypeError("src must be uint16 (bf16 bits) or float32, got %s" % x.dtype)

    def quantize_amax(self, x: np.ndarray, fmt: int, scale: float, amax_in: float = 0.0,
                      threads: int = 1, out: np.ndarray | None = None):
        """Returns (codes uint8[n], amax float32).  x: uint16 bf16 bits or float32."""
        x, dt = self._src(x)
        flat = x.reshape(-1)
        n = flat.size
        dst = np.empty(n, np.uint8) if out is None else out.reshape(-1)
        threads = max(1, min(int(threads), max(1, n // (1 << 16))))
        bounds = [n * k // threads for k in range(threads + 1)]
        # amax travels as its bit pattern: a float32 -> Python float conversion would
        # quiet a signaling NaN and so raise its magnitude bits above the true maximum.
        a_in = np.asarray(amax_in, np.float32).reshape(1).view(np.uint32)
        amaxes = np.zeros(threads, np.uint32)

        def run(k):
            lo, hi = bounds[k], bounds[k + 1]
            a = a_in.copy()                  # every chunk max-accumulates into amax_in
            self.lib.oracle_quantize_amax(flat[lo:].ctypes.data if hi > lo else None, dt,
                                          dst[lo:].ctypes.data if hi > lo else None,
                                          hi - lo, fmt, float(scale),
                                          a.ctypes.data_as(ctypes.POINTER(ctypes.c_float)))
            amaxes[k] = a[0]

        if threads == 1:
            run(0)
        else:
            with ThreadPoolExecutor(threads) as ex:
                list(ex.map(run, range(threads)))
        return dst.reshape(x.shape), amaxes.max().view(np.float32)

    def amax_and_scale_update(self, amax, hist, scale, formats, algo=AMAX_MAX, margin=0,
                              reset_amax=False):
        """Out-of-place update.  hist: float32[H, n].  Returns dict of new arrays."""
        amax = np.ascontiguousarray(amax, np.float32)
        hist = np.ascontiguousarray(hist, np.float32)
        scale = np.ascontiguousarray(scale, np.float32)
        formats = np.ascontiguousarray(formats, np.uint8)
        H, n = hist.shape
        assert amax.shape == (n,) and scale.shape == (n,) and formats.shape == (n,)
        out = dict(hist=np.empty_like(hist), scale=np.empty_like(scale),
                   scale_inv=np.empty_like(scale), amax=np.empty_like(amax))
        self.lib.oracle_amax_and_scale_update(
            amax.ctypes.data, hist.ctypes.data, out["hist"].ctypes.data, scale.ctypes.data,
            out["scale"].ctypes.data, out["scale_inv"].ctypes.data, out["amax"].ctypes.data,
            formats.ctypes.data, n, H, int(algo), int(margin), int(bool(reset_amax)))
        return out

    def dequantize(self, codes: np.ndarray, fmt: int, scale: float, out_dtype: int = F32):
        codes = np.ascontiguousarray(codes, np.uint8)
        dst = np.empty(codes.shape, np.float32 if out_dtype == F32 else np.uint16)
        self.lib.oracle_dequantize(codes.ctypes.data, fmt, dst.ctypes.data, out_dtype,
                                   codes.size, float(scale))
        return dst

    def gelu_bf16(self, x: np.ndarray, threads: int = 1):
        """y = RN_bf16(gelu_tanh(x)) for bf16 bits x; returns (y, alt) uint16 arrays where
        alt is the other admissible neighbour near a rounding midpoint (else alt == y).
        `threads` splits the array into contiguous pieces (elementwise, so the result
        does not depend on it)."""
        x = np.ascontiguousarray(x, np.uint16).reshape(-1)
        y = np.empty_like(x)
        alt = np.empty_like(x)

        def run(lo, hi):
            self.lib.oracle_gelu_bf16_array(x[lo:].ctypes.data, y[lo:].ctypes.data,
                                            alt[lo:].ctypes.data, hi - lo)

        n = x.size
        if threads <= 1 or n < (1 << 20):
            run(0, n)
        else:
            bounds = np.linspace(0, n, threads + 1).astype(np.int64)
            with ThreadPoolExecutor(threads) as ex:
                list(ex.map(run, bounds[:-1], bounds[1:]))
        return y, alt

    def gelu_double(self, x: float) -> float:
        return float(self.lib.oracle_gelu_double(float(x)))

    def gelu_quantize_amax(self, x: np.ndarray, fmt: int, scale: float, amax_in: float = 0.0,
                           threads: int = 1):
        """Producer-fused quantize of gelu(x): returns (codes, amax, codes_alt, amax_lo,
        amax_hi).  codes/amax follow y = RN_bf16(gelu(x)); codes_alt are the codes of the
        admissible alternative y; [amax_lo, amax_hi] bounds the amax over every admissible
        choice (bit patterns)."""
        y, alt = self.gelu_bf16(x, threads=threads)
        codes, amax = self.quantize_amax(y, fmt, scale, amax_in=amax_in, threads=threads)
        codes_alt, _ = self.quantize_amax(alt, fmt, scale, amax_in=amax_in, threads=threads)
        my = y.astype(np.uint32) & 0x7FFF
        ma = alt.astype(np.uint32) & 0x7FFF
        a_in = int(np.float32(amax_in).view(np.uint32))
        lo = max(int(np.minimum(my, ma).max(initial=0)) << 16, a_in)
        hi = max(int(np.maximum(my, ma).max(initial=0)) << 16, a_in)
        return (codes.reshape(x.shape), amax, codes_alt.reshape(x.shape),
                np.uint32(lo).view(np.float32), np.uint32(hi).view(np.float32))

    def layernorm_bf16(self, x: np.ndarray, gamma=None, beta=None, eps: float = 1e-6,
                       threads: int = 1):
        """LayerNorm over the last axis of bf16 bits x (rows, H): returns (y, y_lo, y_hi,
        mean, rstd) -- y = RN_bf16 of the exact value, [y_lo, y_hi] the admissible range
        of a binary32 evaluation (bf16 bits; y_lo == y == y_hi away from rounding
        midpoints), mean and rstd per row in double.  gamma/beta are float32 arrays of
        length H or None.  Rows are split over `threads`."""
        x = np.ascontiguousarray(x, np.uint16)
        H = x.shape[-1]
        x2 = x.reshape(-1, H)
        rows = x2.shape[0]
        g = None if gamma is None else np.ascontiguousarray(gamma, np.float32)
        b = None if beta is None else np.ascontiguousarray(beta, np.float32)
        assert g is None or g.size == H
        assert b is None or b.size == H
        y = np.empty_like(x2)
        y_lo = np.empty_like(x2)
        y_hi = np.empty_like(x2)
        mean = np.empty(rows, np.float64)
        rstd = np.empty(rows, np.float64)

        def run(r0, r1):
            if r1 > r0:
                self.lib.oracle_layernorm_bf16(
                    x2[r0:].ctypes.data, None if g is None else g.ctypes.data,
                    None if b is None else b.ctypes.data, float(np.float32(eps)), r1 - r0, H,
                    y[r0:].ctypes.data, y_lo[r0:].ctypes.data, y_hi[r0:].ctypes.data,
                    mean[r0:].ctypes.data, rstd[r0:].ctypes.data)

        if threads <= 1 or rows < 64:
            run(0, rows)
        else:
            bounds = np.linspace(0, rows, threads + 1).astype(np.int64)
            with ThreadPoolExecutor(threads) as ex:
                list(ex.map(run, bounds[:-1], bounds[1:]))
        return (y.reshape(x.shape), y_lo.reshape(x.shape), y_hi.reshape(x.shape), mean, rstd)

    def layernorm_quantize_amax(self, x: np.ndarray, fmt: int, scale: float, gamma=None,
                                beta=None, eps: float = 1e-6, amax_in: float = 0.0,
                                threads: int = 1):
        """Producer-fused quantize of LayerNorm(x): returns (codes, amax, codes_lo,
        codes_hi, amax_lo, amax_hi, mean, rstd): codes/amax of y, the codes of the ends
        of the admissible range (every admissible code lies between them in value, as
        the quantize is monotone), and the bounds of the amax over every admissible
        choice."""
        y, y_lo, y_hi, mean, rstd = self.layernorm_bf16(x, gamma, beta, eps, threads=threads)
        codes, amax = self.quantize_amax(y, fmt, scale, amax_in=amax_in, threads=threads)
        codes_lo, _ = self.quantize_amax(y_lo, fmt, scale, amax_in=amax_in, threads=threads)
        codes_hi, _ = self.quantize_amax(y_hi, fmt, scale, amax_in=amax_in, threads=threads)
        ml = y_lo.astype(np.uint32) & 0x7FFF
        mh = y_hi.astype(np.uint32) & 0x7FFF
        crosses = ((y_lo & 0x8000) != 0) | (ml == 0)
        crosses &= ((y_hi & 0x8000) == 0) | (mh == 0)
        min_mag = np.where(crosses, 0, np.minimum(ml, mh))
        a_in = int(np.float32(amax_in).view(np.uint32))
        lo = max(int(min_mag.max(initial=0)) << 16, a_in)
        hi = max(int(np.maximum(ml, mh).max(initial=0)) << 16, a_in)
        return (codes.reshape(x.shape), amax, codes_lo.reshape(x.shape),
                codes_hi.reshape(x.shape), np.uint32(lo).view(np.float32),
                np.uint32(hi).view(np.float32), mean, rstd)

    def fp8_gemm(self, A: np.ndarray, a_fmt: int, B: np.ndarray, b_fmt: int, sa: float = 1.0,
                 sb: float = 1.0, threads: int = 1):
        """C = sa*sb * decode(A) @ decode(B).T for FP8 codes A (M, K) and B (N, K): returns
        (C_exact, C_abs, C_gmax) in float64: C_abs = |sa*sb| * sum_k |a_k b_k| and C_gmax =
        |sa*sb| * sum over k-groups [8q, 8q+8) of the group's largest |a_k b_k| (the scales
        of an accumulation's error bound).  Rows of C are split over `threads`."""
        A = np.ascontiguousarray(A, np.uint8)
        B = np.ascontiguousarray(B, np.uint8)
        M, K = A.shape
        N, K2 = B.shape
        assert K == K2
        C = np.empty((M, N), np.float64)
        Cabs = np.empty((M, N), np.float64)
        Cg = np.empty((M, N), np.float64)

        def run(r0, r1):
            if r1 > r0:
                self.lib.oracle_fp8_gemm(A[r0:].ctypes.data, a_fmt, B.ctypes.data, b_fmt,
                                         r1 - r0, N, K, float(sa), float(sb), C[r0:].ctypes.data,
                                         Cabs[r0:].ctypes.data, Cg[r0:].ctypes.data)

        if threads <= 1 or M < 2 * threads:
            run(0, M)
        else:
            bounds = np.linspace(0, M, threads + 1).astype(np.int64)
            with ThreadPoolExecutor(threads) as ex:
                list(ex.map(run, bounds[:-1], bounds[1:]))
        return C, Cabs, Cg

    def count_saturated(self, x: np.ndarray, fmt: int, scale: float) -> int:
        x, dt = self._src(x)
        return int(self.lib.oracle_count_saturated(x.ctypes.data, dt, x.size, fmt,
                                                   float(scale)))


def load(build_if_missing: bool = True) -> Oracle:
    """The oracle library built from fp8_oracle.c (compiled here if not built yet)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH) and build_if_missing:
            build()
        _lib = Oracle(LIB_PATH)
    return _lib
