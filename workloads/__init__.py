"""Seeded synthetic inputs for the FP8 delayed-scaling hot path.

This module only draws random numbers and rounds them to the storage dtype (bf16
round-to-nearest-even from float32).  It holds none of the method's arithmetic (no
quantization, amax, scale or history logic) and imports neither the oracle nor the
GPU library; both sides read the bytes it returns.

Randomness: numpy ``Generator(PCG64)`` seeded from ``SeedSequence(12, spawn_key=
(workload, tensor, chunk))`` -- 12 is the PRNG key of the reproducer on the page
"Fusion of Fp8 quantization and amax reduction kernels" (openxla/xla issue 7432,
``run_benchmark``).  Every fixed-size chunk has its own stream, so the bytes do not
depend on the number of threads used to produce them.

Workloads (shapes from that reproducer's layer configuration, and the MLP sizes the
design notes list):
  single_1024       one bf16 1024x1024 tensor ~ U[0,1), E4M3, prior scale 1.0,
                    history 16.
  mlp_4096          activation (2048,4,4096) ~ U[0,1); weights wi 4096x16384 and wo
                    16384x4096 ~ truncated normal (+-2 sigma, Flax variance_scaling
                    fan_in), all E4M3, history 16.
  grad_8192x16384   gradient 8192x16384 ~ 1e-3 * Student-t(3), 0.01% of entries x1e4,
                    E5M2 with a stale scale so ~0.1% of quotients saturate.
  update_1152       96 layers x 4 linears x 3 FP8 tensors = 1152 histories of length
                    1024, history and new amaxes ~ lognormal(0, 2).
  mlp_12288         activations (2048,12288), (2048,49152) ~ N(0,1); weights
                    12288x49152 ~ N(0,1/12288), 49152x12288 ~ N(0,1/49152); output
                    gradient (2048,12288) ~ N(0,1e-4) (variance); 4x E4M3 + 1x E5M2,
                    history 1024.
  mlp_4096_preact   the FFN pre-activation of mlp_4096, (2048,4,16384) bf16 ~ N(0,1/3):
                    the dense output of U[0,1) inputs (E[x^2] = 1/3) through unit-
                    variance fan_in weights; the input of the gelu-fused quantize.
  list_1152         the 1152 FP8 tensors of the batched-update layout (96 layers x 4
                    linear modules x input, weight, gradient) as one quantize list, at
                    hidden 512 and 128 tokens: per layer the inputs (128,512) x3 and
                    (128,2048), weights 512x1536, 512x512, 512x2048, 2048x512, output
                    gradients (128,1536), (128,512), (128,2048), (128,512); inputs
                    N(0,1), weights N(0,1/fan_in), gradients N(0,1e-4) (variance), as in
                    mlp_12288; inputs and weights E4M3, gradients E5M2.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

SEED = 12
CHUNK = 1 << 22          # elements per independent random stream

E4M3, E5M2 = "e4m3", "e5m2"

# Flax's truncated_normal initializer draws N(0,1) truncated to +-2 and divides by the
# standard deviation of that truncated distribution so the result has unit variance.
TRUNC2_STD = 0.87962566103423978

# Two-sided 0.09% quantile of Student-t with 3 degrees of freedom; the stale gradient
# scale is set so that |x| beyond ~this many 1e-3 units saturates E5M2.
T3_Q00045 = 13.39244106178217


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def f32_to_bf16_bits(x: np.ndarray, out: np.ndarray | None = None) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (inputs hold no NaN)."""
    u = x.view(np.uint32)
    r = (u >> 16) & 1
    r += 0x7FFF
    r += u
    r >>= 16
    if out is None:
        return r.astype(np.uint16)
    out[...] = r
    return out


def _rng(workload: int, tensor: int, chunk: int) -> np.random.Generator:
    ss = np.random.SeedSequence(SEED, spawn_key=(workload, tensor, chunk))
    return np.random.Generator(np.random.PCG64(ss))


# ---------------------------------------------------------------------------------
# Per-chunk samplers: each fills out[:m] (uint16 bf16 bits or float32) from g.
# ---------------------------------------------------------------------------------
def _uniform_trunc(g, out):
    # U[0,1) in float32, truncated (not rounded) to bf16 so every value stays < 1.
    v = g.random(out.size, dtype=np.float32)
    out[...] = (v.view(np.uint32) >> 16).astype(np.uint16)


def _normal(std):
    def f(g, out):
        v = g.standard_normal(out.size, dtype=np.float32)
        v *= np.float32(std)
        f32_to_bf16_bits(v, out)
    return f


def _trunc_normal(fan_in):
    std = math.sqrt(1.0 / fan_in) / TRUNC2_STD

    def f(g, out):
        v = g.standard_normal(out.size, dtype=np.float32)
        bad = np.abs(v) > 2.0
        while bad.any():
            v[bad] = g.standard_normal(int(bad.sum()), dtype=np.float32)
            bad = np.abs(v) > 2.0
        v *= np.float32(std)
        f32_to_bf16_bits(v, out)
    return f


def _student_t_outliers(g, out):
    v = g.standard_t(3, out.size)                  # float64
    v *= 1e-3
    v[g.random(out.size) < 1e-4] *= 1e4            # ~0.01% outliers
    f32_to_bf16_bits(v.astype(np.float32), out)


def _lognormal_f32(g, out):
    out[...] = g.lognormal(0.0, 2.0, out.size).astype(np.float32)


def _generate(workload_id, tensor_id, shape, dtype, sampler, threads):
    n = int(np.prod(shape))
    out = np.empty(n, dtype)
    nchunks = (n + CHUNK - 1) // CHUNK

    def run(c):
        lo = c * CHUNK
        sampler(_rng(workload_id, tensor_id, c), out[lo:min(n, lo + CHUNK)])

    if threads <= 1 or nchunks == 1:
        for c in range(nchunks):
            run(c)
    else:
        with ThreadPoolExecutor(min(threads, nchunks)) as ex:
            list(ex.map(run, range(nchunks)))
    return out.reshape(shape)


# ---------------------------------------------------------------------------------
@dataclass
class QTensor:
    name: str
    data: np.ndarray          # uint16 (bf16 bits) or float32
    fmt: str                  # "e4m3" | "e5m2"


@dataclass
class Workload:
    name: str
    description: str
    tensors: list = field(default_factory=list)   # list[QTensor]
    history_len: int = 16
    first_scale: list | None = None               # scale used by the first step
    # batched-update-only workloads
    hist: np.ndarray | None = None
    amax: np.ndarray | None = None
    scale: np.ndarray | None = None
    formats: list | None = None

    @property
    def numel(self) -> int:
        return sum(int(t.data.size) for t in self.tensors)

    def src_bytes(self) -> int:
        return sum(int(t.data.nbytes) for t in self.tensors)


def single_1024(threads=None, side=1024) -> Workload:
    th = threads or default_threads()
    x = _generate(1, 0, (side, side), np.uint16, _uniform_trunc, th)
    return Workload("single_1024" if side == 1024 else "single_%d" % side,
                    "one bf16 %dx%d tensor ~U[0,1) -> E4M3, prior scale 1.0, history 16"
                    % (side, side),
                    [QTensor("x", x, E4M3)], history_len=16, first_scale=[1.0])


def mlp_4096(threads=None, hidden=4096, ffn=16384, seq=2048, batch=4) -> Workload:
    th = threads or default_threads()
    act = _generate(2, 0, (seq, batch, hidden), np.uint16, _uniform_trunc, th)
    wi = _generate(2, 1, (hidden, ffn), np.uint16, _trunc_normal(hidden), th)
    wo = _generate(2, 2, (ffn, hidden), np.uint16, _trunc_normal(ffn), th)
    return Workload("mlp_%d" % hidden,
                    "MLP hidden %d ffn %d: act (%d,%d,%d) U[0,1), wi/wo truncated normal "
                    "fan_in; 3x E4M3 in one launch; history 16" % (hidden, ffn, seq, batch,
                                                                   hidden),
                    [QTensor("act", act, E4M3), QTensor("wi", wi, E4M3),
                     QTensor("wo", wo, E4M3)],
                    history_len=16, first_scale=[1.0, 1.0, 1.0])


def stale_grad_scale() -> np.float32:
    """Deliberately stale E5M2 scale: 1e-3 * t3 quantile / 57344, in float32."""
    return np.float32(np.float32(1e-3 * T3_Q00045) / np.float32(57344.0))


def grad_8192x16384(threads=None, rows=8192, cols=16384) -> Workload:
    th = threads or default_threads()
    g = _generate(3, 0, (rows, cols), np.uint16, _student_t_outliers, th)
    return Workload("grad_%dx%d" % (rows, cols),
                    "gradient %dx%d 1e-3*t3 with 0.01%% x1e4 outliers -> E5M2, stale "
                    "scale (~0.1%% saturate)" % (rows, cols),
                    [QTensor("grad", g, E5M2)], history_len=16,
                    first_scale=[float(stale_grad_scale())])


def update_1152(threads=None, layers=96, modules=4, history_len=1024) -> Workload:
    th = threads or default_threads()
    n = layers * modules * 3
    hist = _generate(4, 0, (history_len, n), np.float32, _lognormal_f32, th)
    amax = _generate(4, 1, (n,), np.float32, _lognormal_f32, th)
    formats = [E4M3, E4M3, E5M2] * (layers * modules)
    return Workload("update_%d" % n,
                    "batched update: %d layers x %d linears x 3 tensors = %d histories "
                    "of length %d, lognormal(0,2)" % (layers, modules, n, history_len),
                    history_len=history_len, hist=hist, amax=amax,
                    scale=np.ones(n, np.float32), formats=formats)


def mlp_12288(threads=None, hidden=12288, ffn=49152, tokens=2048) -> Workload:
    th = threads or default_threads()
    a1 = _generate(5, 0, (tokens, hidden), np.uint16, _normal(1.0), th)
    a2 = _generate(5, 1, (tokens, ffn), np.uint16, _normal(1.0), th)
    w1 = _generate(5, 2, (hidden, ffn), np.uint16, _normal(math.sqrt(1.0 / hidden)), th)
    w2 = _generate(5, 3, (ffn, hidden), np.uint16, _normal(math.sqrt(1.0 / ffn)), th)
    gr = _generate(5, 4, (tokens, hidden), np.uint16, _normal(math.sqrt(1e-4)), th)
    return Workload("mlp_%d" % hidden,
                    "MLP hidden %d ffn %d full step: 2 activations N(0,1), 2 weights "
                    "N(0,1/fan_in) to E4M3, output grad N(0,1e-4) to E5M2, history 1024"
                    % (hidden, ffn),
                    [QTensor("a1", a1, E4M3), QTensor("a2", a2, E4M3),
                     QTensor("w1", w1, E4M3), QTensor("w2", w2, E4M3),
                     QTensor("grad", gr, E5M2)],
                    history_len=1024, first_scale=[1.0] * 5)


def mlp_4096_preact(threads=None, ffn=16384, seq=2048, batch=4) -> Workload:
    th = threads or default_threads()
    h = _generate(6, 0, (seq, batch, ffn), np.uint16, _normal(math.sqrt(1.0 / 3.0)), th)
    return Workload("mlp_4096_preact",
                    "FFN pre-activation (%d,%d,%d) N(0,1/3) -> gelu -> E4M3, history 16"
                    % (seq, batch, ffn),
                    [QTensor("h", h, E4M3)], history_len=16, first_scale=[1.0])


def list_1152(threads=None, hidden=512, tokens=128, layers=96) -> Workload:
    """The c4 layout's tensors with concrete shapes, in module order (input, weight,
    gradient per linear: qkv, attention output, fc1, fc2)."""
    th = threads or default_threads()
    h, t = hidden, tokens
    linears = [((t, h), (h, 3 * h), (t, 3 * h)), ((t, h), (h, h), (t, h)),
               ((t, h), (h, 4 * h), (t, 4 * h)), ((t, 4 * h), (4 * h, h), (t, h))]
    specs = []  # (name, stream id, shape, sampler, format)
    for layer in range(layers):
        for m, (xs, ws, gs) in enumerate(linears):
            k = len(specs)
            specs.append(("l%d.m%d.x" % (layer, m), k, xs, _normal(1.0), E4M3))
            specs.append(("l%d.m%d.w" % (layer, m), k + 1, ws,
                          _normal(math.sqrt(1.0 / ws[0])), E4M3))
            specs.append(("l%d.m%d.g" % (layer, m), k + 2, gs, _normal(math.sqrt(1e-4)), E5M2))

    def make_one(sp):  # each tensor from its own streams: the same bytes in any order
        name, k, shape, sampler, fmt = sp
        return QTensor(name, _generate(7, k, shape, np.uint16, sampler, 1), fmt)

    with ThreadPoolExecutor(max(1, th)) as ex:
        tensors = list(ex.map(make_one, specs))
    return Workload("list_%d" % len(tensors),
                    "%d tensors: %d layers x 4 linears x (input, weight, gradient) at hidden "
                    "%d, %d tokens" % (len(tensors), layers, h, t),
                    tensors, history_len=1024, first_scale=[1.0] * len(tensors))


WORKLOADS = {
    "single_1024": single_1024,
    "mlp_4096": mlp_4096,
    "grad_8192x16384": grad_8192x16384,
    "update_1152": update_1152,
    "mlp_12288": mlp_12288,
    "mlp_4096_preact": mlp_4096_preact,
    "list_1152": list_1152,
}


def make(name: str, threads=None) -> Workload:
    return WORKLOADS[name](threads=threads)


# ---------------------------------------------------------------------------------
# Small generic generators for edge-case tests.
# ---------------------------------------------------------------------------------
def random_bf16(n: int, tag: int, lo_exp=-30, hi_exp=30, specials=False) -> np.ndarray:
    """bf16 bit patterns with log-uniform magnitudes 2^[lo_exp, hi_exp), random signs;
    with specials=True a few +-0, +-inf and NaNs are mixed in."""
    g = _rng(100, tag, 0)
    mag = np.exp2(g.uniform(lo_exp, hi_exp, n)).astype(np.float32)
    mag *= np.where(g.random(n) < 0.5, -1, 1).astype(np.float32)
    out = f32_to_bf16_bits(mag)
    if specials and n >= 16:
        idx = g.choice(n, 8, replace=False)
        out[idx] = np.array([0x0000, 0x8000, 0x7F80, 0xFF80, 0x7FC0, 0xFFC1, 0x7F81, 0x0001],
                            np.uint16)
    return out


def random_f32(n: int, tag: int, lo_exp=-30, hi_exp=30) -> np.ndarray:
    g = _rng(101, tag, 0)
    mag = np.exp2(g.uniform(lo_exp, hi_exp, n))
    return (mag * np.where(g.random(n) < 0.5, -1.0, 1.0)).astype(np.float32)


def all_bf16() -> np.ndarray:
    return np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
