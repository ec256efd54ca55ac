"""GPU parity: producer-fused gelu -> FP8 quantize + amax (HIP, through the C ABI) vs
the CPU oracle.

gelu is transcendental, so the bf16 activation y = RN_bf16(gelu(x)) is fixed by the
oracle's double evaluation except within a binary32 error window of a bf16 rounding
midpoint, where the oracle also names the other neighbour.  The bar: each FP8 byte is
the oracle's code of y or of that admissible alternative, and the amax lies between
the smallest and largest amax any admissible choice gives (bit patterns).  Everything
after y (quantize, saturation, amax) is bit-exact as in the plain path."""
import numpy as np
import pytest
import torch

import workloads
from gpu_path import bits, dev_src, f32, note

pytestmark = pytest.mark.gpu

E4M3, E5M2 = 0, 1


def gelu_quantize(x: np.ndarray, fmt: int, scale: float, amax_in: float = 0.0, offset=0):
    """Run the fused entry point on x placed `offset` elements into its buffers."""
    import delayed_scaling_amax_amd as d
    src_all = dev_src(np.concatenate([np.zeros(offset, np.uint16), x]))
    dst_all = torch.zeros(x.size + offset, dtype=torch.uint8, device="cuda")
    s, a = f32([scale]), f32([amax_in])
    d.fp8_gelu_quantize_amax(src_all[offset:], dst_all[offset:], s, a, fmt)
    torch.cuda.synchronize()
    return dst_all[offset:].cpu().numpy(), a.cpu().numpy()[0]


def check(orc, x, fmt, scale, got, got_amax, amax_in=0.0, threads=1):
    """Compare with the oracle; returns the oracle's amax (of its RN choice)."""
    codes, amax_o, codes_alt, lo, hi = orc.gelu_quantize_amax(x, fmt, scale, amax_in=amax_in,
                                                              threads=threads)
    codes, codes_alt = codes.reshape(-1), codes_alt.reshape(-1)
    got = got.reshape(-1)
    bad = np.nonzero((got != codes) & (got != codes_alt))[0]
    xf = x.reshape(-1)
    assert bad.size == 0, (fmt, scale, bad.size,
                           [(hex(xf[j]), hex(got[j]), hex(codes[j]), hex(codes_alt[j]))
                            for j in bad[:6]])
    if np.isnan(lo) or np.isnan(hi):
        assert np.isnan(got_amax)
    else:
        assert bits(lo) <= bits(got_amax) <= bits(hi), (hex(bits(lo)), hex(bits(got_amax)),
                                                       hex(bits(hi)))
    return amax_o


def test_gelu_of_every_bf16_value(orc):
    """Each bf16 pattern alone in a one-element tensor: its amax is |y| itself, so the
    gelu value's magnitude is checked exactly against the oracle (y or its admissible
    neighbour), and its code fixes the sign."""
    import delayed_scaling_amax_amd as d
    x = workloads.all_bf16()
    y, alt = orc.gelu_bf16(x)
    src = dev_src(x)
    dst = torch.zeros(x.size, dtype=torch.uint8, device="cuda")
    amax = torch.zeros(x.size, dtype=torch.float32, device="cuda")
    scale = f32([1.0])
    note("gelu per-element amax, 65536 one-element calls")
    for i in range(x.size):
        d.fp8_gelu_quantize_amax(src[i:i + 1], dst[i:i + 1], scale, amax[i:i + 1], E5M2)
    torch.cuda.synchronize()
    got = amax.cpu().numpy().view(np.uint32)
    want_y = (y.astype(np.uint32) & 0x7FFF) << 16
    want_alt = (alt.astype(np.uint32) & 0x7FFF) << 16
    bad = np.nonzero((got != want_y) & (got != want_alt))[0]
    assert bad.size == 0, [(hex(x[j]), hex(got[j]), hex(want_y[j]), hex(want_alt[j]))
                           for j in bad[:8]]
    codes, _, codes_alt, _, _ = orc.gelu_quantize_amax(x, E5M2, 1.0)
    g = dst.cpu().numpy()
    assert ((g == codes) | (g == codes_alt)).all()
    # how often the binary32 evaluation took the admissible neighbour (reported only)
    print("gelu: %d of %d values took the neighbour" % (int((got != want_y).sum()), x.size))


SCALES = [1.0, 1 / 448, 2.0 ** -7, 0.37, 3.0, 1 / 57344, 2.0 ** 20, 2.0 ** -90, 0.0,
          float("inf"), float("nan"), -1.5]


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_gelu_all_bf16_many_scales(orc, fmt):
    """Every bf16 pattern through the vector body (one aligned tensor) at in-window,
    out-of-window and degenerate scales."""
    x = workloads.all_bf16()
    for s in SCALES:
        note("gelu all bf16 fmt %d scale %r" % (fmt, s))
        got, a = gelu_quantize(x, fmt, s)
        check(orc, x, fmt, s, got, a)


@pytest.mark.parametrize("offset", [0, 1, 3, 7])
def test_gelu_ragged_multi_chunk(orc, offset):
    """Several 32768-element chunks plus a ragged tail, misaligned starts, N(0,3)
    pre-activations with specials; amax accumulates onto a prior value."""
    n = 5 * 32768 + 1237
    x = workloads.random_bf16(n, 900 + offset, lo_exp=-20, hi_exp=6, specials=True)
    g = np.random.Generator(np.random.PCG64(901 + offset))
    normal = workloads.f32_to_bf16_bits((g.standard_normal(n) * 3).astype(np.float32))
    x = np.where(g.random(n) < 0.9, normal, x).astype(np.uint16)
    x[x == 0x7FC0] = 0x3F80      # keep NaNs out of this case so the amax stays finite
    x[(x & 0x7F80) == 0x7F80] = 0x4000
    for fmt, s, a_in in ((E4M3, 0.05, 0.0), (E5M2, 1e-3, 2.5), (E4M3, 2.0 ** -100, 0.0)):
        note("gelu ragged n=%d offset=%d fmt %d scale %r" % (n, offset, fmt, s))
        got, a = gelu_quantize(x, fmt, s, amax_in=a_in, offset=offset)
        check(orc, x, fmt, s, got, a, amax_in=a_in)


def test_gelu_small_and_empty(orc):
    import delayed_scaling_amax_amd as d
    for n in (1, 2, 7, 8, 9, 15, 16, 17, 255):
        x = workloads.random_bf16(n, 950 + n, lo_exp=-8, hi_exp=4)
        for offset in (0, 5):
            note("gelu small n=%d offset=%d" % (n, offset))
            got, a = gelu_quantize(x, E4M3, 0.125, offset=offset)
            check(orc, x, E4M3, 0.125, got, a)
    # numel 0 enqueues nothing: amax untouched
    src = torch.zeros(4, dtype=torch.bfloat16, device="cuda")
    dst = torch.zeros(4, dtype=torch.uint8, device="cuda")
    a = f32([1.25])
    d.fp8_gelu_quantize_amax(src[:0], dst[:0], f32([1.0]), a, E4M3)
    torch.cuda.synchronize()
    assert a.item() == 1.25 and not dst.any()


def test_gelu_rejects_f32_sources():
    import delayed_scaling_amax_amd as d
    src = torch.zeros(16, dtype=torch.float32, device="cuda")
    dst = torch.zeros(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(d.Fp8qError):
        d.fp8_gelu_quantize_amax(src, dst, f32([1.0]), f32([0.0]), E4M3)


def test_gelu_full_size_mlp_4096_preact(orc):
    """The (2048,4,16384) FFN pre-activation at its full size, two delayed-scaling
    steps: the first at scale 1, the second at the scale the oracle's first-step amax
    gives (amax / 448), both checked element by element."""
    import delayed_scaling_amax_amd as d
    w = workloads.make("mlp_4096_preact")
    x = w.tensors[0].data.reshape(-1)
    src = dev_src(x)
    dst = torch.empty(x.size, dtype=torch.uint8, device="cuda")
    scale = 1.0
    for step in range(2):
        note("gelu full size step %d scale %r" % (step, scale))
        a = f32([0.0])
        d.fp8_gelu_quantize_amax(src, dst, f32([scale]), a, E4M3)
        torch.cuda.synchronize()
        amax_o = check(orc, x, E4M3, scale, dst.cpu().numpy(), a.cpu().numpy()[0], threads=8)
        scale = float(np.float32(amax_o) / np.float32(448.0))
