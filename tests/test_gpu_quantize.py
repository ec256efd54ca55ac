"""GPU parity: fused quantize + amax (HIP, through the C ABI) vs the CPU oracle.

The bar is bit-exact: every FP8 byte and the amax bit pattern."""
import numpy as np
import pytest
import torch

import workloads
from gpu_path import bits, dev_src, f32, note, quantize

pytestmark = pytest.mark.gpu

E4M3, E5M2 = 0, 1


def scales_grid():
    g = np.random.Generator(np.random.PCG64(77))
    s = [1.0, 1 / 448, 1 / 57344, 2.0, 0.5, 3.0, 1e-3, 7.123e4,
         float(workloads.stale_grad_scale())]
    s += [2.0 ** e for e in range(-80, 126, 9)]
    s += list(np.exp2(g.uniform(-40, 40, 24)))
    return [float(np.float32(v)) for v in s]


# scales outside the fast window or degenerate: IEEE path, NaN, inf, sign flips
ODD_SCALES = [2.0 ** -90, 2.0 ** -126, 1e-40, 2.0 ** -149, 2.0 ** 126, 3.0e38, -3.0e30, 0.0,
              -0.0, -1.5, float("inf"), float("-inf"), float("nan")]


def test_worked_tensor(orc):
    note("worked tensor")
    x = np.array([0x3F00, 0xBF80, 0x4040, 0x0000, 0x8000, 0x447A, 0x3980, 0x40E0], np.uint16)
    for fmt in (E4M3, E5M2):
        for s in (1.0, float(np.uint32(0x400EDB6E).view(np.float32))):
            got, a = quantize(x, fmt, s)
            want, wa = orc.quantize_amax(x, fmt, s)
            assert got.tobytes() == want.tobytes()
            assert bits(a) == bits(wa)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_all_bf16_many_scales(orc, fmt):
    """Every bf16 bit pattern (incl. +-0, subnormals, +-inf, NaNs) x ~60 scales."""
    import delayed_scaling_amax_amd as d
    x = workloads.all_bf16()
    src = dev_src(x)
    scales = scales_grid() + ODD_SCALES
    note("all bf16 x %d scales fmt %d" % (len(scales), fmt))
    dsts = [torch.empty(x.size, dtype=torch.uint8, device="cuda") for _ in scales]
    s_dev = f32(scales)
    a_dev = torch.zeros(len(scales), dtype=torch.float32, device="cuda")
    d.fp8_multi_quantize_amax([(src, dsts[i], s_dev[i:i + 1], a_dev[i:i + 1], fmt)
                               for i in range(len(scales))])
    torch.cuda.synchronize()
    amaxes = a_dev.cpu().numpy()
    for i, s in enumerate(scales):
        want, wa = orc.quantize_amax(x, fmt, s)
        got = dsts[i].cpu().numpy()
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, (s, [(hex(x[j]), hex(got[j]), hex(want[j])) for j in bad[:6]])
        assert bits(amaxes[i]) == bits(wa)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_convert_sweep_f32(orc, fmt):
    """Scale 1.0 on fp32 sources: the quotient is x itself, so this checks saturation
    and the native convert on every upper-16-bit pattern with low-bit patterns that
    set the round and sticky bits of both formats (ties included)."""
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x4000, 0xC000],
                    np.uint32)
    x = (hi[:, None] | lows[None, :]).reshape(-1).view(np.float32)
    note("convert sweep fp32 fmt %d" % fmt)
    got, a = quantize(x, fmt, 1.0)
    want, wa = orc.quantize_amax(x, fmt, 1.0, threads=8)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(hex(x.view(np.uint32)[j]), hex(got[j]), hex(want[j])) for j in bad[:6]]
    assert bits(a) == bits(wa)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
@pytest.mark.parametrize("scale", [1.0, 0.0173, 2.3e-7, 5.5e3, 2.0 ** -100, float("inf")])
def test_random_f32(orc, fmt, scale):
    x = workloads.random_f32(300_000, 5, -40, 40)
    x[::9973] = np.float32(np.nan)
    x[1::9973] = np.float32(-np.inf)
    x[2::9973] = np.float32(1e-42)
    note("random f32 fmt %d scale %g" % (fmt, scale))
    got, a = quantize(x, fmt, scale)
    want, wa = orc.quantize_amax(x, fmt, scale)
    assert got.tobytes() == want.tobytes()
    assert bits(a) == bits(wa)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ragged_and_misaligned(orc, dtype):
    """Sizes around the vector group and tile boundaries, and views whose source and
    destination start at every byte offset (aligned-alike and not)."""
    import delayed_scaling_amax_amd as d
    base_np = (workloads.random_bf16(70_000, 9, -12, 12, specials=True) if dtype == "bf16"
               else workloads.random_f32(70_000, 9, -12, 12))
    base = dev_src(base_np)
    out = torch.zeros(70_000 + 64, dtype=torch.uint8, device="cuda")
    sizes = [0, 1, 2, 7, 8, 9, 15, 16, 17, 255, 256, 257, 2047, 2048, 2049, 8191, 8193,
             33_331, 65_537]
    for n in sizes:
        for so, do in ((0, 0), (1, 1), (3, 3), (0, 5), (2, 13), (7, 0), (4, 4)):
            if so + n > base.numel():
                continue
            note("ragged %s n=%d src_off=%d dst_off=%d" % (dtype, n, so, do))
            src = base[so:so + n]
            dst = out[do:do + n]
            out.fill_(0xAB)
            s, a = f32([0.37]), f32([0.0])
            d.fp8_quantize_amax(src, dst, s, a, E4M3 if n % 2 else E5M2)
            torch.cuda.synchronize()
            want, wa = orc.quantize_amax(base_np[so:so + n], E4M3 if n % 2 else E5M2, 0.37)
            o = out.cpu().numpy()
            assert o[do:do + n].tobytes() == want.tobytes(), (n, so, do)
            assert (o[:do] == 0xAB).all() and (o[do + n:] == 0xAB).all(), "wrote out of range"
            assert bits(a.cpu().numpy()[0]) == bits(wa)


def test_multi_tensor_mixed_and_shared_amax(orc):
    """40 entries (two launches of 32 + 8), mixed dtypes/formats/sizes/scales, some
    entries sharing one amax, one empty entry."""
    import delayed_scaling_amax_amd as d
    g = np.random.Generator(np.random.PCG64(99))
    entries, host = [], []
    amax = torch.zeros(20, dtype=torch.float32, device="cuda")
    scales = f32(np.exp2(g.uniform(-8, 8, 40)))
    for i in range(40):
        n = int(g.integers(0, 50_000)) if i != 7 else 0
        x = (workloads.random_bf16(n, 200 + i, -10, 10) if i % 3 else
             workloads.random_f32(n, 200 + i, -10, 10))
        fmt = int(g.integers(0, 2))
        dst = torch.empty(n, dtype=torch.uint8, device="cuda")
        slot = i % 20
        entries.append((dev_src(x), dst, scales[i:i + 1], amax[slot:slot + 1], fmt))
        host.append((x, fmt, slot, dst))
    note("multi-tensor 40 entries")
    d.fp8_multi_quantize_amax(entries)
    torch.cuda.synchronize()
    sc = scales.cpu().numpy()
    want_amax = np.zeros(20, np.float32)
    for i, (x, fmt, slot, dst) in enumerate(host):
        want, wa = orc.quantize_amax(x, fmt, float(sc[i]), amax_in=want_amax[slot])
        want_amax[slot] = wa
        assert dst.cpu().numpy().tobytes() == want.tobytes(), i
    assert (bits(amax.cpu().numpy()) == bits(want_amax)).all()


def test_out_of_window_tensors_inside_one_run(orc):
    """One launch of five bf16 E4M3 tensors spanning several 16384-element chunks per
    block, the first and the fourth with scales outside the division window (done
    element-wise in the second phase): blocks whose first chunk lies in the first tensor
    have their speculative first loads discarded and reload from the second, and the
    pipeline skips the fourth tensor mid-run.  Codes and amaxes against the oracle."""
    import delayed_scaling_amax_amd as d
    sizes = [3_000_000, 5_000_123, 2_000_007, 4_000_000, 1_000_005]
    scales = [2.0 ** -90, 0.37, 1.7, 3.0e38, 0.05]
    note("out-of-window tensors inside one run")
    entries, host = [], []
    amax = torch.zeros(len(sizes), dtype=torch.float32, device="cuda")
    sc = f32(scales)
    for i, n in enumerate(sizes):
        x = workloads.random_bf16(n, 700 + i, -12, 12)
        dst = torch.empty(n, dtype=torch.uint8, device="cuda")
        entries.append((dev_src(x), dst, sc[i:i + 1], amax[i:i + 1], E4M3))
        host.append((x, dst))
    d.fp8_multi_quantize_amax(entries)
    torch.cuda.synchronize()
    got_amax = amax.cpu().numpy()
    for i, (x, dst) in enumerate(host):
        want, wa = orc.quantize_amax(x, E4M3, float(np.float32(scales[i])),
                                     threads=workloads.default_threads())
        bad = np.flatnonzero(dst.cpu().numpy() != want)
        assert bad.size == 0, (i, bad[:8], bad.size)
        assert bits(got_amax[i]) == bits(wa), i


def test_amax_max_accumulates_and_is_deterministic(orc):
    import delayed_scaling_amax_amd as d
    x1 = workloads.random_bf16(1 << 20, 31, -5, 5)
    x2 = workloads.random_bf16(1 << 19, 32, -3, 9)
    s1, s2 = dev_src(x1), dev_src(x2)
    a = f32([0.0])
    s = f32([0.01])
    outs = []
    note("amax accumulation")
    for rep in range(2):
        a.zero_()
        o1 = torch.empty(x1.size, dtype=torch.uint8, device="cuda")
        o2 = torch.empty(x2.size, dtype=torch.uint8, device="cuda")
        d.fp8_quantize_amax(s1, o1, s, a, E4M3)
        d.fp8_quantize_amax(s2, o2, s, a, E4M3)
        torch.cuda.synchronize()
        outs.append((o1.cpu().numpy(), o2.cpu().numpy(), a.cpu().numpy()[0]))
    _, a1 = orc.quantize_amax(x1, E4M3, 0.01)
    _, a12 = orc.quantize_amax(x2, E4M3, 0.01, amax_in=a1)
    assert bits(outs[0][2]) == bits(a12)
    for k in range(3):
        assert np.array_equal(np.atleast_1d(outs[0][k]).view(np.uint8),
                              np.atleast_1d(outs[1][k]).view(np.uint8))


def test_timed_form_matches_oracle(orc):
    """fp8_multi_quantize_amax_timed: the same codes and amaxes as the oracle over 40
    entries (two launches: start taken by the first, stop by the last), events that
    bound a positive interval no longer than the stream events around the call, and an
    empty call that still records both events."""
    import delayed_scaling_amax_amd as d
    g = np.random.Generator(np.random.PCG64(4242))
    n = 40
    # bf16 (truncated binary32) N(0, 100) tensors of ragged sizes
    xs = [((g.standard_normal(int(g.integers(1, 70000))) * 10).astype(np.float32)
           .view(np.uint32) >> 16).astype(np.uint16) for _ in range(n)]
    fmts = [i % 2 for i in range(n)]
    scales = [float(np.float32(2.0 ** g.uniform(-8, 4))) for _ in range(n)]
    note("timed form: %d entries, %d elements" % (n, sum(x.size for x in xs)))
    srcs = [dev_src(x) for x in xs]
    dsts = [torch.empty(x.size, dtype=torch.uint8, device="cuda") for x in xs]
    s_dev, a_dev = f32(scales), torch.zeros(n, dtype=torch.float32, device="cuda")
    outer = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    inner = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    outer[0].record()
    d.fp8_multi_quantize_amax_timed([(srcs[i], dsts[i], s_dev[i:i + 1], a_dev[i:i + 1],
                                      fmts[i]) for i in range(n)], inner[0], inner[1])
    outer[1].record()
    torch.cuda.synchronize()
    amaxes = a_dev.cpu().numpy()
    for i in range(n):
        want, wa = orc.quantize_amax(xs[i], fmts[i], scales[i])
        assert dsts[i].cpu().numpy().tobytes() == want.tobytes(), i
        assert bits(amaxes[i]) == bits(wa), i
    t_in, t_out = inner[0].elapsed_time(inner[1]), outer[0].elapsed_time(outer[1])
    assert 0.0 < t_in <= t_out + 1e-3, (t_in, t_out)
    e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    d.fp8_multi_quantize_amax_timed([], e[0], e[1])
    torch.cuda.synchronize()
    assert e[0].elapsed_time(e[1]) >= 0.0
