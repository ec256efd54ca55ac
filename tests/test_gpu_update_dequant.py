"""GPU parity: batched amax_and_scale_update and dequantize vs the CPU oracle.

Bit-exact on history, amax, scale and scale_inv (0 ulp), and on dequantized values."""
import numpy as np
import pytest
import torch

import workloads
from gpu_path import bits, f32, note

pytestmark = pytest.mark.gpu


def run_update(amax, hist, scale, formats, algo=0, margin=0, reset=False):
    import delayed_scaling_amax_amd as d
    a = torch.from_numpy(np.ascontiguousarray(amax, np.float32)).cuda()
    h = torch.from_numpy(np.ascontiguousarray(hist, np.float32)).cuda()
    s = torch.from_numpy(np.ascontiguousarray(scale, np.float32)).cuda()
    si = torch.full_like(s, -7.0)
    f = torch.from_numpy(np.ascontiguousarray(formats, np.uint8)).cuda()
    d.fp8_amax_and_scale_update(a, h, s, si, f, algo=algo, margin=margin, reset_amax=reset)
    torch.cuda.synchronize()
    return dict(amax=a.cpu().numpy(), hist=h.cpu().numpy(), scale=s.cpu().numpy(),
                scale_inv=si.cpu().numpy())


def check_update(orc, amax, hist, scale, formats, **kw):
    got = run_update(amax, hist, scale, formats, **kw)
    want = orc.amax_and_scale_update(amax, hist, scale, formats, algo=kw.get("algo", 0),
                                     margin=kw.get("margin", 0),
                                     reset_amax=kw.get("reset", False))
    for k in ("hist", "scale", "scale_inv", "amax"):
        gb, wb = bits(got[k]), bits(want[k])
        bad = np.argwhere(gb != wb)
        assert bad.size == 0, (k, bad[:5].tolist())


def lognormal(shape, tag):
    g = np.random.Generator(np.random.PCG64(tag))
    return g.lognormal(0, 2, shape).astype(np.float32)


@pytest.mark.parametrize("margin", [0, 1])
@pytest.mark.parametrize("algo", [0, 1])
def test_update_1152_workload(orc, margin, algo):
    w = workloads.update_1152()
    fm = np.array([workloads.E5M2 == f for f in w.formats], np.uint8)
    note("update_1152 margin %d algo %d" % (margin, algo))
    check_update(orc, w.amax, w.hist, w.scale, fm, algo=algo, margin=margin)


@pytest.mark.parametrize("n,H", [(1, 1), (1, 16), (3, 16), (5, 1024), (4, 2), (7, 3),
                                 (1151, 1024), (1152, 1023), (1152, 1025), (12, 2049),
                                 (64, 4100), (9, 1), (4, 1025), (8, 1026), (1152, 1026),
                                 (1156, 2), (6, 1026)])
def test_update_shapes(orc, n, H):
    g = np.random.Generator(np.random.PCG64(n * 7919 + H))
    amax = lognormal(n, n + H)
    hist = lognormal((H, n), n * H + 1)
    scale = np.exp2(g.uniform(-4, 4, n)).astype(np.float32)
    fm = (g.random(n) < 0.4).astype(np.uint8) * np.uint8(g.integers(1, 255))
    note("update n=%d H=%d" % (n, H))
    check_update(orc, amax, hist, scale, fm, margin=int(g.integers(-3, 4)),
                 reset=bool(n % 2))


def test_update_special_amaxes(orc):
    amax = np.array([0.0, np.inf, np.nan, 1e-45, 3e38, 1e-30, 5.0, 0.0], np.float32)
    hist = np.zeros((4, 8), np.float32)
    hist[2, 7] = 9.0
    hist[1, 6] = np.nan
    scale = np.array([0.5, 0.25, 2.0, 4.0, 8.0, 1.0, 1.0, 1.0], np.float32)
    fm = np.array([0, 1, 0, 1, 0, 1, 0, 1], np.uint8)
    note("update special amaxes")
    for margin in (0, 5, 126, -126):
        for algo in (0, 1):
            check_update(orc, amax, hist, scale, fm, margin=margin, algo=algo, reset=True)


def test_update_sequence_matches_oracle(orc):
    """k successive in-place updates (device history kept resident) equal k oracle steps."""
    import delayed_scaling_amax_amd as d
    n, H = 37, 8
    h = torch.zeros(H, n, dtype=torch.float32, device="cuda")
    s = torch.ones(n, dtype=torch.float32, device="cuda")
    si = torch.empty_like(s)
    f = torch.from_numpy((np.arange(n) % 3 == 2).astype(np.uint8)).cuda()
    hw, sw = np.zeros((H, n), np.float32), np.ones(n, np.float32)
    note("update sequence")
    for step in range(12):
        amax_np = lognormal(n, 1000 + step)
        a = torch.from_numpy(amax_np).cuda()
        d.fp8_amax_and_scale_update(a, h, s, si, f, reset_amax=True)
        r = orc.amax_and_scale_update(amax_np, hw, sw, f.cpu().numpy(), reset_amax=True)
        hw, sw = r["hist"], r["scale"]
    torch.cuda.synchronize()
    assert (bits(h.cpu().numpy()) == bits(hw)).all()
    assert (bits(s.cpu().numpy()) == bits(sw)).all()
    assert (bits(si.cpu().numpy()) == bits(r["scale_inv"])).all()


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_dequantize_all_codes(orc, fmt, out):
    import delayed_scaling_amax_amd as d
    codes = np.tile(np.arange(256, dtype=np.uint8), 37)
    for s in (1.0, 0.0123, 3.7e4, 2.0 ** -20, 3e36, 1.7e-41, 0.0, float("inf")):
        note("dequant fmt %d %s scale %g" % (fmt, out, s))
        src = torch.from_numpy(codes).cuda()
        dst = torch.empty(codes.size, dtype=torch.float32 if out == "f32" else torch.bfloat16,
                          device="cuda")
        d.fp8_dequantize(src, dst, f32([s]), fmt)
        torch.cuda.synchronize()
        got = dst.cpu().view(torch.int32 if out == "f32" else torch.int16).numpy()
        want = orc.dequantize(codes, fmt, s, out_dtype=1 if out == "f32" else 0)
        ut = np.uint32 if out == "f32" else np.uint16
        assert (got.view(ut) == want.view(ut)).all()


def test_dequantize_ragged_misaligned(orc):
    import delayed_scaling_amax_amd as d
    g = np.random.Generator(np.random.PCG64(5))
    codes_np = g.integers(0, 256, 20_000).astype(np.uint8)
    codes = torch.from_numpy(codes_np).cuda()
    for out in ("f32", "bf16"):
        buf = torch.zeros(20_100, dtype=torch.float32 if out == "f32" else torch.bfloat16,
                          device="cuda")
        for n in (0, 1, 7, 8, 9, 257, 4099, 19_000):
            for so, do in ((0, 0), (1, 0), (3, 5), (8, 2)):
                note("dequant ragged %s n=%d so=%d do=%d" % (out, n, so, do))
                buf.fill_(-3.0)
                d.fp8_dequantize(codes[so:so + n], buf[do:do + n], f32([0.75]), n % 2)
                torch.cuda.synchronize()
                want = orc.dequantize(codes_np[so:so + n], n % 2, 0.75,
                                      out_dtype=1 if out == "f32" else 0)
                b = buf.cpu().view(torch.int32 if out == "f32" else torch.int16).numpy()
                b = b.view(np.uint32 if out == "f32" else np.uint16)
                assert (b[do:do + n] == want.view(b.dtype)).all()
                fill = np.float32(-3.0).view(np.uint32)
                fill = fill if out == "f32" else np.uint16(fill >> 16)
                assert (b[:do] == fill).all() and (b[do + n:] == fill).all()
