"""GPU parity: LayerNorm-output -> FP8 quantize + amax (HIP, through the C ABI) vs the
CPU oracle.

The LayerNorm value is irrational in general, so y = RN_bf16(LN(x)) is fixed by the
oracle's double evaluation up to the error window of a binary32 evaluation: the oracle
returns the admissible bf16 range [RN(y - w), RN(y + w)] (y alone away from rounding
midpoints).  The bar: each FP8 byte decodes to a value between the codes of the
range's ends (the quantize is monotone), the amax lies between the smallest and largest
amax any admissible choice gives (bit patterns), everything after y is bit-exact, and
the per-row mean and rstd are within the binary32 evaluation's error bound of the exact
values."""
import math

import numpy as np
import pytest
import torch

import workloads
from gpu_path import bits, dev_src, f32, note

pytestmark = pytest.mark.gpu

E4M3, E5M2 = 0, 1


def bf16_f64(x: np.ndarray) -> np.ndarray:
    return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def run_ln(x, fmt, scale, gamma=None, beta=None, eps=1e-6, amax_in=0.0, stats=True):
    import delayed_scaling_amax_amd as d
    rows, H = x.shape
    src = dev_src(x.reshape(-1)).view(rows, H)
    dst = torch.zeros(rows * H, dtype=torch.uint8, device="cuda")
    s, a = f32([scale]), f32([amax_in])
    g = None if gamma is None else torch.from_numpy(gamma).cuda()
    b = None if beta is None else torch.from_numpy(beta).cuda()
    mean = torch.full((rows,), float("nan"), device="cuda") if stats else None
    rstd = torch.full((rows,), float("nan"), device="cuda") if stats else None
    d.fp8_layernorm_quantize_amax(src, dst, s, a, fmt, gamma=g, beta=b, eps=eps, mean=mean,
                                  rstd=rstd)
    torch.cuda.synchronize()
    return (dst.cpu().numpy().reshape(rows, H), a.cpu().numpy()[0],
            None if mean is None else mean.cpu().numpy(),
            None if rstd is None else rstd.cpu().numpy())


def check_ln(orc, x, fmt, scale, gamma=None, beta=None, eps=1e-6, amax_in=0.0, threads=1,
             stats=True):
    got, got_amax, gmean, grstd = run_ln(x, fmt, scale, gamma, beta, eps, amax_in, stats)
    codes, amax_o, c_lo, c_hi, lo, hi, mean, rstd = orc.layernorm_quantize_amax(
        x, fmt, scale, gamma, beta, eps, amax_in=amax_in, threads=threads)
    table = decode_table(orc, fmt)
    dl, dh, dg = table[c_lo], table[c_hi], table[got]
    in_range = (dg >= np.minimum(dl, dh)) & (dg <= np.maximum(dl, dh))
    nan_case = np.isnan(dl) | np.isnan(dh) | np.isnan(dg)
    ok = in_range | (nan_case & ((got == c_lo) | (got == c_hi) | (got == codes)))
    bad = np.nonzero(~ok)
    assert bad[0].size == 0, (fmt, scale, bad[0].size,
                              [(r, c, hex(x[r, c]), hex(got[r, c]), hex(codes[r, c]),
                                hex(c_lo[r, c]), hex(c_hi[r, c])) for r, c in zip(*bad)][:6])
    print("ln: %d of %d codes differ from the code of y (inside the admissible range)"
          % (int((got != codes).sum()), got.size))
    if np.isnan(lo) or np.isnan(hi):
        assert np.isnan(got_amax)
    else:
        assert bits(lo) <= bits(got_amax) <= bits(hi), (hex(bits(lo)), hex(bits(got_amax)),
                                                       hex(bits(hi)))
    if stats:
        H = x.shape[1]
        L = math.ceil(math.log2(H)) + 10
        xf = bf16_f64(x)
        fin = np.isfinite(mean)
        A = np.abs(xf).mean(axis=1)
        Ad = np.abs(xf - np.where(fin, mean, 0)[:, None]).mean(axis=1)
        u = 2.0 ** -24
        tol_m = 2 * u * (L * Ad + 2 * np.abs(mean) + L * L * u * A) + 2.0 ** -140
        r2 = np.where(fin, rstd, 0) ** 2
        tol_r = 2 * u * (L / 2 + 5 + L * L * u * A * Ad * r2) * np.abs(rstd)
        assert np.array_equal(np.isnan(gmean), ~fin) and np.array_equal(np.isnan(grstd), ~fin)
        assert (np.abs(gmean[fin] - mean[fin]) <= tol_m[fin]).all(), \
            np.max(np.abs(gmean[fin] - mean[fin]) / tol_m[fin])
        ok_r = np.isinf(rstd[fin]) | (np.abs(grstd[fin] - rstd[fin]) <= tol_r[fin])
        assert ok_r.all(), np.max(np.abs(grstd[fin] - rstd[fin]) / tol_r[fin])
    return amax_o


_TABLES = {}


def decode_table(orc, fmt):
    if fmt not in _TABLES:
        _TABLES[fmt] = np.array([orc.decode(fmt, c) for c in range(256)], np.float64)
    return _TABLES[fmt]


def ln_input(seed, rows, H, offset=0.0, spread=1.0):
    g = np.random.Generator(np.random.PCG64(seed))
    v = (g.standard_normal(rows * H) * spread + offset).astype(np.float32)
    return workloads.f32_to_bf16_bits(v).reshape(rows, H)


def affine(seed, H):
    g = np.random.Generator(np.random.PCG64(seed))
    return ((1 + 0.2 * g.standard_normal(H)).astype(np.float32),
            (0.3 * g.standard_normal(H)).astype(np.float32))


@pytest.mark.parametrize("H", [8, 64, 512, 520, 768, 1000, 2048, 4096, 8192, 10000, 12288,
                               12296, 16384])
def test_ln_row_lengths(orc, H):
    """Every kernel instance (units per lane 1-32, full and masked) over several rows,
    affine gamma/beta, both formats; 12288 is the hidden size of the hidden-12288 MLP."""
    for rows, fmt, scale in ((1, E4M3, 0.02), (37, E5M2, 1e-3), (131, E4M3, 0.013)):
        x = ln_input(700 + H + rows, rows, H, offset=0.3)
        gamma, beta = affine(800 + H, H)
        note("ln H=%d rows=%d fmt %d" % (H, rows, fmt))
        check_ln(orc, x, fmt, scale, gamma, beta)


def test_ln_without_affine_and_without_stats(orc):
    x = ln_input(710, 64, 4096)
    note("ln no gamma/beta, no stats")
    check_ln(orc, x, E4M3, 1 / 64, stats=False)
    check_ln(orc, x, E4M3, 1 / 64, gamma=affine(711, 4096)[0])


def test_ln_special_rows(orc):
    """Constant rows (y = beta exactly at eps > 0; NaN at eps = 0), rows with inf/NaN,
    rows whose mean dwarfs their spread, subnormal-valued rows, +-a rows."""
    H = 1024
    x = ln_input(720, 16, H)
    x[0] = 0x4040                                     # constant 3.0
    x[1, 17] = 0x7F80                                 # +inf
    x[2, 5] = 0xFFC1                                  # NaN
    x[3] = ln_input(721, 1, H, offset=1e4, spread=5.0)   # mean >> spread
    x[4] = ln_input(722, 1, H, offset=-300.0, spread=0.3)
    x[5] = (np.arange(H) % 7 + 1).astype(np.uint16)   # bf16 subnormals
    x[6] = np.where(np.arange(H) % 2 == 0, 0x4040, 0xC040)   # +-3
    x[7, :] = 0x3F80
    x[7, 0] = 0x3F81                                  # one ulp above a constant row
    gamma, beta = affine(723, H)
    for eps in (1e-6, 1e-3, 0.0):
        # at eps = 0 the subnormal row's variance (~2^-266) underflows binary32, where
        # any binary32 evaluation departs from the exact value: that row only with eps > 0
        sel = [0, 3, 4, 5, 6, 7, 8] if eps > 0 else [0, 3, 4, 6, 7, 8]
        note("ln special rows eps=%r" % eps)
        check_ln(orc, x[sel], E4M3, 0.02, gamma, beta, eps=eps)
    note("ln nonfinite rows")
    check_ln(orc, x, E4M3, 0.02, gamma, beta, eps=1e-6)


@pytest.mark.parametrize("H", [1024, 4096])
def test_ln_nonfinite_beta_and_huge_gamma(orc, H):
    """beta with a NaN and an inf column (every row's y there is NaN / inf: the kernel's
    per-unit NaN handling stays on for the whole launch), and gamma of 1e38 in a few
    columns with finite beta (y overflows to +-inf there, never to NaN, in rows the kernel
    treats as giving no NaN)."""
    x = ln_input(740 + H, 8, H, offset=0.25)
    gamma, beta = affine(741, H)
    b2 = beta.copy()
    b2[3], b2[H - 2] = np.float32(np.nan), np.float32(np.inf)
    note("ln H=%d beta with NaN and inf" % H)
    check_ln(orc, x, E4M3, 0.02, gamma, b2)
    g2 = gamma.copy()
    g2[[1, 100, H - 1]] = np.float32(1e38)
    note("ln H=%d gamma 1e38 in 3 columns" % H)
    check_ln(orc, x, E5M2, 1.0, g2, beta)


@pytest.mark.parametrize("H", [1000, 4096, 8192])
def test_ln_saturating_scales(orc, H):
    """Scales inside the division window at which most units hold quotients beyond
    FP8_MAX (the saturating form of the codes) in rows that give no NaN, and a column of
    gamma 3e38 whose y overflows to +-inf there (the fixed-code patch in the same rows)."""
    x = ln_input(760 + H, 12, H, offset=0.1)
    gamma, beta = affine(761 + H, H)
    for fmt, scale in ((E4M3, 1 / 512), (E5M2, 2.0 ** -15)):
        note("ln H=%d saturating scale %r fmt %d" % (H, scale, fmt))
        check_ln(orc, x, fmt, scale, gamma, beta)
    g2 = gamma.copy()
    g2[H // 2] = np.float32(3e38)
    note("ln H=%d saturating scale with an overflowing column" % H)
    check_ln(orc, x, E4M3, 1 / 512, g2, beta)


@pytest.mark.parametrize("scale", [2.0 ** -100, 0.0, float("inf"), float("nan"), -0.5, 3e38])
def test_ln_odd_scales(orc, scale):
    x = ln_input(730, 24, 768)
    gamma, beta = affine(731, 768)
    note("ln scale %r" % scale)
    check_ln(orc, x, E5M2, scale, gamma, beta)


def test_ln_amax_accumulates(orc):
    x = ln_input(740, 8, 512)
    note("ln amax accumulation")
    check_ln(orc, x, E4M3, 0.05, amax_in=1e6)
    check_ln(orc, x, E4M3, 0.05, amax_in=0.5)


def test_ln_empty_and_rejections():
    import delayed_scaling_amax_amd as d
    x = torch.zeros(0, 64, dtype=torch.bfloat16, device="cuda")
    dst = torch.zeros(0, dtype=torch.uint8, device="cuda")
    a = f32([1.25])
    d.fp8_layernorm_quantize_amax(x, dst, f32([1.0]), a, E4M3)
    torch.cuda.synchronize()
    assert a.item() == 1.25
    xb = torch.zeros(4, 65, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(d.Fp8qError):      # hidden not a multiple of 8
        d.fp8_layernorm_quantize_amax(xb, torch.zeros(4 * 65, dtype=torch.uint8,
                                                      device="cuda"), f32([1.0]), a, E4M3)
    big = torch.zeros(8 * 64 + 1, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(d.Fp8qError):      # source not 16-byte aligned
        d.fp8_layernorm_quantize_amax(big[1:].view(8, 64), torch.zeros(8 * 64, dtype=torch.uint8,
                                                                       device="cuda"),
                                      f32([1.0]), a, E4M3)


def test_ln_full_size_transformer_input(orc):
    """The reproducer's LayerNorm input, (2048,4,4096) ~ U[0,1) (the mlp_4096
    activation), at full size: two delayed-scaling steps (scale 1, then the oracle's
    amax / 448), once with the layer's initial gamma = 1, beta = 0 and once with
    random gamma/beta."""
    w = workloads.make("mlp_4096")
    x = w.tensors[0].data.reshape(-1, 4096)
    gamma, beta = affine(750, 4096)
    for g, b in ((None, None), (gamma, beta)):
        scale = 1.0
        for step in range(2):
            note("ln full size affine=%s step %d scale %r" % (g is not None, step, scale))
            amax_o = check_ln(orc, x, E4M3, scale, g, b, threads=8)
            scale = float(np.float32(amax_o) / np.float32(448.0))
