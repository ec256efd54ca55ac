"""GPU parity: FP8 GEMM with per-tensor scales (HIP matrix cores, through the C ABI) vs
the exact CPU oracle.

The FP8 products are exact. The gfx950 matrix core sums each aligned group of 8
consecutive products in fixed point, keeping 13 bits below the group's largest product
(smaller products are truncated toward zero to that grid), and accumulates the group
sums in binary32 (test_gemm_accumulation_model pins this on crafted dot products). The
bar is the resulting error bound around the exact value (computed by the oracle in
128-bit fixed point), plus the final rounding to the output type:
    |C - exact| <= (2^-10 G + 2^-24 (ceil(K/8) + 2) S) |sa sb|   (+ the output rounding)
with G = sum over k-groups of the group's largest |a_k b_k| and S = sum_k |a_k b_k|.
NaN operands must give NaN."""
import math

import numpy as np
import pytest
import torch

from gpu_path import f32, note

pytestmark = pytest.mark.gpu

E4M3, E5M2 = 0, 1


def random_codes(g, shape, fmt, spread=True):
    """Finite FP8 codes: uniform over all finite codes, or (spread=False) the values an
    activation quantized with a fitted scale takes (a normal distribution)."""
    if spread:
        c = g.integers(0, 256, shape).astype(np.uint8)
    else:
        dt = torch.float8_e4m3fn if fmt == E4M3 else torch.float8_e5m2
        v = torch.from_numpy(g.standard_normal(shape).astype(np.float32) * 40)
        c = v.to(dt).view(torch.uint8).numpy()
    if fmt == E4M3:
        c[(c & 0x7F) == 0x7F] = 0x38
    else:
        c[(c & 0x7C) == 0x7C] = 0x3C
    return c


def run_gemm(A, fa, B, fb, sa, sb, out_dtype):
    import delayed_scaling_amax_amd as d
    M, K = A.shape
    N = B.shape[0]
    Ad = torch.from_numpy(A).cuda()
    Bd = torch.from_numpy(B).cuda()
    C = torch.full((M, N), float("nan"), dtype=out_dtype, device="cuda")
    d.fp8_gemm(Ad, fa, Bd, fb, f32([sa]), f32([sb]), C)
    torch.cuda.synchronize()
    return C.float().cpu().numpy().astype(np.float64)


def acc_bound(K, cabs, cgmax):
    return 2.0 ** -10 * cgmax + 2.0 ** -24 * (math.ceil(K / 8) + 2) * cabs


def check(orc, A, fa, B, fb, sa=1.0, sb=1.0, out_dtype=torch.bfloat16, threads=1):
    got = run_gemm(A, fa, B, fb, sa, sb, out_dtype)
    exact, cabs, cg = orc.fp8_gemm(A, fa, B, fb, sa, sb, threads=threads)
    K = A.shape[1]
    acc_tol = acc_bound(K, cabs, cg)
    if out_dtype == torch.bfloat16:
        tol = acc_tol + 2.0 ** -8 * (np.abs(exact) + acc_tol) + 2.0 ** -133
    else:
        tol = acc_tol + 2.0 ** -23 * (np.abs(exact) + acc_tol) + 2.0 ** -149
    nan = np.isnan(exact)
    assert (np.isnan(got) == nan).all(), (np.argwhere(np.isnan(got) != nan)[:5])
    err = np.abs(got - exact)
    fin = ~nan
    bad = np.argwhere(fin & ~(err <= tol))
    assert bad.size == 0, [(int(m), int(n), got[m, n], exact[m, n], tol[m, n]) for m, n in bad[:5]]
    ratio = float(np.max(np.where(fin & (acc_tol > 0), err / np.maximum(tol, 1e-300), 0)))
    print("gemm %s: max |err| / bound = %.3f" % (str(A.shape + B.shape), ratio))
    return got, exact


def grouped_model(a_vals, b_vals):
    """The matrix core's sum of one dot product as measured: each aligned group of 8
    products is summed after truncating every product toward zero to the grid
    2^(e - 13), 2^e <= the group's largest |product| < 2^(e+1); group sums add up
    exactly here (the crafted cases keep every binary32 addition exact)."""
    total = 0.0
    for q in range(0, len(a_vals), 8):
        p = [float(x) * float(y) for x, y in zip(a_vals[q:q + 8], b_vals[q:q + 8])]
        mx = max(abs(v) for v in p)
        if mx == 0:
            continue
        grid = 2.0 ** (math.floor(math.log2(mx)) - 13)
        total += sum(math.trunc(v / grid) * grid for v in p)
    return total


def test_gemm_accumulation_model():
    """Crafted single dot products (M = N = 1, K = 64 or 128) whose results pin the
    accumulation model the tolerance rests on: a product 2^-13 below the group's
    largest is kept, 2^-14 below is dropped (either sign), groups are k in [8q, 8q+8)
    (a small product one slot later, in the next group, is kept), the largest need not
    come first, the 64 slots split into 8 groups, and separate steps accumulate in
    binary32."""
    import delayed_scaling_amax_amd as d
    cases = []
    for e in range(2, 10):
        for sg in (1.0, -1.0):
            cases.append({0: (256.0, 1.0), 1: (sg * 2.0 ** -e, 1.0)})
    for j in range(1, 12):
        cases.append({0: (256.0, 1.0), j: (2.0 ** -6, 1.0)})
    cases += [{7: (256.0, 1.0), 0: (2.0 ** -6, 1.0)}, {32: (256.0, 1.0), 33: (2.0 ** -6, 1.0)},
              {32: (256.0, 1.0), 40: (2.0 ** -6, 1.0)}, {0: (448.0, 448.0), 1: (1.0, 3.0), 2: (0.5, 0.75)},
              {0: (256.0, 1.0), 1: (-256.0, 1.0), 2: (2.0 ** -6, 1.0)},
              {0: (256.0, 1.0), **{j: (2.0 ** -5, 1.0) for j in range(1, 8)}},
              {0: (256.0, 1.0), 64: (2.0 ** -9, 1.0)}]
    for c in cases:
        K = 128 if max(c) >= 64 else 64
        a = [0.0] * K
        b = [0.0] * K
        for j, (x, y) in c.items():
            a[j], b[j] = x, y
        A = torch.tensor(a).to(torch.float8_e4m3fn).view(torch.uint8).view(1, K)
        B = torch.tensor(b).to(torch.float8_e4m3fn).view(torch.uint8).view(1, K)
        av = A.view(torch.float8_e4m3fn).double().view(-1).tolist()
        bv = B.view(torch.float8_e4m3fn).double().view(-1).tolist()
        C = torch.zeros(1, 1, device="cuda")
        note("gemm accumulation model case %r" % sorted(c))
        d.fp8_gemm(A.cuda(), E4M3, B.cuda(), E4M3, f32([1.0]), f32([1.0]), C)
        torch.cuda.synchronize()
        assert C.item() == grouped_model(av, bv), (sorted(c.items()), C.item(), grouped_model(av, bv))


@pytest.mark.parametrize("fa,fb", [(E4M3, E4M3), (E4M3, E5M2), (E5M2, E4M3), (E5M2, E5M2)])
def test_gemm_formats_small(orc, fa, fb):
    g = np.random.Generator(np.random.PCG64(900 + 2 * fa + fb))
    for M, N, K in ((1, 1, 16), (32, 32, 64), (33, 31, 80), (256, 256, 128)):
        A = random_codes(g, (M, K), fa)
        B = random_codes(g, (N, K), fb)
        note("gemm fmt %d/%d M=%d N=%d K=%d" % (fa, fb, M, N, K))
        check(orc, A, fa, B, fb, 0.37, 2.5e-3, torch.float32)
        check(orc, A, fa, B, fb, 0.37, 2.5e-3, torch.bfloat16)


@pytest.mark.parametrize("M,N,K", [(300, 200, 144), (257, 513, 1040), (512, 256, 4096),
                                   (1000, 300, 16), (64, 700, 2048)])
def test_gemm_ragged_shapes(orc, M, N, K):
    """Ragged M and N (partial block tiles), K a multiple of 16 but not of 64 (the last
    step's chunks past K load as zeros), long K."""
    g = np.random.Generator(np.random.PCG64(M * 7 + N * 3 + K))
    A = random_codes(g, (M, K), E4M3, spread=False)
    B = random_codes(g, (N, K), E4M3, spread=False)
    note("gemm ragged M=%d N=%d K=%d" % (M, N, K))
    check(orc, A, E4M3, B, E4M3, 0.05, 0.02, torch.bfloat16, threads=8)


def test_gemm_k_zero_and_scales(orc):
    import delayed_scaling_amax_amd as d
    g = np.random.Generator(np.random.PCG64(950))
    A = random_codes(g, (70, 64), E4M3)
    B = random_codes(g, (40, 64), E5M2)
    for sa, sb in ((0.0, 1.0), (-2.0, 0.5), (1e-20, 1e-18), (3e4, 2e3)):
        note("gemm scales %r %r" % (sa, sb))
        check(orc, A, E4M3, B, E5M2, sa, sb, torch.float32)
    # K = 0: an empty sum
    C = torch.full((5, 7), float("nan"), dtype=torch.float32, device="cuda")
    d.fp8_gemm(torch.zeros(5, 0, dtype=torch.uint8, device="cuda"), E4M3,
               torch.zeros(7, 0, dtype=torch.uint8, device="cuda"), E4M3, f32([1.0]),
               f32([1.0]), C)
    torch.cuda.synchronize()
    assert (C == 0).all()


def test_gemm_nan_propagates(orc):
    g = np.random.Generator(np.random.PCG64(960))
    A = random_codes(g, (64, 128), E4M3)
    B = random_codes(g, (64, 128), E4M3)
    A[3, 17] = 0x7F
    B[9, 100] = 0xFF
    note("gemm NaN operands")
    got, exact = check(orc, A, E4M3, B, E4M3, 1.0, 1.0, torch.float32)
    assert np.isnan(got[3]).all() and np.isnan(got[:, 9]).all()


def test_gemm_mlp_wi_sampled(orc):
    """The MLP's first dense at full size: activation (8192 x 4096) E4M3 times the wi
    weight (16384 x 4096 after transposition) E4M3, bf16 out, checked on 96 sampled rows
    x 96 sampled columns (the oracle's exact sums over K = 4096) plus every row and
    column of the last, partial-free tile corner."""
    g = np.random.Generator(np.random.PCG64(970))
    M, N, K = 8192, 16384, 4096
    A = random_codes(g, (M, K), E4M3, spread=False)
    B = random_codes(g, (N, K), E4M3, spread=False)
    note("gemm mlp wi full size")
    got = run_gemm(A, E4M3, B, E4M3, 0.011, 0.0023, torch.bfloat16)
    rows = np.unique(np.concatenate([g.integers(0, M, 90), [0, 255, 256, M - 1, M - 256]]))
    cols = np.unique(np.concatenate([g.integers(0, N, 90), [0, 255, 256, N - 1, N - 256]]))
    exact, cabs, cg = orc.fp8_gemm(A[rows], E4M3, B[cols], E4M3, 0.011, 0.0023, threads=8)
    sub = got[np.ix_(rows, cols)]
    acc_tol = acc_bound(K, cabs, cg)
    tol = acc_tol + 2.0 ** -8 * (np.abs(exact) + acc_tol)
    assert (np.abs(sub - exact) <= tol).all(), float(np.max(np.abs(sub - exact) / tol))
    print("gemm wi sampled: max |err| / bound = %.3f" % float(np.max(np.abs(sub - exact) / tol)))


@pytest.mark.parametrize("M,N,K", [(4200, 4096, 64), (6000, 2600, 32)])
def test_gemm_tile_order_full(orc, M, N, K):
    """Every output of grids with more than 256 tiles (so persistent blocks take a second
    tile and prefetch it during the first one's epilogue) and a ragged last row of 4 x 8
    super-tiles: 17 x 16 tiles (column count a multiple of 8: strided super-tile columns)
    and 24 x 11 tiles (contiguous super-tile columns, a narrower last group)."""
    g = np.random.Generator(np.random.PCG64(M + N + K))
    A = random_codes(g, (M, K), E4M3, spread=False)
    B = random_codes(g, (N, K), E4M3, spread=False)
    note("gemm tile order M=%d N=%d K=%d" % (M, N, K))
    check(orc, A, E4M3, B, E4M3, 0.05, 0.02, torch.bfloat16, threads=16)


def test_gemm_inf_operands(orc):
    """E5M2 +-inf codes (M3): inf times a finite nonzero value gives a signed inf, inf
    times zero and inf - inf give NaN, rows and columns without an inf are unaffected."""
    g = np.random.Generator(np.random.PCG64(990))
    M, N, K = 64, 48, 128
    A = random_codes(g, (M, K), E5M2, spread=False)
    B = random_codes(g, (N, K), E5M2, spread=False)
    A[A == 0] = 0x3C  # no accidental zeros: placed zeros below decide inf * 0
    B[B == 0] = 0x3C
    A[2, 5] = 0x7C                      # +inf against column 5 of every B row
    A[7, 40] = 0xFC                     # -inf
    A[11, 3] = 0x7C
    A[11, 90] = 0xFC                    # +inf and -inf in one row: NaN where the products differ in sign
    A[20, 64] = 0x7C
    B[4, 64] = 0x00                     # inf * 0 -> NaN at C[20, 4]
    B[9, 70] = 0x7C                     # column 9 of C: +inf against row 30's entry
    A[30, 70] = 0x80                    # -0 * inf -> NaN at C[30, 9]
    note("gemm inf operands")
    got = run_gemm(A, E5M2, B, E5M2, 0.5, 0.25, torch.float32)
    exact, cabs, cg = orc.fp8_gemm(A, E5M2, B, E5M2, 0.5, 0.25)
    nan = np.isnan(exact)
    inf = np.isinf(exact)
    assert nan.sum() > 0 and inf.sum() > 0
    assert (np.isnan(got) == nan).all(), np.argwhere(np.isnan(got) != nan)[:8]
    assert (got[inf] == exact[inf]).all(), np.argwhere(inf & (got != exact))[:8]
    fin = ~(nan | inf)
    tol = acc_bound(K, cabs, cg) + 2.0 ** -23 * np.abs(exact) + 2.0 ** -149
    assert (np.abs(got[fin] - exact[fin]) <= tol[fin]).all()
