"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError when it
disagrees with:
  * values worked by hand from the format definitions (tests/golden/*.txt, cited there);
  * torch's CPU float8_e4m3fn / float8_e5m2 decode and cast, and its bfloat16 cast
    (an independent library; the oracle does not use torch);
  * exact rational arithmetic (``fractions.Fraction``) with round-half-even done here,
    independent of the host's IEEE hardware;
  * brute-force nearest-code search over the decoded code table;
  * invariants (monotonicity, power-of-two margin, roll bookkeeping, error bound).

test_oracle_pins.py runs them on the real oracle; test_oracle_mutants.py runs them on
oracle copies with planted mistakes and requires each mistake to fail at least one pin.
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np
import torch

E4M3, E5M2 = 0, 1
BF16, F32 = 0, 1
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
TORCH_FP8 = {E4M3: torch.float8_e4m3fn, E5M2: torch.float8_e5m2}
FMT_NAME = {"e4m3": E4M3, "e5m2": E5M2}


# ------------------------------------------------------------------ helpers
def u2f(u: int) -> float:
    return float(np.uint32(u).view(np.float32))


def f2u(f) -> int:
    return int(np.float32(f).view(np.uint32))


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def rn_binary(fr: Fraction, mant_bits: int, emin: int, emax_bound: int) -> Fraction | None:
    """Exact round-to-nearest-even of a non-negative rational to a binary format with
    `mant_bits` fraction bits and minimum normal exponent `emin`; None on overflow
    (result >= 2^emax_bound)."""
    if fr == 0:
        return Fraction(0)
    p, q = fr.numerator, fr.denominator
    e = p.bit_length() - q.bit_length()
    if Fraction(2) ** e > fr:
        e -= 1
    e = max(e, emin)
    quantum = Fraction(2) ** (e - mant_bits)
    r = round(fr / quantum) * quantum          # Fraction.__round__ is half-to-even
    if r >= Fraction(2) ** emax_bound:
        return None
    return r


def rn32(fr: Fraction) -> float:
    """Exact RN-even of a rational to binary32 (sign handled, overflow -> inf)."""
    sgn = -1.0 if fr < 0 else 1.0
    r = rn_binary(abs(fr), 23, -126, 128)
    return sgn * (float("inf") if r is None else float(r))


def code_table(fmt: int) -> np.ndarray:
    """Decoded values of all 256 codes from torch (independent library)."""
    return torch.arange(256, dtype=torch.uint8).view(TORCH_FP8[fmt]).float().numpy()


def brute_encode(fmt: int, v: np.ndarray) -> np.ndarray:
    """Nearest finite code by exhaustive search over the code table; ties go to the
    code with an even mantissa (LSB 0); zero keeps its sign.  |v| <= max assumed."""
    tab = code_table(fmt).astype(np.float64)
    pos = [c for c in range(128) if np.isfinite(tab[c])]
    vals = tab[pos]
    codes = np.array(pos)
    v = np.asarray(v, np.float64)
    a = np.abs(v)
    d = np.abs(vals[None, :] - a[:, None])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # among candidates prefer even LSB
    even = (codes[None, :] & 1) == 0
    pick = np.where((cand & even).any(axis=1), np.argmax(cand & even, axis=1),
                    np.argmax(cand, axis=1))
    out = codes[pick].astype(np.uint8)
    out |= (np.signbit(v).astype(np.uint8) << 7)
    return out


def read_golden(name: str):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line)
    return rows


def golden_kv(name: str) -> dict:
    kv = {}
    for r in read_golden(name):
        if ":" in r:
            k, v = r.split(":", 1)
            kv[k.strip()] = v.split()
    return kv


# ------------------------------------------------------------------ pins: formats
def pin_format_constants(o):
    for row in read_golden("fp8_formats.txt"):
        f = row.split()
        if f[0] not in FMT_NAME:
            continue
        fmt = FMT_NAME[f[0]]
        mx = float(f[1])
        mn = 2.0 ** int(f[2].split("^")[1])
        ms = 2.0 ** int(f[3].split("^")[1])
        assert o.fp8_max(fmt) == mx
        assert o.decode(fmt, int(f[4], 16)) == mx
        assert o.decode(fmt, int(f[5], 16)) == mn
        assert o.decode(fmt, int(f[6], 16)) == ms
        vals = np.array([o.decode(fmt, c) for c in range(256)])
        assert np.isfinite(vals).sum() == int(f[7])
        assert np.isnan(vals).sum() == int(f[8])
        assert np.isinf(vals).sum() == int(f[9])
        assert torch.finfo(TORCH_FP8[fmt]).max == mx


def pin_decode_matches_torch(o):
    for fmt in (E4M3, E5M2):
        ref = code_table(fmt)
        got = np.array([o.decode(fmt, c) for c in range(256)], np.float32)
        same = (got.view(np.uint32) == ref.view(np.uint32)) | (np.isnan(got) & np.isnan(ref))
        assert same.all(), np.nonzero(~same)[0][:8]


def pin_decode_monotone(o):
    for fmt in (E4M3, E5M2):
        pos = np.array([o.decode(fmt, c) for c in range(128)])
        fin = pos[np.isfinite(pos)]
        assert (np.diff(fin) > 0).all()
        neg = np.array([o.decode(fmt, c | 0x80) for c in range(128)])
        assert (np.signbit(neg)).all()


def pin_encode_roundtrip(o):
    for fmt in (E4M3, E5M2):
        for c in range(256):
            v = o.decode(fmt, c)
            if np.isfinite(v):
                assert o.encode(fmt, v) == c, (fmt, hex(c))


def pin_encode_bruteforce_all_bf16(o):
    """Every finite bf16 value, clamped to +-max, vs exhaustive nearest search and
    vs torch's CPU cast (which agrees once the value is in range)."""
    allb = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    x = bf16_to_f32(allb)
    x = x[np.isfinite(x)]
    for fmt in (E4M3, E5M2):
        mx = np.float32(o.fp8_max(fmt))
        v = np.clip(x, -mx, mx)
        got = np.array([o.encode(fmt, float(t)) for t in v], np.uint8)
        tor = torch.from_numpy(v.copy()).to(TORCH_FP8[fmt]).view(torch.uint8).numpy()
        assert (got == tor).all(), np.nonzero(got != tor)[0][:8]
        # brute force on a strided subset (the full set is covered by torch above)
        sub = v[::7]
        assert (brute_encode(fmt, sub) == got[::7]).all()


def pin_encode_random_f32(o):
    g = np.random.Generator(np.random.PCG64(7))
    for fmt in (E4M3, E5M2):
        mx = o.fp8_max(fmt)
        v = (np.exp2(g.uniform(-20, np.log2(mx), 4000)) *
             np.where(g.random(4000) < 0.5, -1, 1)).astype(np.float32)
        got = np.array([o.encode(fmt, float(t)) for t in v], np.uint8)
        assert (got == brute_encode(fmt, v)).all()


def pin_encode_worked_ties(o):
    """Ties and underflow by hand: E4M3 2^-10 is half the smallest subnormal (tie ->
    0x00), 1.5*2^-10 -> 0x01 (2^-9 nearer), -1e-9 -> 0x80 (signed zero); E5M2
    480 = midpoint of 448 (0x5f) and 512 (0x60) -> 0x60 (even), 2^-17 -> 0x00 (tie),
    3*2^-18 -> 0x01."""
    assert o.encode(E4M3, 2.0 ** -10) == 0x00
    assert o.encode(E4M3, 1.5 * 2.0 ** -10) == 0x01
    assert o.encode(E4M3, -1e-9) == 0x80
    assert o.encode(E4M3, 440.0) == 0x7E            # between 416 and 448, nearer 448
    assert o.encode(E4M3, 432.0) == 0x7E            # midpoint 416|448 -> even 448 (0x7e)
    assert o.encode(E4M3, 400.0) == 0x7C            # midpoint 384|416 -> even 384 (0x7c)
    assert o.encode(E5M2, 448.0) == 0x5F
    assert o.encode(E5M2, 480.0) == 0x60
    assert o.encode(E5M2, 2.0 ** -17) == 0x00
    assert o.encode(E5M2, 3 * 2.0 ** -18) == 0x01
    assert o.encode(E5M2, -1e-9) == 0x80


# ------------------------------------------------------------------ pins: quantize
def pin_quantize_worked_tensor(o):
    kv = golden_kv("quantize_worked.txt")
    x = np.array([int(h, 16) for h in kv["x_bf16"]], np.uint16)
    for key, fmt in (("e4m3_scale_3f800000", E4M3), ("e5m2_scale_3f800000", E5M2),
                     ("e4m3_scale_400edb6e", E4M3)):
        scale = u2f(int(key.rsplit("_", 1)[1], 16))
        want = bytes(int(h, 16) for h in kv[key])
        codes, amax = o.quantize_amax(x, fmt, scale)
        assert codes.tobytes() == want, (key, codes.tobytes().hex())
        assert f2u(amax) == int(kv["amax"][0], 16)


def _exact_quantize(o, fmt, x: float, s: float) -> int:
    """RN32 of the exact quotient (rational), saturation, brute-force encode."""
    if np.isnan(x):
        return 0x7F | (0x80 if np.signbit(x) else 0)
    q = rn32(Fraction(x) / Fraction(s))
    mx = o.fp8_max(fmt)
    q = min(max(q, -mx), mx)
    if q == 0.0:
        return 0x80 if (np.signbit(x) != np.signbit(s)) else 0x00
    return int(brute_encode(fmt, np.array([q]))[0])


def pin_quantize_exact_quotient(o):
    """Random (x, s) and near-midpoint quotients: the oracle's element result equals
    exact-rational RN32(x/s) -> clamp -> nearest code.  Near-midpoint pairs make the
    double rounding (binary32, then FP8) decide the byte."""
    g = np.random.Generator(np.random.PCG64(11))
    cases = []
    for _ in range(1500):
        s = float(np.float32(np.exp2(g.uniform(-30, 30))))
        x = float(bf16_to_f32(np.array([g.integers(0, 1 << 16)], np.uint16))[0])
        if np.isfinite(x):
            cases.append((x, s))
    for fmt in (E4M3, E5M2):
        tab = code_table(fmt)
        fin = np.sort(tab[np.isfinite(tab) & (tab >= 0)])
        mids = (fin[1:] + fin[:-1]) / 2
        for _ in range(600):
            m = float(mids[g.integers(0, len(mids))])
            s = float(np.float32(np.exp2(g.uniform(-20, 20))))
            x = np.float32(m * s)
            for k in (-2, -1, 0, 1, 2):
                xx = float(np.nextafter(x, np.float32(np.inf) if k > 0 else np.float32(0)))
                xx = float(x) if k == 0 else xx
                cases.append((xx, s))
    for fmt in (E4M3, E5M2):
        for x, s in cases:
            want = _exact_quantize(o, fmt, x, s)
            got = o.quantize_element(fmt, x, s)
            assert got == want, (fmt, x, s, hex(got), hex(want))


def pin_quantize_extreme_scales(o):
    """R12: a scale outside the normal range, negative, zero, infinite or NaN still gives
    the IEEE quotient x / scale, then R2-R4.  Finite nonzero scales (subnormal, the
    largest finite, negative) against the exact rational RN32 of x / s (overflow to inf,
    underflow to a zero signed by sign(x) xor sign(s)); zero, infinite and NaN scales
    against IEEE's special cases written out: x/0 = inf (0/0 NaN), x/inf = 0 (inf/inf
    NaN), NaN anything = NaN; a NaN quotient encodes as 0x7F with x's sign (R4)."""
    xb = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x0080, 0x3E80, 0x3F80, 0xBF80,
                   0x43E0, 0xC2F6, 0x4780, 0x7F7F, 0xFF7F, 0x7F80, 0xFF80, 0x7FC0, 0xFFC0],
                  np.uint16)
    xs = [float(v) for v in bf16_to_f32(xb)]
    f32 = lambda v: float(np.float32(v))
    finite = [f32(2.0 ** -149), f32(3 * 2.0 ** -149), f32(2.0 ** -130), f32(2.0 ** -126),
              f32(1e-30), 1.5, -1.5, f32(-(2.0 ** -140)), f32(1e20), f32(-3e30),
              f32(1.5 * 2.0 ** 127), f32(3.4028234663852886e38), f32(-3.4028234663852886e38)]
    special = [0.0, -0.0, float("inf"), float("-inf"), float("nan")]
    for fmt in (E4M3, E5M2):
        mx = o.fp8_max(fmt)
        for x in xs:
            sx = bool(np.signbit(x))
            for sc in finite + special:
                ss = bool(np.signbit(sc))
                if np.isnan(x) or np.isnan(sc):
                    q = float("nan")
                elif sc == 0.0:
                    q = float("nan") if x == 0.0 else (-1.0 if sx != ss else 1.0) * float("inf")
                elif np.isinf(sc):
                    q = float("nan") if np.isinf(x) else (-0.0 if sx != ss else 0.0)
                elif np.isinf(x):
                    q = (-1.0 if sx != ss else 1.0) * float("inf")
                else:
                    q = None                               # finite / finite: exact rational
                if q is None:
                    want = _exact_quantize(o, fmt, x, sc)
                elif np.isnan(q):
                    want = 0x7F | (0x80 if sx else 0x00)
                elif q == 0.0:
                    want = 0x80 if np.signbit(q) else 0x00
                else:
                    want = int(brute_encode(fmt, np.array([max(min(q, mx), -mx)]))[0])
                got = o.quantize_element(fmt, x, sc)
                assert got == want, (fmt, x, sc, hex(got), hex(want))


def pin_quantize_f32_matches_encode_at_scale_one(o):
    g = np.random.Generator(np.random.PCG64(3))
    v = (np.exp2(g.uniform(-30, 20, 3000)) * np.where(g.random(3000) < .5, -1, 1)).astype(
        np.float32)
    for fmt in (E4M3, E5M2):
        codes, _ = o.quantize_amax(v, fmt, 1.0)
        mx = np.float32(o.fp8_max(fmt))
        want = torch.from_numpy(np.clip(v, -mx, mx)).to(TORCH_FP8[fmt]).view(
            torch.uint8).numpy()
        assert (codes == want).all()


def pin_quantize_specials(o):
    # +-inf saturate, NaN -> 0x7f with the sign of x, huge quotients saturate.
    for fmt in (E4M3, E5M2):
        mxc = 0x7E if fmt == E4M3 else 0x7B
        assert o.quantize_element(fmt, float("inf"), 1.0) == mxc
        assert o.quantize_element(fmt, float("-inf"), 1.0) == mxc | 0x80
        assert o.quantize_element(fmt, float("nan"), 1.0) == 0x7F
        assert o.quantize_element(fmt, -float("nan"), 1.0) == 0xFF
        assert o.quantize_element(fmt, 1e30, 1e-6) == mxc
        assert o.quantize_element(fmt, -0.0, 3.0) == 0x80


def pin_quantize_monotone(o):
    allb = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    x = bf16_to_f32(allb)
    x = np.sort(x[np.isfinite(x)])
    for fmt, s in ((E4M3, 0.37), (E5M2, 1e-5)):
        codes, _ = o.quantize_amax(x, fmt, s)
        dec = code_table(fmt)[codes]
        assert (np.diff(dec) >= 0).all()


def pin_amax(o):
    g = np.random.Generator(np.random.PCG64(5))
    x = (g.standard_normal(10001) * 3).astype(np.float32)
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)        # bf16 by truncation
    _, a = o.quantize_amax(xb, E4M3, 1.0)
    assert a == np.abs(bf16_to_f32(xb)).max()
    _, a = o.quantize_amax(x, E5M2, 2.0)
    assert a == np.abs(x).max()
    # max-accumulation: a larger incoming amax survives, a smaller one is replaced
    _, a = o.quantize_amax(x, E4M3, 1.0, amax_in=1e6)
    assert a == np.float32(1e6)
    _, a = o.quantize_amax(x, E4M3, 1.0, amax_in=1e-6)
    assert a == np.abs(x).max()
    # negative values count by magnitude
    _, a = o.quantize_amax(np.array([-5.0, 2.0], np.float32), E4M3, 1.0)
    assert a == 5.0
    # NaN propagates (largest bit pattern)
    y = x.copy()
    y[17] = np.nan
    _, a = o.quantize_amax(y, E4M3, 1.0)
    assert np.isnan(a)
    # the NaN payload (R5: the largest sign-cleared bit pattern): among NaNs of both signs
    # the largest payload wins, and any NaN beats inf; bf16 sources count by their
    # binary32 upcast
    zb = np.concatenate([np.array([1.0, -np.inf, 3.0, 0.0], np.float32).view(np.uint32),
                         np.array([0xFFE12345, 0x7FC00001, 0xFFC00100], np.uint32)])
    _, a = o.quantize_amax(zb.view(np.float32), E4M3, 1.0)
    assert np.float32(a).view(np.uint32) == (zb & 0x7FFFFFFF).max() == 0x7FE12345
    hb = np.array([0x3F80, 0xFFE1, 0x7FC3, 0xFF80], np.uint16)  # 1, -NaN, +NaN, -inf
    _, a = o.quantize_amax(hb, E5M2, 1.0)
    assert np.float32(a).view(np.uint32) == 0x7FE10000
    # signaling NaNs count by their own bits, never quieted: a quieted 0x7F81F558 would
    # read 0x7FC1F558 and beat the quiet 0x7FC1EA99 that is the true bit maximum; the
    # incoming amax keeps its bits the same way
    sn = np.array([0x3F800000, 0xFF81F558, 0x7FC1EA99], np.uint32)
    _, a = o.quantize_amax(sn.view(np.float32), E4M3, 1.0, threads=1)
    assert np.float32(a).view(np.uint32) == 0x7FC1EA99
    _, a = o.quantize_amax(sn[:2].view(np.float32), E4M3, 1.0)
    assert np.float32(a).view(np.uint32) == 0x7F81F558
    _, a = o.quantize_amax(sn[:1].view(np.float32), E4M3, 1.0,
                           amax_in=np.uint32(0x7F80ABCD).view(np.float32))
    assert np.float32(a).view(np.uint32) == 0x7F80ABCD
    _, a = o.quantize_amax(np.array([0x3F80, 0xFF81, 0x7F80], np.uint16), E5M2, 1.0)
    assert np.float32(a).view(np.uint32) == 0x7F810000


def pin_saturation_count(o):
    x = np.array([447.0, 448.0, 463.9, 464.0, 470.0, -500.0, 1e9, np.inf], np.float32)
    assert o.count_saturated(x, E4M3, 1.0) == 6
    assert o.count_saturated(x, E5M2, 1.0) == 2


def pin_dequant_error_bound(o):
    """|dq(q(x)) - x| <= half an FP8 ulp of x/s, times s (plus binary32 rounding)."""
    g = np.random.Generator(np.random.PCG64(9))
    for fmt, s in ((E4M3, 0.013), (E5M2, 3.1e-4)):
        mx = o.fp8_max(fmt)
        xs = (g.uniform(-mx, mx, 3000) * s).astype(np.float32)
        codes, _ = o.quantize_amax(xs, fmt, s)
        y = o.dequantize(codes, fmt, s)
        tab = code_table(fmt)
        fin = np.sort(np.unique(np.abs(tab[np.isfinite(tab)])))
        q = np.abs(xs.astype(np.float64) / s)
        i = np.clip(np.searchsorted(fin, q), 1, len(fin) - 1)
        gap = fin[i] - fin[i - 1]
        err = np.abs(y.astype(np.float64) - xs)
        assert (err <= 0.5 * gap * s * (1 + 2e-6) + np.abs(xs) * 2e-7).all()


# ------------------------------------------------------------------ pins: scale update
def pin_scale_update_worked(o):
    for row in read_golden("scale_update_worked.txt"):
        f = row.split()
        if f[0].startswith("h4") or len(f) != 5:
            continue
        amax = u2f(int(f[0], 16))
        fmt = FMT_NAME[f[1]]
        r = o.amax_and_scale_update(np.array([amax], np.float32),
                                    np.zeros((4, 1), np.float32),
                                    np.ones(1, np.float32), np.array([fmt], np.uint8),
                                    margin=int(f[2]))
        assert f2u(r["scale"][0]) == int(f[3], 16), row
        assert f2u(r["scale_inv"][0]) == int(f[4], 16), row


def pin_history_worked(o):
    hist = np.zeros((4, 1), np.float32)
    scale = np.ones(1, np.float32)
    for row in read_golden("scale_update_worked.txt"):
        f = row.split()
        if f[0] != "h4":
            continue
        a = np.array([float(f[1])], np.float32)
        r = o.amax_and_scale_update(a, hist, scale, np.zeros(1, np.uint8))
        hist, scale = r["hist"], r["scale"]
        assert list(hist[:, 0]) == [float(v) for v in f[2:6]], row
        sel = float(f[6])
        assert f2u(scale[0]) == f2u(np.float32(rn32(Fraction(sel) / 448))), row
    want = int(golden_kv("scale_update_worked.txt")["h4_last_scale"][0], 16)
    assert f2u(scale[0]) == want


def pin_scale_update_exact(o):
    """Scale and scale_inv equal exact-rational RN32 of sel/MAX * 2^margin and of
    1/scale, for random amaxes across the binary32 range, both formats, margins."""
    g = np.random.Generator(np.random.PCG64(21))
    n = 400
    amax = np.exp2(g.uniform(-60, 60, n)).astype(np.float32)
    fmts = (g.random(n) < 0.5).astype(np.uint8)
    for margin in (0, 1, 3, -2):
        r = o.amax_and_scale_update(amax, np.zeros((1, n), np.float32),
                                    np.ones(n, np.float32), fmts, margin=margin)
        for t in range(n):
            mx = 448 if fmts[t] == 0 else 57344
            c = rn32(Fraction(float(amax[t])) / mx)
            c = rn32(Fraction(c) * Fraction(2) ** margin)
            assert f2u(r["scale"][t]) == f2u(np.float32(c)), (t, margin)
            inv = rn32(1 / Fraction(c))
            assert f2u(r["scale_inv"][t]) == f2u(np.float32(inv)), (t, margin)


def pin_scale_update_invariants(o):
    g = np.random.Generator(np.random.PCG64(23))
    H, n = 6, 50
    hist = np.exp2(g.uniform(-10, 10, (H, n))).astype(np.float32)
    amax = np.exp2(g.uniform(-10, 10, n)).astype(np.float32)
    scale = np.exp2(g.uniform(-3, 3, n)).astype(np.float32)
    fmts = np.tile(np.array([0, 0, 1], np.uint8), n)[:n]
    r0 = o.amax_and_scale_update(amax, hist, scale, fmts, margin=0)
    r1 = o.amax_and_scale_update(amax, hist, scale, fmts, margin=1)
    # roll: row 0 = new amax, row h = old row h-1, old last row dropped
    assert (r0["hist"][0] == amax).all()
    assert (r0["hist"][1:] == hist[:-1]).all()
    # margin 1 doubles the scale exactly
    assert (r1["scale"] == 2 * r0["scale"]).all()
    # algo max selects the max of the rolled window
    sel = np.maximum(amax, hist[:-1].max(axis=0))
    mx = np.where(fmts == 0, np.float32(448), np.float32(57344))
    assert (r0["scale"] == (sel / mx).astype(np.float32)).all()
    # most recent: selection is the new amax
    rm = o.amax_and_scale_update(amax, hist, scale, fmts, algo=1)
    assert (rm["scale"] == (amax / mx).astype(np.float32)).all()
    assert (rm["hist"] == r0["hist"]).all()
    # amax output: untouched without reset, zero with reset
    assert (r0["amax"] == amax).all()
    rr = o.amax_and_scale_update(amax, hist, scale, fmts, reset_amax=True)
    assert (rr["amax"] == 0).all() and (rr["scale"] == r0["scale"]).all()
    # k <= H steps from zero history: rows 0..k-1 hold the last k amaxes, newest first
    h = np.zeros((H, 2), np.float32)
    seq = [np.array([i + 1.0, 10.0 * (i + 1)], np.float32) for i in range(4)]
    for a in seq:
        h = o.amax_and_scale_update(a, h, np.ones(2, np.float32), np.zeros(2, np.uint8))["hist"]
    assert (h[:4] == np.array(seq[::-1])).all() and (h[4:] == 0).all()


def pin_scale_update_keep_previous(o):
    prev = np.array([0.5, 0.25, 2.0, 4.0, 8.0], np.float32)
    amax = np.array([0.0, np.inf, np.nan, 1e-45, 3.0e38], np.float32)
    # zero history: sel = amax itself
    r = o.amax_and_scale_update(amax, np.zeros((1, 5), np.float32), prev,
                                np.zeros(5, np.uint8), margin=0)
    # 0 -> keep; inf -> keep; NaN -> keep; 1e-45/448 underflows to 0 -> keep;
    assert list(r["scale"][:4]) == list(prev[:4])
    assert r["scale"][4] == np.float32(np.float32(3.0e38) / np.float32(448))
    r = o.amax_and_scale_update(amax, np.zeros((1, 5), np.float32), prev,
                                np.zeros(5, np.uint8), margin=120)
    # 3e38/448 * 2^120 overflows -> keep
    assert r["scale"][4] == prev[4]
    assert (r["scale_inv"] == (np.float32(1) / r["scale"]).astype(np.float32)).all()


# ------------------------------------------------------------------ pins: dequantize
def pin_dequantize_matches_torch(o):
    codes = np.arange(256, dtype=np.uint8)
    for fmt in (E4M3, E5M2):
        dec = torch.from_numpy(codes).view(TORCH_FP8[fmt]).float()
        for s in (1.0, 0.0123, 3.7e4, 2.0 ** -20):
            y = o.dequantize(codes, fmt, s)
            want = (dec * torch.tensor(s, dtype=torch.float32)).numpy()
            fin = ~np.isnan(want)
            assert (y[fin].view(np.uint32) == want[fin].view(np.uint32)).all()
            nanb = 0x7FC00000 | ((codes[~fin].astype(np.uint32) & 0x80) << 24)
            assert (y[~fin].view(np.uint32) == nanb).all()
            yb = o.dequantize(codes, fmt, s, out_dtype=BF16)
            wb = torch.from_numpy(want).to(torch.bfloat16).view(torch.int16).numpy().view(
                np.uint16)
            assert (yb[fin] == wb[fin]).all()
            assert (yb[~fin] == (nanb >> 16).astype(np.uint16)).all()


def pin_bf16_rounding_random(o):
    """bf16 output rounding vs torch's RNE cast on values with random low bits, incl.
    overflow to inf and bf16-subnormal results."""
    g = np.random.Generator(np.random.PCG64(29))
    codes = g.integers(0, 256, 5000).astype(np.uint8)
    for fmt in (E4M3, E5M2):
        dec = torch.from_numpy(codes).view(TORCH_FP8[fmt]).float()
        for s in (float(np.float32(1.2345678)), 3.0e36, 1.7e-41):
            want = (dec * torch.tensor(s, dtype=torch.float32))
            yb = o.dequantize(codes, fmt, s, out_dtype=BF16)
            fin = ~torch.isnan(want).numpy()
            wb = want.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
            assert (yb[fin] == wb[fin]).all()




def pin_microbatch_accumulation(o):
    """Max-accumulating amax over microbatches ("Gradient accumulation of FP8 params":
    FP8 meta combines with max) equals the amax of the concatenated tensor, and the
    codes of each microbatch do not depend on the accumulated amax."""
    g = np.random.Generator(np.random.PCG64(31))
    parts = [(g.standard_normal(n) * 10.0 ** g.uniform(-2, 2)).astype(np.float32)
             for n in (1000, 1, 777, 4096)]
    a = 0.0
    for p in parts:
        codes, a = o.quantize_amax(p, E4M3, 0.25, amax_in=a)
        alone, _ = o.quantize_amax(p, E4M3, 0.25)
        assert (codes == alone).all()
    _, whole = o.quantize_amax(np.concatenate(parts), E4M3, 0.25)
    assert f2u(a) == f2u(whole)




# ------------------------------------------------------------------ pins: fused gelu
def _bf16_grid_sample():
    allb = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    x = bf16_to_f32(allb)
    return allb[np.isfinite(x) & (np.abs(x) < 30)], allb


def gelu_decimal(x: float) -> float:
    """tanh-GELU in its tanh form at 150 significant digits with Python's decimal module
    (exp correctly rounded at the context precision; no libm; 150 digits absorb the
    cancellation of 1 + tanh(u) for every x >= -14)."""
    import decimal
    with decimal.localcontext() as ctx:
        ctx.prec = 150
        X = decimal.Decimal(x)
        pi = decimal.Decimal("3.14159265358979323846264338327950288419716939937510")
        c = (2 / pi).sqrt()
        u = c * (X + decimal.Decimal("0.044715") * X * X * X)
        e2u = (2 * u).exp()
        t = (e2u - 1) / (e2u + 1)
        return float(decimal.Decimal("0.5") * X * (1 + t))


def pin_gelu_double_vs_independent(o):
    """The oracle's double gelu against a 150-digit decimal evaluation of the tanh form
    (independent of libm; covers the negative tail), against torch's CPU float64
    tanh-GELU where its 1 + tanh form does not cancel (|x| <= 4), and the exact identity
    gelu(x) - gelu(-x) = x of the tanh form."""
    g = np.random.Generator(np.random.PCG64(51))
    xs = np.concatenate([g.standard_normal(300) * 3, g.uniform(-14, 12, 300),
                         [0.0, 1.0, -1.0, 5.5, -5.5, -7.17, -9.0, -11.5]])
    mine = np.array([o.gelu_double(x) for x in xs])
    ref = np.array([gelu_decimal(x) for x in xs])
    # double evaluation error: exp of an argument carrying |2u| * 2^-53 absolute error
    u2 = np.abs(2 * np.sqrt(2 / np.pi) * (xs + 0.044715 * xs ** 3))
    tol = (8 + 2 * u2) * 2.0 ** -52 * np.abs(ref)
    assert (np.abs(mine - ref) <= tol).all(), np.max(np.abs(mine - ref) / np.abs(ref))
    # torch evaluates the 1 + tanh(u) form, which loses ~|2u|/ln(10) digits to
    # cancellation for negative x: compare where that loss is small
    small = np.abs(xs) <= 2
    t = torch.nn.functional.gelu(torch.from_numpy(xs[small]), approximate="tanh").numpy()
    assert np.allclose(mine[small], t, rtol=1e-12, atol=1e-300), "torch"
    sym = np.array([o.gelu_double(x) - o.gelu_double(-x) for x in xs[np.abs(xs) < 5]])
    assert np.allclose(sym, xs[np.abs(xs) < 5], rtol=1e-14, atol=1e-14), "symmetry"


def pin_gelu_bf16_rounding(o):
    """y = RN_bf16(gelu(x)) for every finite bf16 x with |x| < 30: one rounding of the
    double value (exact rational round-half-even here), specials by their limits, and
    `alt` is either y or an adjacent bf16 value of the same sign."""
    xs, _ = _bf16_grid_sample()
    y, alt = o.gelu_bf16(xs)
    for i in range(0, xs.size, 37):
        gd = o.gelu_double(float(bf16_to_f32(xs[i:i + 1])[0]))
        want = rn_binary(abs(Fraction(gd)), 7, -126, 128)
        wb = (f2u(np.float32(float(want))) >> 16) | (0x8000 if gd < 0 or (gd == 0 and np.signbit(gd)) else 0)
        assert y[i] == wb, (hex(xs[i]), hex(y[i]), hex(wb))
    diff = y != alt
    assert diff.mean() < 0.01
    yd = y[diff].astype(np.int32)
    ad = alt[diff].astype(np.int32)
    assert ((yd ^ ad) & 0x8000 == 0).all() or ((yd & 0x7FFF) == 0).all()
    assert (np.abs((yd & 0x7FFF) - (ad & 0x7FFF)) == 1).all()
    sp = np.array([0x7F80, 0xFF80, 0x7FC0, 0x0000, 0x8000], np.uint16)
    ys, _ = o.gelu_bf16(sp)
    assert list(ys[:2]) == [0x7F80, 0x8000] and (ys[2] & 0x7FFF) > 0x7F80
    assert list(ys[3:]) == [0x0000, 0x8000]


def pin_gelu_ties_offer_both(o):
    """For tiny x, exp(-2u) rounds to 1 and gelu(x) = x/2 exactly; for bf16 x just above
    the normal minimum with an odd last bit, x/2 is an exact tie between two bf16
    subnormals.  RN picks the even one, and since the tie is inside any error window the
    other one must be offered as `alt` (both signs)."""
    m = np.arange(1, 128, 2, dtype=np.uint16)
    for sign in (0, 0x8000):
        xs = (0x0080 | m | sign).astype(np.uint16)      # (1 + m/128) * 2^-126, m odd
        y, alt = o.gelu_bf16(xs)
        lo = ((0x0040 | (m >> 1)) | sign).astype(np.uint16)   # (64 + (m-1)/2) * 2^-133
        hi = (lo + 1).astype(np.uint16)
        even = np.where((lo & 1) == 0, lo, hi)
        odd = np.where((lo & 1) == 0, hi, lo)
        assert (y == even).all(), (y[:4], even[:4])
        assert (alt == odd).all(), (alt[:4], odd[:4])


def pin_gelu_quantize(o):
    """The fused quantize is the plain bf16 quantize of y (and of alt)."""
    g = np.random.Generator(np.random.PCG64(53))
    x = f32_to_bf16_np((g.standard_normal(5000) * 4).astype(np.float32))
    codes, amax, codes_alt, lo, hi = o.gelu_quantize_amax(x, E4M3, 0.05)
    y, alt = o.gelu_bf16(x)
    c2, a2 = o.quantize_amax(y, E4M3, 0.05)
    assert (codes == c2).all() and f2u(amax) == f2u(a2)
    assert f2u(lo) <= f2u(amax) <= f2u(hi)


def _ln_case(seed, rows, H, lo_exp=-4, hi_exp=3, affine=True):
    g = np.random.Generator(np.random.PCG64(seed))
    x = f32_to_bf16_np((g.standard_normal(rows * H) * np.exp2(g.integers(lo_exp, hi_exp, rows * H))
                        + g.standard_normal(rows * H).astype(np.float32) * 0.5)
                       .astype(np.float32)).reshape(rows, H)
    gamma = (1 + 0.2 * g.standard_normal(H)).astype(np.float32) if affine else None
    beta = (0.3 * g.standard_normal(H)).astype(np.float32) if affine else None
    return x, gamma, beta


def pin_layernorm_vs_torch(o):
    """Mean, rstd and y against torch's CPU float64 layer_norm (an independent
    implementation: biased variance, eps inside the square root, affine gamma/beta);
    y must be RN_bf16 of torch's value wherever that value is not within 1e-9 relative
    of a bf16 rounding midpoint."""
    for seed, rows, H, eps in ((61, 16, 4096, 1e-6), (62, 9, 1000, 1e-6), (63, 5, 8, 1e-3),
                               (64, 7, 768, 0.0)):
        x, gamma, beta = _ln_case(seed, rows, H)
        y, _, _, mean, rstd = o.layernorm_bf16(x, gamma, beta, eps)
        xt = torch.from_numpy(bf16_to_f32(x.reshape(-1)).astype(np.float64).reshape(rows, H))
        e32 = float(np.float32(eps))
        ref = torch.nn.functional.layer_norm(xt, (H,), torch.from_numpy(gamma.astype(np.float64)),
                                             torch.from_numpy(beta.astype(np.float64)),
                                             eps=e32).numpy()
        var, mu = torch.var_mean(xt, dim=1, unbiased=False)
        assert np.allclose(mean, mu.numpy(), rtol=1e-12, atol=1e-15)
        assert np.allclose(rstd, 1 / np.sqrt(var.numpy() + e32), rtol=1e-12)
        # rounding of torch's value: f32 cast is RN to 24 bits, then RN to bf16 of that
        # f32 (double rounding) is only wrong near midpoints, which are excluded
        r32 = ref.astype(np.float32)
        want = f32_to_bf16_np(r32)
        b = r32.view(np.uint32)
        mid_dist = np.abs((b & 0xFFFF).astype(np.int64) - 0x8000)
        safe = mid_dist > 2
        assert (y.reshape(-1)[safe.reshape(-1)] == want.reshape(-1)[safe.reshape(-1)]).all()


def pin_layernorm_closed_forms(o):
    """Rows with known answers: +-a alternating (mean 0, V = a^2, y = +-a/sqrt(a^2+eps),
    exactly +-1 at eps = 0); a constant row gives beta exactly (d = 0) at eps > 0 and the
    positive NaN at eps = 0 (0/0); inf or NaN in a row makes the whole row NaN; H = 1 is
    a constant row; shifting integer rows by 128 and doubling at eps = 0 change nothing."""
    H = 64
    a = 3.0
    row = np.where(np.arange(H) % 2 == 0, a, -a).astype(np.float32)
    xb = f32_to_bf16_np(row).reshape(1, H)
    y, _, _, mean, rstd = o.layernorm_bf16(xb, None, None, 0.0)
    assert (y == f32_to_bf16_np(np.where(np.arange(H) % 2 == 0, 1.0, -1.0).astype(np.float32))).all()
    assert mean[0] == 0.0 and rstd[0] == 1 / 3.0
    eps = float(np.float32(1e-2))
    y = o.layernorm_bf16(xb, None, None, 1e-2)[0]
    v = a / np.sqrt(a * a + eps)
    assert (bf16_to_f32(y.reshape(-1))[::2] == bf16_to_f32(f32_to_bf16_np(np.float32([v])))[0]).all()
    const = np.full((2, 16), 0x4040, np.uint16)                 # 3.0
    beta = np.linspace(-2, 2, 16).astype(np.float32)
    y, _, _, mean, rstd = o.layernorm_bf16(const, None, beta, 1e-6)
    assert (y == f32_to_bf16_np(beta)[None, :]).all() and mean[0] == 3.0
    y, y_lo, y_hi, _, _ = o.layernorm_bf16(const, None, beta, 0.0)
    assert (y == 0x7FC0).all() and (y_lo == 0x7FC0).all() and (y_hi == 0x7FC0).all()
    bad = np.tile(np.uint16(0x3F80), (3, 8))
    bad[0, 3] = 0x7F80
    bad[1, 5] = 0xFFC1
    bad[2, 0] = 0xFF80
    y, _, _, mean, rstd = o.layernorm_bf16(bad, None, None, 1e-6)
    assert (y == 0x7FC0).all() and np.isnan(mean).all() and np.isnan(rstd).all()
    y = o.layernorm_bf16(np.array([[0x4000], [0xC2F6]], np.uint16), None,
                         np.array([0.75], np.float32), 1e-6)[0]
    assert list(y[:, 0]) == [0x3F40, 0x3F40]
    g = np.random.Generator(np.random.PCG64(65))
    ints = g.integers(0, 128, (4, 256)).astype(np.float32)
    y1 = o.layernorm_bf16(f32_to_bf16_np(ints), None, None, 0.0)[0]
    y2 = o.layernorm_bf16(f32_to_bf16_np(ints + 128), None, None, 0.0)[0]
    y3 = o.layernorm_bf16(f32_to_bf16_np(ints * 2), None, None, 0.0)[0]
    assert (y1 == y2).all() and (y1 == y3).all()


def _bf16_order(h: np.ndarray) -> np.ndarray:
    """bf16 bits -> integers in value order (-0 and +0 equal)."""
    h = h.astype(np.int64)
    return np.where(h & 0x8000, -(h & 0x7FFF), h & 0x7FFF)


def pin_layernorm_admissible_range(o):
    """[y_lo, y_hi] holds y; it is y alone for most elements, a range wider than one
    bf16 step only where |y| is small against the window's absolute terms; it equals
    [y - w, y + w] rounded, checked against the window recomputed here from its formula
    on a sample; an exact tie (a constant row gives y = beta exactly, beta a bf16
    midpoint) has y even and the range holding both neighbours; the fused quantize
    equals the plain quantize of y, and the amax bounds bracket it."""
    x, gamma, beta = _ln_case(66, 32, 2048)
    y, y_lo, y_hi, mean, rstd = o.layernorm_bf16(x, gamma, beta, 1e-6)
    oy, ol, oh = _bf16_order(y), _bf16_order(y_lo), _bf16_order(y_hi)
    assert (ol <= oy).all() and (oy <= oh).all()
    assert 0 < (ol != oh).mean() < 0.05
    # the window from its definition, on every element of row 3
    H = 2048
    L = math.ceil(math.log2(H)) + 10
    xf = bf16_to_f32(x[3]).astype(np.float64)
    mu = xf.mean()
    d = xf - mu
    r = 1 / np.sqrt((d * d).mean() + float(np.float32(1e-6)))
    A, Ad = np.abs(xf).mean(), np.abs(d).mean()
    g64, b64 = gamma.astype(np.float64), beta.astype(np.float64)
    v = g64 * d * r + b64
    w = 2.0 ** -23 * (np.abs(g64) * r * (np.abs(d) * (L / 2 + 7 + L * L * 2.0 ** -24 * A * Ad * r * r)
                                       + L * Ad + L * L * 2.0 ** -24 * A) + np.abs(v)) + 2.0 ** -147
    def rn_bf16_exact(val: float) -> float:
        r = rn_binary(abs(Fraction(val)), 7, -126, 128)
        return math.copysign(float("inf") if r is None else float(r), val)

    for i in range(H):
        lo_f = float(bf16_to_f32(y_lo[3, i:i + 1])[0])
        hi_f = float(bf16_to_f32(y_hi[3, i:i + 1])[0])
        # v and w carry double rounding (~2^-50 relative); the ends are compared where
        # v -+ w is not within 2^-40 of a bf16 rounding midpoint
        for end, val in ((lo_f, v[i] - w[i]), (hi_f, v[i] + w[i])):
            near = rn_bf16_exact(val * (1 - 2.0 ** -40)) != rn_bf16_exact(val * (1 + 2.0 ** -40))
            assert near or end == rn_bf16_exact(val), (i, end, val)
    # ties with the even neighbour above and below, both signs
    mids = np.array([1 + 2 ** -8, -(1 + 3 * 2 ** -8), 1.5 * 2 ** -9 + 2 ** -17, 1 + 3 * 2 ** -8,
                     -(1 + 2 ** -8)], np.float32)
    const = np.full((1, mids.size), 0x3F80, np.uint16)
    y, y_lo, y_hi, _, _ = o.layernorm_bf16(const, None, mids, 1e-6)
    m = mids.view(np.uint32)
    lo = (m >> 16).astype(np.uint16)
    assert ((y[0] & 1) == 0).all()
    for k in range(mids.size):  # each range is exactly the two neighbours, in value order
        assert {int(y_lo[0, k]), int(y_hi[0, k])} == {int(lo[k]), int(lo[k]) + 1}
        assert _bf16_order(y_lo[0, k:k + 1])[0] < _bf16_order(y_hi[0, k:k + 1])[0]
    codes, amax, c_lo, c_hi, a_lo, a_hi, _, _ = o.layernorm_quantize_amax(x, E4M3, 0.02, gamma,
                                                                         beta, 1e-6)
    c2, am2 = o.quantize_amax(o.layernorm_bf16(x, gamma, beta, 1e-6)[0], E4M3, 0.02)
    assert (codes == c2).all() and f2u(amax) == f2u(am2)
    assert f2u(a_lo) <= f2u(amax) <= f2u(a_hi)


def _torch_decode(codes: np.ndarray, fmt: int) -> np.ndarray:
    """FP8 codes -> float64 through torch's CPU float8 types (independent of the oracle)."""
    dt = torch.float8_e4m3fn if fmt == E4M3 else torch.float8_e5m2
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(dt).to(torch.float64).numpy()


def _finite_codes(g, shape, fmt):
    c = g.integers(0, 256, shape).astype(np.uint8)
    if fmt == E4M3:
        c[(c & 0x7F) == 0x7F] = 0x38
    else:
        c[(c & 0x7C) == 0x7C] = 0x3C
    return c


def pin_gemm_vs_float64_matmul(o):
    """E4M3 x E4M3 with K <= 64: every partial sum of decoded products fits a double (the
    products span 2^-18 .. 2^17.6), so numpy's float64 matmul of torch-decoded operands is
    exact and the oracle must equal it bit for bit (times the scales). Pairings with E5M2
    span too many binades for that: there the oracle is compared with the exact rational
    sum (Python Fractions) to its stated 2^-51. C_abs is the matmul of |.| in all cases."""
    g = np.random.Generator(np.random.PCG64(81))
    sa, sb = float(np.float32(0.37)), float(np.float32(3.5e-3))
    for fa, fb, M, N, K in ((E4M3, E4M3, 7, 5, 64), (E4M3, E4M3, 3, 2, 17), (E5M2, E4M3, 3, 4, 48),
                            (E4M3, E5M2, 4, 4, 33), (E5M2, E5M2, 5, 6, 16)):
        A = _finite_codes(g, (M, K), fa)
        B = _finite_codes(g, (N, K), fb)
        C, Cabs, Cg = o.fp8_gemm(A, fa, B, fb, sa, sb)
        da, db = _torch_decode(A, fa), _torch_decode(B, fb)
        # group maxima over k in [8q, 8q + 8), from the decoded products
        P = np.abs(da[:, None, :] * db[None, :, :])
        pad = (-K) % 8
        Pg = np.pad(P, ((0, 0), (0, 0), (0, pad))).reshape(M, N, -1, 8).max(axis=3).sum(axis=2)
        assert np.allclose(Cg, Pg * abs(sa * sb), rtol=1e-14, atol=0)
        if fa == E4M3 and fb == E4M3:
            ref = (da @ db.T) * (sa * sb)
            assert (C == ref).all(), np.max(np.abs(C - ref))
        else:
            for m in range(M):
                for n in range(N):
                    ex = sum(Fraction(float(da[m, k])) * Fraction(float(db[n, k])) for k in range(K))
                    want = float(ex * Fraction(sa) * Fraction(sb))
                    assert abs(C[m, n] - want) <= 2.0 ** -50 * abs(want) + 1e-300, (m, n)
        assert np.allclose(Cabs, (np.abs(da) @ np.abs(db).T) * abs(sa * sb), rtol=1e-14, atol=0)
        assert (Cabs >= np.abs(C) * (1 - 1e-15)).all()


def pin_gemm_exact_large_k(o):
    """Sums that do not fit a double: E5M2 extremes (57344^2 against 2^-16 * 2^-16 terms)
    over K = 4096, against Python integers; identity operands return the other operand."""
    g = np.random.Generator(np.random.PCG64(82))
    K = 4096
    A = np.full((2, K), 0x01, np.uint8)              # 2^-16 (smallest E5M2 subnormal)
    B = np.full((2, K), 0x01, np.uint8)
    A[0, 0] = B[0, 0] = 0x7B                          # 57344
    A[1, 5] = 0xFB                                    # -57344 against +2^-16
    C = o.fp8_gemm(A, E5M2, B, E5M2)[0]
    exact00 = Fraction(57344) ** 2 + (K - 1) * Fraction(1, 2 ** 32)
    assert C[0, 0] == float(exact00)
    exact10 = sum(Fraction(_torch_decode(A[1:2, k:k + 1], E5M2)[0, 0]) *
                  Fraction(_torch_decode(B[0:1, k:k + 1], E5M2)[0, 0]) for k in range(K))
    assert C[1, 0] == float(exact10)
    # identity: A = I (codes of 1.0), C = decode(B) as rows
    n = 16
    I = np.zeros((n, n), np.uint8)
    I[np.arange(n), np.arange(n)] = 0x38           # E4M3 1.0
    Bc = _finite_codes(g, (5, n), E4M3)
    C = o.fp8_gemm(I, E4M3, Bc, E4M3)[0]
    assert (C == _torch_decode(Bc, E4M3).T).all()


def pin_gemm_specials(o):
    """NaN operands, inf * 0 and inf - inf give NaN; inf times a nonzero finite value
    gives a signed inf (E5M2 has inf codes); finite rows elsewhere are unaffected."""
    A = np.full((4, 4), 0x3C, np.uint8)              # E5M2 1.0
    B = np.full((3, 4), 0x3C, np.uint8)
    A[0, 1] = 0x7F                                    # NaN
    A[1, 2] = 0x7C                                    # +inf
    A[2, 2] = 0x7C
    A[2, 3] = 0xFC                                    # +inf and -inf in one dot
    B[1, 2] = 0x00                                    # 0 against row 1's inf
    B[2, :] = 0xBC                                    # -1.0
    C = o.fp8_gemm(A, E5M2, B, E5M2)[0]
    assert np.isnan(C[0]).all()
    assert C[1, 0] == np.inf and np.isnan(C[1, 1]) and C[1, 2] == -np.inf
    assert np.isnan(C[2]).all()
    assert (C[3] == np.array([4.0, 3.0, -4.0])).all()     # B row 1 has one zero


def f32_to_bf16_np(v: np.ndarray) -> np.ndarray:
    u = v.view(np.uint32)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
