"""GPU parity on seeded random tensor lists: fp8_multi_quantize_amax (argument tables)
and the planned launch (fp8_multi_quantize_plan + fp8_multi_quantize_amax_planned) against
the CPU oracle, bit-exact on every code byte and amax bit.

Each list mixes what the fixed cases test one at a time: 1-32 tensors of sizes from 0 to
~1.3 M elements (empty, below one 16-byte unit, ragged tails, several chunks), bf16 and
fp32 sources, both formats, views starting 1-3 elements into their buffer, magnitudes over
2^-40 .. 2^40 with zeros, subnormals, infinities and NaNs mixed in, scales inside and
outside the division window (and zero, negative, infinite, NaN), and amax slots shared by
several tensors (accumulated in list order, starting from a nonzero value)."""
import numpy as np
import pytest
import torch

import workloads
from gpu_path import bits, note

pytestmark = pytest.mark.gpu

E4M3, E5M2 = 0, 1
ODD = [2.0 ** -100, 2.0 ** 126, 0.0, -1.5, float("inf"), float("nan"), 1e-40]


def make_list(seed):
    g = np.random.Generator(np.random.PCG64(5000 + seed))
    n = int(g.integers(1, 33))
    items = []
    for i in range(n):
        r = g.random()
        size = (0 if r < 0.06 else int(g.integers(1, 8)) if r < 0.15
                else int(g.integers(8, 4000)) if r < 0.45 else int(g.integers(4000, 300000))
                if r < 0.9 else int(g.integers(300000, 1300000)))
        lo = int(g.integers(-40, 0))
        x = workloads.random_bf16(size, 9000 + 37 * seed + i, lo_exp=lo,
                                  hi_exp=lo + int(g.integers(1, 41)), specials=True)
        if size and g.random() < 0.2:  # bf16 subnormals in a stretch
            k = int(g.integers(0, size))
            x[k:k + 64] = (np.arange(min(64, size - k)) % 127 + 1).astype(np.uint16)
        if g.random() < 0.3:  # fp32 source: the bf16 values with random low bits
            low = g.integers(0, 1 << 16, size).astype(np.uint32)
            x = ((x.astype(np.uint32) << 16) | low).view(np.float32)
        off = int(g.integers(1, 4)) if g.random() < 0.3 else 0
        fmt = E4M3 if g.random() < 0.6 else E5M2
        s = ODD[int(g.integers(0, len(ODD)))] if g.random() < 0.1 else \
            float(np.exp2(g.uniform(-20, 20)))
        items.append((x, off, fmt, float(np.float32(s))))
    slots = [int(g.integers(0, max(1, n // 3))) if g.random() < 0.4 else n + i
             for i in range(n)]
    amax0 = float(np.float32(np.exp2(g.uniform(-30, 0))))
    return items, slots, amax0


def device_list(items, slots, amax0):
    keep = []
    n_slots = max(slots) + 1
    amax = torch.full((n_slots,), amax0, dtype=torch.float32, device="cuda")
    scale = torch.tensor(np.asarray([it[3] for it in items], np.float32), device="cuda")
    entries = []
    for i, (x, off, fmt, _) in enumerate(items):
        if x.dtype == np.uint16:
            buf = torch.empty(x.size + off, dtype=torch.bfloat16, device="cuda")
            src = buf[off:]
            src.copy_(torch.from_numpy(x.view(np.int16)).view(torch.bfloat16))
        else:
            buf = torch.empty(x.size + off, dtype=torch.float32, device="cuda")
            src = buf[off:]
            src.copy_(torch.from_numpy(x))
        dbuf = torch.full((x.size + off,), 0xAA, dtype=torch.uint8, device="cuda")
        dst = dbuf[off:]
        keep += [buf, dbuf]
        entries.append((src, dst, scale[i:i + 1], amax[slots[i]:slots[i] + 1], fmt))
    return entries, amax, keep


def oracle_list(orc, items, slots, amax0):
    amax = np.full(max(slots) + 1, amax0, np.float32)
    codes = []
    for i, (x, _, fmt, s) in enumerate(items):
        c, a = orc.quantize_amax(x, fmt, s, amax_in=amax[slots[i]], threads=8)
        amax[slots[i]] = a
        codes.append(c.reshape(-1))
    return codes, amax


def check(entries, amax, codes, amax_o, what):
    torch.cuda.synchronize()
    for i, e in enumerate(entries):
        got = e[1].cpu().numpy()
        bad = np.nonzero(got != codes[i])[0]
        assert bad.size == 0, (what, "entry", i, bad[:8])
    assert (bits(amax.cpu().numpy()) == bits(amax_o)).all(), (what, "amax")


@pytest.mark.parametrize("seed", range(8))
def test_random_list(orc, seed):
    import delayed_scaling_amax_amd as d
    items, slots, amax0 = make_list(seed)
    note("random list %d: %d tensors, %d elements" % (seed, len(items),
                                                      sum(it[0].size for it in items)))
    codes, amax_o = oracle_list(orc, items, slots, amax0)
    entries, amax, keep = device_list(items, slots, amax0)
    d.fp8_multi_quantize_amax(entries)
    check(entries, amax, codes, amax_o, "argument tables")
    entries, amax, keep = device_list(items, slots, amax0)
    note("random list %d: planned launch" % seed)
    d.fp8_multi_quantize_amax_planned(d.fp8_multi_quantize_plan(entries))
    check(entries, amax, codes, amax_o, "planned")
