"""GPU parity: planned multi-tensor quantize (fp8_multi_quantize_plan +
fp8_multi_quantize_amax_planned) against the CPU oracle, bit-exact on every code byte and
amax bit: the 1152-tensor list of the batched-update layout in one launch, with fp32
sources, misaligned views, shared amaxes, empty entries and a scale outside the division
window mixed in; the same plan reused for a second step with new scales; identical
results to the 32-entry launches of fp8_multi_quantize_amax."""
import numpy as np
import pytest
import torch

import workloads
from gpu_path import bits, note

pytestmark = pytest.mark.gpu


def _build_list(hidden=256, tokens=64, layers=96):
    """The 1152-tensor list (hidden 256, 64 tokens: 100.7 M elements) with variations:
    every 7th tensor as fp32, every 11th as a view starting 1-3 elements into its
    buffer, every 13th empty, and tensors of the same layer and module sharing one amax
    slot when their index is a multiple of 5."""
    w = workloads.list_1152(hidden=hidden, tokens=tokens, layers=layers)
    items = []
    for i, t in enumerate(w.tensors):
        x = t.data.reshape(-1)
        if i % 13 == 12:
            x = x[:0]
        if i % 7 == 3:
            x = (x.astype(np.uint32) << 16).view(np.float32)
        off = (i % 3) + 1 if i % 11 == 5 else 0
        fmt = 0 if t.fmt == workloads.E4M3 else 1
        items.append((x, off, fmt))
    return items


def _device(items, scales, slot_of):
    srcs, dsts, keep = [], [], []
    n_slots = max(slot_of) + 1
    amax = torch.zeros(n_slots, dtype=torch.float32, device="cuda")
    scale = torch.tensor(np.asarray(scales, np.float32), device="cuda")
    entries = []
    for i, (x, off, fmt) in enumerate(items):
        if x.dtype == np.uint16:
            buf = torch.empty(x.size + off, dtype=torch.bfloat16, device="cuda")
            src = buf[off:]
            src.copy_(torch.from_numpy(x.view(np.int16)).view(torch.bfloat16))
        else:
            buf = torch.empty(x.size + off, dtype=torch.float32, device="cuda")
            src = buf[off:]
            src.copy_(torch.from_numpy(x))
        dbuf = torch.empty(x.size + off, dtype=torch.uint8, device="cuda")
        dst = dbuf[off:]
        keep += [buf, dbuf]
        entries.append((src, dst, scale[i:i + 1], amax[slot_of[i]:slot_of[i] + 1], fmt))
        srcs.append(src)
        dsts.append(dst)
    return entries, amax, scale, keep


def _oracle(orc, items, scales, slot_of):
    n_slots = max(slot_of) + 1
    amax = np.zeros(n_slots, np.float32)
    codes = []
    for i, (x, off, fmt) in enumerate(items):
        c, a = orc.quantize_amax(x, fmt, float(scales[i]), amax_in=amax[slot_of[i]],
                                 threads=8)
        amax[slot_of[i]] = a
        codes.append(c.reshape(-1))
    return codes, amax


def _slots(n):
    # entries whose index is a multiple of 5 share the slot of their module (3 tensors)
    return [i // 3 if i % 5 == 0 else n + i for i in range(n)]


def _check(entries, amax, codes_o, amax_o):
    torch.cuda.synchronize()
    for i, e in enumerate(entries):
        got = e[1].cpu().numpy()
        assert got.tobytes() == codes_o[i].tobytes(), "entry %d codes differ" % i
    assert (bits(amax.cpu().numpy()) == bits(amax_o)).all()


def test_plan_1152_entries_one_launch(orc):
    import delayed_scaling_amax_amd as d
    items = _build_list()
    n = len(items)
    g = np.random.Generator(np.random.PCG64(1152))
    scales = np.exp2(g.uniform(-6, 2, n)).astype(np.float32)
    scales[100] = np.float32(2.0 ** -100)  # outside the division window: element-wise path
    slot_of = _slots(n)
    entries, amax, scale, keep = _device(items, scales, slot_of)
    note("plan: 1152 entries, %d elements" % sum(x.size for x, _, _ in items))
    plan = d.fp8_multi_quantize_plan(entries)
    d.fp8_multi_quantize_amax_planned(plan)
    codes_o, amax_o = _oracle(orc, items, scales, slot_of)
    _check(entries, amax, codes_o, amax_o)

    # the same plan, a second step: new scales (device values), amax zeroed
    scales2 = np.exp2(g.uniform(-8, 0, n)).astype(np.float32)
    scale.copy_(torch.tensor(scales2))
    amax.zero_()
    for e in entries:
        e[1].fill_(0xAA)
    note("plan: second step with new scales")
    d.fp8_multi_quantize_amax_planned(plan)
    codes_o2, amax_o2 = _oracle(orc, items, scales2, slot_of)
    _check(entries, amax, codes_o2, amax_o2)


def test_plan_equals_chunked_launches():
    """Same list through the 32-entry launches of fp8_multi_quantize_amax: identical
    codes and amaxes."""
    import delayed_scaling_amax_amd as d
    items = _build_list(hidden=128, tokens=32, layers=40)  # 480 entries
    n = len(items)
    g = np.random.Generator(np.random.PCG64(480))
    scales = np.exp2(g.uniform(-6, 2, n)).astype(np.float32)
    slot_of = _slots(n)
    e1, a1, _, k1 = _device(items, scales, slot_of)
    e2, a2, _, k2 = _device(items, scales, slot_of)
    note("plan vs chunked: 480 entries")
    d.fp8_multi_quantize_amax_planned(d.fp8_multi_quantize_plan(e1))
    d.fp8_multi_quantize_amax(e2)
    torch.cuda.synchronize()
    for i in range(n):
        assert e1[i][1].cpu().numpy().tobytes() == e2[i][1].cpu().numpy().tobytes(), i
    assert (bits(a1.cpu().numpy()) == bits(a2.cpu().numpy())).all()


def test_plan_small_and_empty(orc):
    """A plan of one tensor, of only empty tensors (no launch, amax untouched) and of a
    single element."""
    import delayed_scaling_amax_amd as d
    x = workloads.random_bf16(70001, 77, specials=True)
    items = [(x, 0, 0)]
    entries, amax, scale, keep = _device(items, [0.75], [0])
    note("plan: one tensor")
    d.fp8_multi_quantize_amax_planned(d.fp8_multi_quantize_plan(entries))
    codes_o, amax_o = _oracle(orc, items, [0.75], [0])
    _check(entries, amax, codes_o, amax_o)
    empties = [(x[:0], 0, 0), (x[:0], 2, 1)]
    entries, amax, scale, keep = _device(empties, [1.0, 1.0], [0, 0])
    amax.fill_(3.0)
    note("plan: empty tensors only")
    d.fp8_multi_quantize_amax_planned(d.fp8_multi_quantize_plan(entries))
    torch.cuda.synchronize()
    assert float(amax.item()) == 3.0
    one = [(x[5:6], 0, 1)]
    entries, amax, scale, keep = _device(one, [0.5], [0])
    d.fp8_multi_quantize_amax_planned(d.fp8_multi_quantize_plan(entries))
    codes_o, amax_o = _oracle(orc, one, [0.5], [0])
    _check(entries, amax, codes_o, amax_o)
