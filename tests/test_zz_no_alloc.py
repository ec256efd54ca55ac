"""GPU test of the allocation-free multi-tensor quantize (fp8_multi_quantize_amax_noalloc,
plan in the library's fixed device array) through the C ABI: two calls in a row, the
second with a smaller list, then a larger one again, each bit-exact (codes and amax bits)
against the workspace entry points (fp8_multi_quantize_plan +
fp8_multi_quantize_amax_planned) on the same inputs."""
import ctypes

import numpy as np
import pytest
import torch

import workloads
from gpu_path import note

pytestmark = pytest.mark.gpu


def _entries(n_tensors, tag, misalign):
    """n_tensors bf16/fp32 tensors of ragged sizes (0 .. 300k elements), both formats,
    some views starting 1-3 elements into their buffers; two output sets (reference and
    allocation-free) with their own amax slots, scales shared."""
    g = np.random.Generator(np.random.PCG64(tag))
    sizes = (np.exp2(g.uniform(0, 18.2, n_tensors))).astype(np.int64)
    sizes[::17] = 0
    scale = torch.tensor(np.exp2(g.uniform(-6, 3, n_tensors)).astype(np.float32), device="cuda")
    outs = []
    keep = []
    srcs = []
    for i, m in enumerate(sizes):
        x = workloads.random_bf16(int(m), tag * 10000 + i, lo_exp=-12, hi_exp=12,
                                  specials=(i % 5 == 0))
        off = (i % 3) + 1 if (misalign and i % 4 == 1) else 0
        if i % 6 == 2:
            buf = torch.empty(int(m) + off, dtype=torch.float32, device="cuda")
            src = buf[off:]
            src.copy_(torch.from_numpy((x.astype(np.uint32) << 16).view(np.float32)))
        else:
            buf = torch.empty(int(m) + off, dtype=torch.bfloat16, device="cuda")
            src = buf[off:]
            src.copy_(torch.from_numpy(x.view(np.int16)).view(torch.bfloat16))
        keep.append(buf)
        srcs.append((src, off, i % 2))
    for _ in range(2):
        amax = torch.zeros(n_tensors, dtype=torch.float32, device="cuda")
        ent = []
        for i, (src, off, fmt) in enumerate(srcs):
            dbuf = torch.full((src.numel() + off,), 0x5A, dtype=torch.uint8, device="cuda")
            keep.append(dbuf)
            ent.append((src, dbuf[off:], scale[i:i + 1], amax[i:i + 1], fmt))
        outs.append((ent, amax))
    return outs, keep


def _same(a, b):
    (ea, aa), (eb, ab) = a, b
    torch.cuda.synchronize()
    for i in range(len(ea)):
        assert torch.equal(ea[i][1], eb[i][1]), "entry %d codes differ" % i
    assert torch.equal(aa.view(torch.int32), ab.view(torch.int32)), "amax differs"


def test_noalloc_matches_workspace_entry_points():
    import delayed_scaling_amax_amd as d
    for n_tensors, tag in ((400, 1), (37, 2), (900, 3)):  # the second call is smaller
        (ref, alloc_free), keep = _entries(n_tensors, tag, misalign=True)
        note("noalloc: %d tensors (tag %d)" % (n_tensors, tag))
        d.fp8_multi_quantize_amax_planned(d.fp8_multi_quantize_plan(ref[0]))
        arr = d._entry_table(alloc_free[0], torch.device("cuda", 0))
        st = d.lib.fp8_multi_quantize_amax_noalloc(arr, n_tensors,
                                                   torch.cuda.current_stream().cuda_stream)
        assert st == d.OK, d.fp8_status_string(st)
        _same(ref, alloc_free)
        del keep
