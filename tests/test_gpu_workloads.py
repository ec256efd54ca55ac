"""GPU parity at the full workload sizes: two delayed-scaling steps (quantize with the
previous scale + fused amax in one multi-tensor launch, then the batched in-place
update), every FP8 byte, amax, history, scale and scale_inv compared bit-exactly with
the CPU oracle running the same steps on the same input bytes."""
import numpy as np
import pytest
import torch

import workloads
from gpu_path import FMT, bits, dev_src, f32, note

pytestmark = pytest.mark.gpu


def two_steps(orc, w, steps=2, threads=16):
    import delayed_scaling_amax_amd as d
    n = len(w.tensors)
    fmts = [FMT[t.fmt] for t in w.tensors]
    srcs = [dev_src(t.data) for t in w.tensors]
    dsts = [torch.empty(t.data.size, dtype=torch.uint8, device="cuda") for t in w.tensors]
    scale = f32(w.first_scale)
    scale_inv = torch.empty(n, dtype=torch.float32, device="cuda")
    amax = torch.zeros(n, dtype=torch.float32, device="cuda")
    hist = torch.zeros(w.history_len, n, dtype=torch.float32, device="cuda")
    fdev = torch.tensor(fmts, dtype=torch.uint8, device="cuda")
    # oracle state
    o_scale = np.asarray(w.first_scale, np.float32)
    o_hist = np.zeros((w.history_len, n), np.float32)
    for step in range(steps):
        note("%s step %d" % (w.name, step))
        d.fp8_multi_quantize_amax([(srcs[i], dsts[i], scale[i:i + 1], amax[i:i + 1], fmts[i])
                                   for i in range(n)])
        torch.cuda.synchronize()
        g_amax = amax.cpu().numpy()
        o_amax = np.zeros(n, np.float32)
        for i, t in enumerate(w.tensors):
            want, o_amax[i] = orc.quantize_amax(t.data, fmts[i], float(o_scale[i]),
                                                threads=threads)
            got = dsts[i].cpu().numpy().reshape(t.data.shape)
            if not np.array_equal(got, want):
                bad = np.argwhere(got != want)[:5]
                pytest.fail("%s step %d tensor %s: %d bytes differ, first %s" % (
                    w.name, step, t.name, int((got != want).sum()), bad.tolist()))
            del want, got
        assert (bits(g_amax) == bits(o_amax)).all(), (g_amax, o_amax)
        d.fp8_amax_and_scale_update(amax, hist, scale, scale_inv, fdev, reset_amax=True)
        torch.cuda.synchronize()
        r = orc.amax_and_scale_update(o_amax, o_hist, o_scale, np.array(fmts, np.uint8),
                                      reset_amax=True)
        o_hist, o_scale = r["hist"], r["scale"]
        assert (bits(hist.cpu().numpy()) == bits(o_hist)).all()
        assert (bits(scale.cpu().numpy()) == bits(o_scale)).all()
        assert (bits(scale_inv.cpu().numpy()) == bits(r["scale_inv"])).all()
        assert (amax.cpu().numpy() == 0).all()
    return o_scale


def test_single_1024(orc):
    s = two_steps(orc, workloads.single_1024())
    assert s[0] > 0


def test_mlp_4096(orc):
    two_steps(orc, workloads.mlp_4096())


@pytest.mark.timeout(900)
def test_grad_8192x16384_saturation(orc):
    w = workloads.grad_8192x16384()
    sat = orc.count_saturated(w.tensors[0].data[:512], 1, w.first_scale[0])
    assert sat >= 0
    two_steps(orc, w, steps=1)
    # the stale scale saturates roughly 0.1% of the gradient (reported, loosely bounded)
    full = sum(orc.count_saturated(w.tensors[0].data[r:r + 1024], 1, w.first_scale[0])
               for r in range(0, w.tensors[0].data.shape[0], 1024))
    frac = full / w.tensors[0].data.size
    note("grad saturated fraction %.5f%%" % (100 * frac))
    assert 2e-4 < frac < 2e-3


@pytest.mark.timeout(1200)
def test_mlp_12288_full_step(orc):
    two_steps(orc, workloads.mlp_12288())
