"""GPU parity at the largest sizes: tensors past 2^31 elements and 4 GiB of bytes, where
element indices, unit counts and byte offsets need 64 bits.  Every code byte and the amax
are compared with the oracle; the amax is planted in the scalar tail, past index 2^31."""
import numpy as np
import pytest
import torch

import workloads
from gpu_path import bits, dev_src, f32, note

pytestmark = pytest.mark.gpu

E4M3, E5M2 = 0, 1


def _big(base: np.ndarray, numel: int) -> np.ndarray:
    reps = -(-numel // base.size)
    return np.tile(base, reps)[:numel]


def _compare(orc, x, fmt, scale, got_codes, got_amax):
    want, wa = orc.quantize_amax(x, fmt, scale, threads=workloads.default_threads())
    bad = np.flatnonzero(got_codes != want)
    assert bad.size == 0, ("codes differ", bad[:8], bad.size)
    assert bits(got_amax) == bits(wa), (got_amax, wa)


def test_bf16_past_2_31_elements_one_launch_step(orc):
    """2^31 + 5 bf16 elements (4 GiB + 10 B read, 2 GiB + 5 B of codes) through the
    one-launch step: codes, amax (in history row 0), scale."""
    import delayed_scaling_amax_amd as d
    numel = (1 << 31) + 5
    x = _big(workloads.random_bf16(1 << 20, 51, -8, 8), numel)
    x[numel - 3] = 0x4700  # 32768: the largest |x|, in the scalar tail past 2^31
    x[(1 << 31) + 1] = 0xC6FE  # -32512, also past 2^31 (the second largest)
    note("large: bf16 %d elements, one-launch step" % numel)
    src = dev_src(x)
    dst = torch.empty(numel, dtype=torch.uint8, device="cuda")
    scale, scale_inv = f32([0.3]), torch.zeros(1, dtype=torch.float32, device="cuda")
    amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    hist = torch.zeros(4, 1, dtype=torch.float32, device="cuda")
    fmts = torch.zeros(1, dtype=torch.uint8, device="cuda")
    ws = torch.zeros(1, dtype=torch.int32, device="cuda")
    d.fp8_quantize_amax_and_update([(src, dst, scale, amax, E4M3)], amax, hist, scale,
                                   scale_inv, fmts, ws, reset_amax=True)
    torch.cuda.synchronize()
    del src
    got = dst.cpu().numpy()
    del dst
    h = hist.cpu().numpy()
    assert float(h[0, 0]) == 32768.0
    _compare(orc, x, E4M3, float(np.float32(0.3)), got, h[0, 0])
    r = orc.amax_and_scale_update(h[0].copy(), np.zeros((4, 1), np.float32),
                                  np.array([0.3], np.float32), np.zeros(1, np.uint8),
                                  reset_amax=True)
    assert bits(scale.cpu().numpy()) == bits(r["scale"])
    assert bits(scale_inv.cpu().numpy()) == bits(r["scale_inv"])
    assert int(ws.item()) == 0


def test_f32_past_4_gib(orc):
    """(2^30 + 2^20 + 7) fp32 elements (4.004 GiB read) to E5M2; source 4 bytes and codes
    5 bytes past an aligned address, so the 16-byte body starts after a 3-element head."""
    import delayed_scaling_amax_amd as d
    numel = (1 << 30) + (1 << 20) + 7
    x = _big(workloads.random_f32(1 << 20, 52, -12, 12), numel)
    x[numel - 2] = -1.5e30  # the largest |x| (saturates), past 4 GiB of source bytes
    note("large: f32 %d elements (+1 element offset)" % numel)
    buf = torch.empty(numel + 1, dtype=torch.float32, device="cuda")
    buf[1:].copy_(torch.from_numpy(x))
    src = buf[1:]
    dbuf = torch.empty(numel + 5, dtype=torch.uint8, device="cuda")
    dst = dbuf[5:]
    amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    d.fp8_quantize_amax(src, dst, f32([0.37]), amax, E5M2)
    torch.cuda.synchronize()
    del buf, src
    got = dst.cpu().numpy()
    del dst, dbuf
    _compare(orc, x, E5M2, float(np.float32(0.37)), got, amax.cpu().numpy()[0])


@pytest.mark.parametrize("numel", [(1 << 28) - 8, 1 << 28])
def test_store_policy_threshold(orc, numel):
    """Launches of at least 256 MiB of codes take the instance with non-temporal stores,
    smaller ones the default instance: both sides of the threshold, one bf16 tensor
    with a ragged view (offset 1) in the multi-tensor launch and through a plan, every
    code byte and the amax against the oracle."""
    import delayed_scaling_amax_amd as d
    x = _big(workloads.random_bf16(1 << 20, 52, -6, 6, specials=True), numel)
    note("large: store-policy threshold, %d elements" % numel)
    buf = torch.empty(numel + 1, dtype=torch.bfloat16, device="cuda")
    src = buf[1:]
    src.copy_(dev_src(x))
    dst = torch.empty(numel, dtype=torch.uint8, device="cuda")
    scale = f32([0.05])
    amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    d.fp8_multi_quantize_amax([(src, dst, scale, amax, E5M2)])
    torch.cuda.synchronize()
    got, got_amax = dst.cpu().numpy(), amax.cpu().numpy()[0]
    want, wa = orc.quantize_amax(x, E5M2, float(np.float32(0.05)),
                                 threads=workloads.default_threads())
    assert np.array_equal(got, want)
    assert bits(got_amax) == bits(wa)
    note("large: store-policy threshold, %d elements, planned" % numel)
    dst.fill_(0xAA)
    amax.zero_()
    d.fp8_multi_quantize_amax_planned(d.fp8_multi_quantize_plan([(src, dst, scale, amax, E5M2)]))
    torch.cuda.synchronize()
    assert np.array_equal(dst.cpu().numpy(), want)
    assert bits(amax.cpu().numpy()[0]) == bits(wa)
