"""GPU parity: fp8_quantize_amax_and_update (one delayed-scaling step: the multi-tensor
quantize + amax and the batched update, in one launch when it fits) vs the CPU oracle's
quantize followed by its update.

The bar is bit-exact on every FP8 byte, amax, history, scale and scale_inv, over
several consecutive steps (each step quantizes with the scale the previous step wrote),
and the workspace counter is back at 0 after every call."""
import numpy as np
import pytest
import torch

import workloads
from gpu_path import bits, dev_src, f32, note

pytestmark = pytest.mark.gpu

E4M3, E5M2 = 0, 1


class Step:
    """Device state of one delayed-scaling loop and the oracle's copy of it."""

    def __init__(self, xs, fmts, H, n_upd=None, first_scale=None, hist=None):
        self.xs, self.fmts = xs, list(fmts)
        n = len(xs) if n_upd is None else n_upd
        self.n, self.H = n, H
        upd_fmts = (self.fmts + [E5M2 if k % 3 == 2 else E4M3 for k in range(n)])[:n]
        self.o_fmt = np.array(upd_fmts, np.uint8)
        self.o_scale = (np.ones(n, np.float32) if first_scale is None
                        else np.asarray(first_scale, np.float32).copy())
        self.o_hist = np.zeros((H, n), np.float32) if hist is None else hist.copy()
        self.o_amax = np.zeros(n, np.float32)
        self.srcs = [dev_src(x) for x in xs]
        self.dsts = [torch.empty(x.size, dtype=torch.uint8, device="cuda") for x in xs]
        self.scale = f32(self.o_scale)
        self.scale_inv = torch.zeros(n, dtype=torch.float32, device="cuda")
        self.amax = torch.zeros(n, dtype=torch.float32, device="cuda")
        self.hist = torch.from_numpy(self.o_hist.copy()).cuda()
        self.formats = torch.from_numpy(self.o_fmt.copy()).cuda()
        self.ws = torch.zeros(1, dtype=torch.int32, device="cuda")

    def entries(self):
        return [(self.srcs[i], self.dsts[i], self.scale[i:i + 1], self.amax[i:i + 1],
                 self.fmts[i]) for i in range(len(self.xs))]

    def run(self, orc, algo=0, margin=0, reset=True):
        import delayed_scaling_amax_amd as d
        d.fp8_quantize_amax_and_update(self.entries(), self.amax, self.hist, self.scale,
                                       self.scale_inv, self.formats, self.ws, algo=algo,
                                       margin=margin, reset_amax=reset)
        torch.cuda.synchronize()
        # oracle: quantize every tensor with the current scales, then the update
        codes = []
        for i, x in enumerate(self.xs):
            c, a = orc.quantize_amax(x, self.fmts[i], float(self.o_scale[i]),
                                     self.o_amax[i], threads=8)
            codes.append(c)
            self.o_amax[i] = a
        r = orc.amax_and_scale_update(self.o_amax, self.o_hist, self.o_scale, self.o_fmt,
                                      algo=algo, margin=margin, reset_amax=reset)
        for i, c in enumerate(codes):
            got = self.dsts[i].cpu().numpy().reshape(c.shape)
            bad = np.nonzero(got.reshape(-1) != c.reshape(-1))[0]
            assert bad.size == 0, ("codes", i, bad[:8])
        assert (bits(self.hist.cpu().numpy()) == bits(r["hist"])).all(), "history"
        assert (bits(self.scale.cpu().numpy()) == bits(r["scale"])).all(), "scale"
        assert (bits(self.scale_inv.cpu().numpy()) == bits(r["scale_inv"])).all(), "scale_inv"
        assert (bits(self.amax.cpu().numpy()) == bits(r["amax"])).all(), "amax"
        assert int(self.ws.item()) == 0, "workspace not left at 0"
        self.o_hist, self.o_scale, self.o_amax = r["hist"], r["scale"], r["amax"]


def bf16(g, n, scale=1.0):
    """n seeded N(0, scale^2) values as bf16 bits (round to nearest even)."""
    return workloads.f32_to_bf16_bits((g.standard_normal(n) * scale).astype(np.float32))


def test_single_1024_three_steps(orc):
    w = workloads.single_1024()
    note("fused step: single_1024, 3 steps")
    st = Step([w.tensors[0].data], [E4M3], w.history_len)
    for _ in range(3):
        st.run(orc)


def test_mlp_4096_two_steps(orc):
    """The benchmark's workload at full size: 3 tensors, history 16."""
    w = workloads.mlp_4096(threads=workloads.default_threads())
    note("fused step: mlp_4096 full size, 2 steps")
    st = Step([t.data for t in w.tensors], [E4M3] * 3, w.history_len)
    for _ in range(2):
        st.run(orc)


@pytest.mark.parametrize("algo,margin,reset", [(0, 0, True), (0, 1, False), (1, 0, True),
                                               (1, -1, False), (0, 3, True)])
def test_mixed_formats_history_1024(orc, algo, margin, reset):
    """5 tensors (bf16 and fp32 sources, E4M3 and E5M2, ragged sizes), history 1024
    (5120 history elements: several update chunks), 4 steps."""
    g = np.random.Generator(np.random.PCG64(9100 + 10 * algo + margin))
    xs = [bf16(g, 300001, 3.0), bf16(g, 77777, 1e-3), g.standard_normal(123457).astype(
        np.float32) * 50, bf16(g, 8, 1e4), bf16(g, 262144, 0.5)]
    fmts = [E4M3, E5M2, E4M3, E5M2, E4M3]
    hist = np.exp(g.normal(0, 2, (1024, 5))).astype(np.float32)
    note("fused step: mixed 5 tensors, H 1024, algo %d margin %d reset %d" % (algo, margin,
                                                                              reset))
    st = Step(xs, fmts, 1024, hist=hist)
    for _ in range(4):
        st.run(orc, algo=algo, margin=margin, reset=reset)


def test_special_amaxes_keep_previous_scale(orc):
    """NaN, inf, all-zero and subnormal-only tensors: the update keeps the previous scale
    where the amax is not usable, as the two-call form does."""
    nan = np.array([0x3F80, 0x7FC1, 0x4000], np.uint16)
    inf = np.array([0xFF80, 0x3F80], np.uint16)
    zero = np.zeros(1000, np.uint16)
    sub = np.array([0x0001, 0x8003, 0x0000], np.uint16)
    big = np.array([0x7F7F, 0x3F80], np.uint16)  # largest bf16: scale 7.6e35 / 448
    note("fused step: special amaxes")
    st = Step([nan, inf, zero, sub, big], [E4M3, E5M2, E4M3, E5M2, E4M3], 4,
              first_scale=[2.0, 0.5, 3.0, 1e-30, 1.0])
    for _ in range(3):
        st.run(orc, margin=0)


def test_update_wider_than_the_quantized_tensors(orc):
    """The update covers 7 tensors while the step quantizes 3 of them (the others only
    roll their history, with amax left as it was)."""
    g = np.random.Generator(np.random.PCG64(9200))
    xs = [bf16(g, 5000), bf16(g, 100000, 7.0), bf16(g, 64)]
    note("fused step: update over 7 columns, 3 tensors")
    st = Step(xs, [E4M3, E5M2, E4M3], 16, n_upd=7,
              hist=np.exp(g.normal(0, 1, (16, 7))).astype(np.float32))
    for _ in range(3):
        st.run(orc, reset=False)


@pytest.mark.parametrize("H,n_upd", [(1, 3), (1, 256), (256, 256), (2, 1), (65536, 1)])
def test_history_shapes_at_the_fused_limits(orc, H, n_upd):
    """H = 1 (no roll), 256 update columns (the most one launch takes), H n = 65536."""
    g = np.random.Generator(np.random.PCG64(9300 + H + n_upd))
    xs = [bf16(g, 40000), bf16(g, 999)][:n_upd]  # quantized tensors: amax[0], amax[1]
    hist = np.exp(g.normal(0, 2, (H, n_upd))).astype(np.float32)
    note("fused step: H %d n %d" % (H, n_upd))
    st = Step(xs, [E4M3, E5M2][:len(xs)], H, n_upd=n_upd, hist=hist)
    for _ in range(2):
        st.run(orc)


@pytest.mark.parametrize("H,n_upd", [(1, 1), (16, 1), (1024, 3), (2, 256)])
def test_one_block_grid(orc, H, n_upd):
    """A step small enough for a one-block grid: the block that rolls the history (the
    first to finish) is also the last, so it counts twice and then finishes the update."""
    g = np.random.Generator(np.random.PCG64(9350 + H + n_upd))
    xs = [bf16(g, 100, 3.0)]
    hist = np.exp(g.normal(0, 2, (H, n_upd))).astype(np.float32)
    note("fused step, one-block grid: H %d n %d" % (H, n_upd))
    st = Step(xs, [E4M3], H, n_upd=n_upd, hist=hist)
    for _ in range(3):
        st.run(orc)


@pytest.mark.parametrize("case", ["40 tensors", "H n > 65536", "257 columns", "all empty"])
def test_two_launch_forms(orc, case):
    """Calls the single launch does not take give the same results through two launches."""
    g = np.random.Generator(np.random.PCG64(9400))
    if case == "40 tensors":
        xs = [bf16(g, int(g.integers(1, 20000))) for _ in range(40)]
        fmts, H, n_upd = [i % 2 for i in range(40)], 16, None
    elif case == "H n > 65536":
        xs, fmts, H, n_upd = [bf16(g, 30000), bf16(g, 7)], [E4M3, E5M2], 40000, None
    elif case == "257 columns":
        xs, fmts, H, n_upd = [bf16(g, 30000)], [E4M3], 4, 257
    else:
        xs, fmts, H, n_upd = [np.zeros(0, np.uint16)] * 3, [E4M3] * 3, 8, None
    note("fused step, two-launch form: %s" % case)
    hist = np.exp(g.normal(0, 1, (H, len(xs) if n_upd is None else n_upd))).astype(np.float32)
    st = Step(xs, fmts, H, n_upd=n_upd, hist=hist)
    for _ in range(2):
        st.run(orc)


def test_matches_the_two_call_sequence_on_device(orc):
    """Bit-identical device state to fp8_multi_quantize_amax + fp8_amax_and_scale_update
    over 5 steps of a 3-tensor loop (same inputs, both sides on the GPU)."""
    import delayed_scaling_amax_amd as d
    g = np.random.Generator(np.random.PCG64(9500))
    xs = [bf16(g, 1 << 20), bf16(g, 333333, 1e-2), bf16(g, 4097, 30.0)]
    fmts = [E4M3, E5M2, E4M3]
    note("fused step vs two calls on the device, 5 steps")
    a, b = Step(xs, fmts, 32), Step(xs, fmts, 32)
    for _ in range(5):
        d.fp8_quantize_amax_and_update(a.entries(), a.amax, a.hist, a.scale, a.scale_inv,
                                       a.formats, a.ws, margin=1, reset_amax=True)
        d.fp8_multi_quantize_amax(b.entries())
        d.fp8_amax_and_scale_update(b.amax, b.hist, b.scale, b.scale_inv, b.formats,
                                    margin=1, reset_amax=True)
        torch.cuda.synchronize()
        for u, v in ((a.hist, b.hist), (a.scale, b.scale), (a.scale_inv, b.scale_inv),
                     (a.amax, b.amax)):
            assert (bits(u.cpu().numpy()) == bits(v.cpu().numpy())).all()
        for u, v in zip(a.dsts, b.dsts):
            assert torch.equal(u, v)
    assert int(a.ws.item()) == 0


def test_timed_events_cover_the_fused_kernel(orc):
    import delayed_scaling_amax_amd as d
    g = np.random.Generator(np.random.PCG64(9600))
    xs = [bf16(g, 1 << 22), bf16(g, 1 << 21)]
    note("fused step with profiling events")
    st = Step(xs, [E4M3, E4M3], 16)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    d.fp8_quantize_amax_and_update(st.entries(), st.amax, st.hist, st.scale, st.scale_inv,
                                   st.formats, st.ws, reset_amax=True, start_event=ev[0],
                                   stop_event=ev[1])
    torch.cuda.synchronize()
    assert ev[0].elapsed_time(ev[1]) > 0.0
    assert int(st.ws.item()) == 0
    # and the step's results are the oracle's (the same call once more, checked)
    st2 = Step(xs, [E4M3, E4M3], 16)
    st2.run(orc)


def test_one_workspace_across_grid_sizes(orc):
    """The same workspace through calls whose launches have 1 block, 64 blocks and the
    full persistent grid (and a two-launch form in between): every call is bit-exact and
    leaves the counter at 0."""
    import delayed_scaling_amax_amd as d
    g = np.random.Generator(np.random.PCG64(9700))
    ws = torch.zeros(1, dtype=torch.int32, device="cuda")
    cases = [[bf16(g, 100)], [bf16(g, 1 << 20)], [bf16(g, 1 << 24), bf16(g, 777)],
             [bf16(g, 50) for _ in range(40)], [bf16(g, 3000, 5.0)]]
    note("fused step: one workspace across grid sizes")
    for xs in cases:
        st = Step(xs, [i % 2 for i in range(len(xs))], 8)
        st.ws = ws  # shared
        for _ in range(2):
            st.run(orc)
        assert int(ws.item()) == 0
