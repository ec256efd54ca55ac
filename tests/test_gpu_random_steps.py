"""GPU parity of the whole delayed-scaling step (fp8_quantize_amax_and_update) on seeded
random configurations against the CPU oracle: its quantize of every tensor, then its
update. Codes, amax, history, scale and scale_inv must match bit for bit over three
consecutive steps, and the workspace counter must return to 0 after every call.

Each case draws:
- 1-32 tensors, bf16 and fp32, both formats, sizes from empty to about 600 k elements,
  with special values;
- update columns from the tensor count up to 256 (columns past the tensors carry an
  amax of their own);
- history lengths of 1-1024; every fourth case is past the single-launch limit and
  takes the two-launch form;
- both history reductions, margins from -3 to 3, and amax reset on or off;
- histories with zeros, infinities and NaNs, and first scales over 2^-12 .. 2^4 with
  an odd value now and then."""
import numpy as np
import pytest

import workloads
from gpu_path import note
from test_gpu_step import Step

pytestmark = pytest.mark.gpu

ODD = [0.0, float("inf"), float("nan"), -2.0, 2.0 ** -100]


def make_case(seed):
    g = np.random.Generator(np.random.PCG64(7000 + seed))
    nt = int(g.integers(1, 33))
    xs, fmts = [], []
    for i in range(nt):
        r = g.random()
        size = (0 if r < 0.05 else int(g.integers(1, 4000)) if r < 0.5
                else int(g.integers(4000, 600000)))
        lo = int(g.integers(-30, 0))
        x = workloads.random_bf16(size, 20000 + 41 * seed + i, lo_exp=lo,
                                  hi_exp=lo + int(g.integers(1, 40)), specials=True)
        if g.random() < 0.3:  # fp32 source: the bf16 values with random low bits
            low = g.integers(0, 1 << 16, size).astype(np.uint32)
            x = ((x.astype(np.uint32) << 16) | low).view(np.float32)
        xs.append(x)
        fmts.append(0 if g.random() < 0.6 else 1)
    n_upd = min(256, nt + (int(g.integers(0, 200)) if g.random() < 0.5 else 0))
    H = int(g.choice([1, 2, 3, 16, 64, 255, 1024]))
    if seed % 4 == 3:  # past the single-launch limit (history x columns > 65536)
        H, n_upd = 1024, max(n_upd, 100)
    hist = np.exp(g.normal(0.0, 3.0, (H, n_upd))).astype(np.float32)
    u = g.random((H, n_upd))
    hist[u < 0.1] = 0.0
    hist[(u >= 0.1) & (u < 0.11)] = np.inf
    hist[(u >= 0.11) & (u < 0.12)] = np.nan
    first = np.exp2(g.uniform(-12, 4, n_upd)).astype(np.float32)
    for k in np.nonzero(g.random(n_upd) < 0.05)[0]:
        first[k] = np.float32(ODD[int(g.integers(0, len(ODD)))])
    algo = int(g.integers(0, 2))
    margin = int(g.integers(-3, 4))
    reset = bool(g.random() < 0.7)
    return xs, fmts, n_upd, H, hist, first, algo, margin, reset


@pytest.mark.parametrize("seed", range(8))
def test_random_step(orc, seed):
    xs, fmts, n_upd, H, hist, first, algo, margin, reset = make_case(seed)
    note("random step %d: %d tensors (%d elements), %d columns, history %d, algo %d, "
         "margin %d, reset %d" % (seed, len(xs), sum(x.size for x in xs), n_upd, H, algo,
                                  margin, reset))
    st = Step(xs, fmts, H, n_upd=n_upd, first_scale=first, hist=hist)
    for step in range(3):
        note("random step %d: step %d" % (seed, step))
        st.run(orc, algo=algo, margin=margin, reset=reset)
