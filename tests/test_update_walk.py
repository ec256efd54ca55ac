"""Host check of the in-place history walk the one-launch step's update uses (one block
of 256 threads; thread t owns column t mod n and rows g, g + G, ... of each chunk with
G = 256 // n row groups; chunks of G * 32 destination rows from the top; every load of a
chunk before any of its stores; row 0 written last).  Replays that schedule on a numpy
array for many (n, H) and checks that the result is the roll (row h-1 moves to row h,
the new amax enters row 0), that no element is read after it was overwritten, and that
the per-column maxima taken from the loaded values are the maxima over the old rows
0 .. H-2.  No GPU and no oracle: this checks the schedule's indexing only."""
import numpy as np
import pytest

BLOCK, ROWS_PER_THREAD = 256, 32


def walk(hist: np.ndarray, amax: np.ndarray):
    H, n = hist.shape
    groups = BLOCK // n
    span = groups * ROWS_PER_THREAD
    written = np.zeros_like(hist, dtype=bool)
    colmax = np.zeros(n, hist.dtype)
    d_hi = H
    while d_hi > 1:
        d_lo = max(d_hi - span, 1)
        loads = []
        for tid in range(BLOCK):
            c, g = tid % n, tid // n
            if g >= groups:
                continue
            for k in range(ROWS_PER_THREAD):
                d = d_lo + g + k * groups
                if d < d_hi:
                    assert not written[d - 1, c], "row %d read after it was overwritten" % (d - 1)
                    v = hist[d - 1, c]
                    loads.append((d, c, v))
                    colmax[c] = max(colmax[c], v)
        for d, c, v in loads:  # after the chunk's barrier
            assert not written[d, c]
            hist[d, c] = v
            written[d, c] = True
        d_hi -= span
    hist[0, :] = amax
    return hist, colmax


@pytest.mark.parametrize("n", [1, 2, 3, 5, 7, 8, 64, 100, 255, 256])
@pytest.mark.parametrize("H", [1, 2, 16, 33, 257, 1024])
def test_walk_is_the_roll(n, H):
    if H * n > 65536:
        pytest.skip("beyond the one-launch limit")
    g = np.random.Generator(np.random.PCG64(1000 * n + H))
    old = g.integers(1, 1 << 30, (H, n)).astype(np.int64)
    amax = g.integers(1, 1 << 30, n).astype(np.int64)
    got, colmax = walk(old.copy(), amax)
    want = np.empty_like(old)
    want[0] = amax
    want[1:] = old[:-1]
    assert np.array_equal(got, want)
    expect_max = old[:-1].max(axis=0) if H > 1 else np.zeros(n, np.int64)
    assert np.array_equal(colmax, expect_max)
