"""Host check of the in-place history walk the one-launch step's update uses.  The roll
runs in one block of 256 threads (thread t owns column t mod n and rows g, g + G, ... of
each chunk with G = 256 // n row groups; chunks of G * 32 destination rows from the top;
every load of a chunk before any of its stores) and leaves the column maxima in row 0;
the block that finishes last then selects from row 0 and the new amax and writes the
amax into row 0.  Replays that schedule on a numpy array for many (n, H) and checks that
the result is the roll (row h-1 moves to row h, the new amax enters row 0), that no
element is read after it was overwritten, and that row 0 held the maxima over the old
rows 0 .. H-2 in between.  No GPU and no oracle: this checks the schedule's indexing
only."""
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
    hist[0, :] = colmax  # the rolling block's last stores
    row0 = hist[0].copy()  # what the finishing block reads
    hist[0, :] = amax  # the finishing block
    return hist, row0


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


# ---------------------------------------------------------------------------------
# The batched update kernel (amax_and_scale_update_kernel): blocks of BLOCK_U threads own
# COLS_U adjacent columns and all rows; tpr lanes (a power of two) cover a row of the
# group with W columns each; rows per pass BLOCK_U // tpr; ROWS_U rows per thread per
# chunk; chunks from the top; a lane without a row or column accesses offset 2^31 (out
# of both buffer ranges: the load descriptor covers rows [0, H-1), the store one [0, H)).
BLOCK_U, COLS_U, ROWS_U, OUT = 1024, 32, 8, 0x80000000


def tpr_of(n, W):
    lanes = -(-min(n, COLS_U) // W)
    t = 1
    while t < lanes:
        t *= 2
    return t


def update_walk(hist: np.ndarray, amax: np.ndarray, W: int):
    H, n = hist.shape
    flat = hist.reshape(-1)
    written = np.zeros(flat.size, bool)
    tpr = tpr_of(n, W)
    rpp = BLOCK_U // tpr
    chunk = rpp * ROWS_U
    ld_end, st_end = (H - 1) * n * 4, H * n * 4
    colmax = np.zeros(n, hist.dtype)
    groups = -(-n // COLS_U)
    tid = np.arange(BLOCK_U)
    lc, rr = tid & (tpr - 1), tid // tpr
    for g in range(groups):
        c = g * COLS_U + lc * W
        col_ok = c < n
        d_hi = H
        while True:
            d_lo = max(d_hi - chunk, 1)
            loads = []
            for k in range(ROWS_U):
                d = d_lo + rr + k * rpp
                ok = col_ok & (d < d_hi)
                off = np.where(ok, (d - 1) * n * 4 + c * 4, OUT)
                assert (off[ok] + 4 * W <= ld_end).all() and (off[~ok] >= ld_end).all()
                for j in range(W):
                    e = off[ok] // 4 + j
                    assert not written[e].any(), "element read after it was overwritten"
                    assert ((e % n) >= g * COLS_U).all() and ((e % n) < min(n, (g + 1) * COLS_U)).all()
                    v = flat[e]
                    np.maximum.at(colmax, e % n, v)
                    loads.append((e + n, v))
                so = off + n * 4  # store offsets: one row down
                assert (so[ok] + 4 * W <= st_end).all() and (so[~ok] >= st_end).all()
            for e, v in loads:  # after the chunk's barrier
                assert not written[e].any()
                flat[e] = v
                written[e] = True
            if d_lo == 1:
                break
            d_hi = d_lo
    hist[0, :] = amax
    return hist, colmax


@pytest.mark.parametrize("W", [4, 1])
@pytest.mark.parametrize("n", [1, 3, 4, 5, 8, 12, 31, 32, 36, 1151, 1152, 1156])
@pytest.mark.parametrize("H", [1, 2, 16, 1024, 1025, 1026, 2049])
def test_update_kernel_walk_is_the_roll(n, H, W):
    if W == 4 and n % 4:
        pytest.skip("16-byte lanes need n % 4 == 0")
    if n * H > 1300000:
        pytest.skip("large shapes: covered by the smaller column counts")
    g = np.random.Generator(np.random.PCG64(1000 * n + H + W))
    old = g.integers(1, 1 << 30, (H, n)).astype(np.int64)
    amax = g.integers(1, 1 << 30, n).astype(np.int64)
    got, colmax = update_walk(old.copy(), amax, W)
    want = np.empty_like(old)
    want[0] = amax
    want[1:] = old[:-1]
    assert np.array_equal(got, want)
    expect_max = old[:-1].max(axis=0) if H > 1 else np.zeros(n, np.int64)
    assert np.array_equal(colmax, expect_max)
