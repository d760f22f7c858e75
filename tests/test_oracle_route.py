"""Pins of the token-route oracle (TERRA section IV-D routes, section V-A Eq. 4 ownership).

Checked against: the Eq. 4 ranges worked by hand (tests/golden/eq4_ranges.txt, including the
ten-windows-on-four-ranks example of section V-B), the properties Eq. 4 guarantees (every
window owned once, contiguous ranges, counts differing by at most one), a route worked by hand
on a 4x4 grid, and identities that hold for any correct route: pack -> exchange -> unpack
equals placing every token directly at its destination, the inverse route restores the
source tensors, and routing through the unshifted window layout equals routing straight to
the shifted one."""
import os

import numpy as np
import pytest

from oracle import route_oracle as RO
from oracle import swin_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "eq4_ranges.txt")


def _golden():
    rows = []
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if not line:
            continue
        mr, lo, counts = (f.split() for f in line.split("|"))
        rows.append((int(mr[0]), int(mr[1]), [int(v) for v in lo], [int(v) for v in counts]))
    return rows


def test_eq4_worked_examples():
    rows = _golden()
    assert rows and rows[0][:2] == (10, 4)
    for M, R, lo, counts in rows:
        L, Rr = RO.eq4_ranges(M, R)
        assert L == lo, (M, R)
        assert [b - a for a, b in zip(L, Rr)] == counts, (M, R)
    # the section V-B example: two ranks with three windows, two with two
    L, Rr = RO.eq4_ranges(10, 4)
    assert sorted(b - a for a, b in zip(L, Rr)) == [2, 2, 3, 3]


def test_eq4_properties():
    rng = np.random.default_rng(0)
    for _ in range(300):
        M, R = int(rng.integers(0, 500)), int(rng.integers(1, 40))
        L, Rr = RO.eq4_ranges(M, R)
        assert L[0] == 0 and Rr[-1] == M
        assert all(Rr[r] == L[r + 1] for r in range(R - 1))            # contiguous, in rank order
        c = [b - a for a, b in zip(L, Rr)]
        assert sum(c) == M and min(c) >= 0 and max(c) - min(c) <= 1      # each window once, balanced
        assert min(c) == M // R


def _check_bijection(lay, n_tok):
    assert lay.rank.size == n_tok and sum(lay.sizes) == n_tok
    for r in range(lay.ranks):
        offs = np.sort(lay.offset[lay.rank == r])
        assert np.array_equal(offs, np.arange(lay.sizes[r]))


def test_stripes_layout_hand_example():
    lay = RO.stripes_layout(1, (1, 5, 3), 2)   # rows [0, 2) and [2, 5)
    assert lay.sizes == [6, 9]
    assert list(lay.rank) == [0] * 6 + [1] * 9
    assert list(lay.offset) == list(range(6)) + list(range(9))
    lay2 = RO.stripes_layout(2, (2, 4, 3), 3)  # rows [0,1), [1,2), [2,4) of each (batch, level)
    _check_bijection(lay2, 2 * 2 * 4 * 3)
    # token (b=1, d=0, h=3, w=2): stripe 2 has 2 rows; offset ((1*2+0)*2 + 1)*3 + 2 = 17
    g = ((1 * 2 + 0) * 4 + 3) * 3 + 2
    assert lay2.rank[g] == 2 and lay2.offset[g] == 17


def test_windows_layout_is_eq4_slicing_of_the_window_major_tensor():
    rng = np.random.default_rng(1)
    for batch, grid, win, sh, per, R in [(1, (1, 20, 30), (1, 6, 8), (0, 3, 4), 4, 5),
                                         (2, (3, 9, 10), (2, 4, 4), (1, 2, 2), 0, 7),
                                         (1, (1, 13, 17), (1, 5, 5), (0, 0, 0), 4, 40)]:
        lay = O.window_layout(batch, grid, win, sh, per)
        x = rng.standard_normal((batch,) + grid + (3,))
        xw = O.gather(x, lay)
        rl = RO.windows_layout(batch, grid, win, sh, per, R)
        _check_bijection(rl, lay.perm.size)
        L, Rr = RO.eq4_ranges(len(lay.windows), R)
        starts = [w.tok_off for w in lay.windows] + [lay.perm.size]
        for r, local in enumerate(RO.distribute(x, rl)):
            assert np.array_equal(local, xw[starts[L[r]]:starts[Rr[r]]])


def test_route_hand_example():
    """4x4 grid, 2x2 windows, 2 stripes (rows 0-1, rows 2-3), 2 window ranks. Unshifted, rank 0
    owns windows 0 and 1 (rows 0-1): the DMP route is local. Shifted by (1, 1) with no periodic
    axis, rank 0's windows hold original rows 1 and 2, rank 1's rows 3 and 0: 4 tokens each way.
    Rank 0's window-major order is (1,1) (1,2) (2,1) (2,2) (1,3) (1,0) (2,3) (2,0), so stripe 0
    sends its row-1 tokens (local offsets 5, 6, 7, 4) to destination offsets 0, 1, 4, 5."""
    st = RO.stripes_layout(1, (1, 4, 4), 2)
    w0 = RO.windows_layout(1, (1, 4, 4), (1, 2, 2), (0, 0, 0), 0, 2)
    w1 = RO.windows_layout(1, (1, 4, 4), (1, 2, 2), (0, 1, 1), 0, 2)
    assert RO.route(st, w0).counts.tolist() == [[8, 0], [0, 8]]
    rt = RO.route(st, w1)
    assert rt.counts.tolist() == [[4, 4], [4, 4]]
    assert rt.send_src[0][:4].tolist() == [5, 6, 7, 4]
    assert rt.recv_dst[0][:4].tolist() == [0, 1, 4, 5]


CASES = [
    (1, (1, 24, 36), (1, 6, 6), (0, 3, 3), 4, 3, 4),      # lon periodic, P != R
    (1, (1, 25, 37), (1, 6, 8), (0, 3, 4), 4, 4, 5),      # ragged edge windows
    (2, (3, 10, 12), (2, 4, 4), (1, 2, 2), 0, 2, 6),      # batch 2, 3-D, nothing periodic
    (1, (1, 12, 12), (1, 6, 6), (0, 3, 3), 6, 3, 7),      # more window ranks than windows
    (1, (1, 18, 24), (1, 6, 6), (0, 3, 3), 4, 1, 1),      # one rank each side
]


@pytest.mark.parametrize("batch,grid,win,sh,per,P,R", CASES)
def test_loopback_routes(batch, grid, win, sh, per, P, R):
    rng = np.random.default_rng(2)
    x = rng.standard_normal((batch,) + grid + (5,))
    st = RO.stripes_layout(batch, grid, P)
    w0 = RO.windows_layout(batch, grid, win, (0, 0, 0), per, R)
    ws = RO.windows_layout(batch, grid, win, sh, per, R)
    xs = RO.distribute(x, st)
    # DMP route: stripes -> unshifted windows equals placing every token directly
    got0 = RO.apply_route(xs, st, w0)
    for a, b in zip(got0, RO.distribute(x, w0)):
        assert np.array_equal(a, b)
    # shift route: unshifted -> shifted windows, and the composition equals the direct route
    got1 = RO.apply_route(got0, w0, ws)
    for a, b, c in zip(got1, RO.distribute(x, ws), RO.apply_route(xs, st, ws)):
        assert np.array_equal(a, b) and np.array_equal(a, c)
    # the inverse routes (the backward) bring every token home
    back = RO.apply_route(RO.apply_route(got1, ws, w0), w0, st)
    for a, b in zip(back, xs):
        assert np.array_equal(a, b)
    # bookkeeping: counts sum to the layouts' sizes; segments are in destination-offset order
    rt = RO.route(st, ws)
    assert rt.counts.sum(axis=1).tolist() == st.sizes and rt.counts.sum(axis=0).tolist() == ws.sizes
    for r in range(R):
        pos = 0
        for p in range(P):
            seg = rt.recv_dst[r][pos:pos + rt.counts[p, r]]
            assert np.all(np.diff(seg) > 0)
            pos += rt.counts[p, r]


def test_shift_route_moves_only_boundary_tokens():
    """Section V-A: with contiguous row-major ownership, the shift route keeps interior windows
    local. At 8 ranks over 45 x 90 windows of 12 x 12 (the 540 x 1080 grid at reduced channel
    count), the tokens that change rank are a small fraction of the grid: they come from the
    window rows next to a rank's range boundaries."""
    grid, win = (1, 540, 1080), (1, 12, 12)
    w0 = RO.windows_layout(1, grid, win, (0, 0, 0), 4, 8)
    w1 = RO.windows_layout(1, grid, win, (0, 6, 6), 4, 8)
    moved = int(np.sum(w0.rank != w1.rank))
    n = 540 * 1080
    # a shifted window row straddles two unshifted window rows and takes s_h = 6 latitude rows
    # from the lower one, so each of the 8 boundaries (7 between ranks, plus the wrap of the
    # first rows to the last shifted row) moves at most 6 full latitude rows plus one window
    # where the boundary falls inside a window row
    assert 0 < moved <= 8 * (6 * 1080 + 12 * 12), moved
    assert moved < 0.1 * n
