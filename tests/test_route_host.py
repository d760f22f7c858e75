"""The library's host route planner (swin_route_host_tables) against the route oracle,
bit-exact, plus the layout validation errors. No GPU needed."""
import ctypes

import numpy as np
import pytest

from oracle import route_oracle as RO


@pytest.fixture(scope="module")
def N():
    from shifted_window_attention_amd import native
    return native


def _grid(N, batch, grid, win, per, C=64, dtype=None):
    return N.make_desc(batch, grid, C, 1, win, (0, 0, 0), per, N.SWIN_BF16 if dtype is None else dtype)


def _oracle_layout(batch, grid, win, per, kind, ranks, shift):
    if kind == 0:
        return RO.stripes_layout(batch, grid, ranks)
    return RO.windows_layout(batch, grid, win, shift, per, ranks)


CASES = [
    # batch, grid, window, periodic, (kind, ranks, shift) src, dst
    (1, (1, 24, 36), (1, 6, 6), 4, (0, 3, (0, 0, 0)), (1, 4, (0, 0, 0))),      # DMP route
    (1, (1, 24, 36), (1, 6, 6), 4, (1, 4, (0, 0, 0)), (1, 4, (0, 3, 3))),      # shift route
    (1, (1, 25, 37), (1, 6, 8), 4, (0, 4, (0, 0, 0)), (1, 5, (0, 3, 4))),      # ragged, straight to shifted
    (2, (3, 10, 12), (2, 4, 4), 0, (1, 6, (1, 2, 2)), (0, 2, (0, 0, 0))),      # inverse direction, 3-D, batch 2
    (1, (1, 12, 12), (1, 6, 6), 6, (0, 3, (0, 0, 0)), (1, 7, (0, 3, 3))),      # ranks without windows
    (1, (1, 45, 90), (1, 12, 12), 4, (1, 8, (0, 0, 0)), (1, 8, (0, 6, 6))),    # 8 ranks, 12x12 windows
]


@pytest.mark.parametrize("batch,grid,win,per,src,dst", CASES)
def test_host_tables_bit_exact(N, batch, grid, win, per, src, dst):
    g = _grid(N, batch, grid, win, per)
    ls, ld = N.make_rank_layout(*src), N.make_rank_layout(*dst)
    counts, send, recv = N.swin_route_host_tables(g, ls, ld)
    rt = RO.route(_oracle_layout(batch, grid, win, per, *src), _oracle_layout(batch, grid, win, per, *dst))
    assert np.array_equal(counts, rt.counts)
    assert np.array_equal(send, np.concatenate(rt.send_src))
    assert np.array_equal(recv, np.concatenate(rt.recv_dst))


def test_route_errors(N):
    g = _grid(N, 1, (1, 24, 36), (1, 6, 6), 4)
    ok = N.make_rank_layout(1, 4)
    bad = [N.make_rank_layout(0, 0),                  # no ranks
           N.make_rank_layout(0, 25),                 # more stripes than latitude rows
           N.make_rank_layout(0, 2, (0, 1, 0)),       # a stripe layout with a shift
           N.make_rank_layout(1, 2, (0, 6, 0)),       # shift >= window
           N.make_rank_layout(7, 2)]                  # unknown kind
    for lay in bad:
        for s, d in ((lay, ok), (ok, lay)):
            st = N.lib.swin_route_host_tables(ctypes.byref(g), ctypes.byref(s), ctypes.byref(d), None, None, None)
            assert st == 1, (lay.kind, lay.ranks, list(lay.shift))
    h = ctypes.c_void_p()
    assert N.lib.swin_route_plan_create(None, ctypes.byref(ok), ctypes.byref(ok), ctypes.byref(h)) == 1
    assert not h.value
