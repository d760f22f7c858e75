"""Seeded fuzz of the library's host-side descriptor checks and window layout (no GPU): random
descriptors, valid and not (zero or negative extents, windows past the grid, shifts out of range,
bad dtype/periodic/scale values, grids past 2^31 tokens), through swin_attn_host_stats and
swin_attn_host_index_map. Every call must return a status (never crash); valid small descriptors
must give a permutation of the tokens whose windows match the statistics. Also run by
tests/test_host_sanitizer.py against the ASan/UBSan build of the host code."""
import ctypes

import numpy as np
import pytest


@pytest.fixture(scope="module")
def N():
    from shifted_window_attention_amd import native
    return native


def _random_desc(N, rng):
    """A valid descriptor, then (half the time) one or two fields set to an invalid value."""
    d = N.SwinAttnDesc()
    nd = int(rng.choice([2, 3]))
    d.ndim = nd
    d.dtype = int(rng.choice([0, 1]))
    d.batch = int(rng.integers(1, 3))
    grid = [1 if nd == 2 else int(rng.integers(1, 6))] + [int(rng.integers(1, 14)) for _ in range(2)]
    for a in range(3):
        d.grid[a] = grid[a]
        d.window[a] = 1 if (nd == 2 and a == 0) else int(rng.integers(1, grid[a] + 1))
        d.shift[a] = 0 if (nd == 2 and a == 0) else int(rng.integers(0, d.window[a]))
    d.heads = int(rng.choice([1, 2, 4]))
    d.channels = d.heads * int(rng.choice([8, 32, 64]))
    d.periodic = int(rng.choice([0, 2, 4, 6]))
    d.scale = float(rng.choice([0.0, 0.125]))
    if rng.random() < 0.5:
        for _ in range(int(rng.integers(1, 3))):
            f = int(rng.integers(0, 12))
            a = int(rng.integers(0, 3))
            if f == 0:
                d.ndim = int(rng.choice([0, 1, 4, -2]))
            elif f == 1:
                d.dtype = int(rng.choice([2, 7, -1]))
            elif f == 2:
                d.batch = int(rng.choice([0, -1]))
            elif f == 3:
                d.grid[a] = int(rng.choice([0, -5]))
            elif f == 4:
                d.window[a] = int(rng.choice([0, -1, d.grid[a] + 1]))
            elif f == 5:
                d.shift[a] = int(rng.choice([-1, d.window[a], d.window[a] + 3]))
            elif f == 6:
                d.heads = int(rng.choice([0, -2]))
            elif f == 7:
                d.channels = d.heads * 32 + 1 if d.heads > 1 else 0
            elif f == 8:
                d.periodic = int(rng.choice([8, 255, 1 << 31]))
            elif f == 9:
                d.scale = float(rng.choice([-1.0, float("nan"), float("inf")]))
            elif f == 10:   # 2^31 tokens or more
                d.grid[1] = d.grid[2] = 1 << 16
                d.window[1] = d.window[2] = 1
                d.shift[1] = d.shift[2] = 0
            else:           # a 2-D descriptor with a level extent
                d.ndim = 2
                d.grid[0] = 2
    return d


def test_descriptor_fuzz_returns_statuses(N):
    rng = np.random.default_rng(2024)
    counts = {}
    for _ in range(3000):
        d = _random_desc(N, rng)
        st = N.SwinAttnStats()
        s = N.lib.swin_attn_host_stats(ctypes.byref(d), ctypes.byref(st))
        assert s in (0, 1, 2), s
        counts[s] = counts.get(s, 0) + 1
        if s != 0:
            assert N.lib.swin_attn_last_error()
            continue
        n_tok = d.batch * d.grid[0] * d.grid[1] * d.grid[2]
        if n_tok > 4096:
            continue
        assert st.n_tokens == n_tok
        m, lab = N.swin_attn_host_index_map(d)
        assert np.array_equal(np.sort(m), np.arange(n_tok))   # every token exactly once
        assert lab.shape == (n_tok,)
        assert st.max_tokens <= d.window[0] * d.window[1] * d.window[2]
    # the fuzz reaches both outcomes
    assert counts.get(0, 0) > 50 and counts.get(1, 0) > 50, counts
