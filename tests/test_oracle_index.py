"""Pins of the oracle's index maps (roll, partition, wrap labels, reverse).

Checked against: hand-derived per-axis examples and window statistics
(tests/golden), the closed-form per-token coordinate formula, the
permutation property and the roll/un-roll identity."""
import os

import numpy as np
import pytest

from oracle import swin_oracle as O
from workloads import get_config
from workloads.configs import ORDER

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _layout(cfg, module=0):
    return O.window_layout(cfg.batch, cfg.grid, cfg.window, cfg.shifts[module], cfg.periodic)


def _parse_axis_rolls():
    cases, cur = [], None
    for line in open(os.path.join(GOLDEN, "axis_rolls.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        if line.startswith("case"):
            N, w, s, per = map(int, line.split()[1:])
            cur = {"N": N, "w": w, "s": s, "periodic": per, "wins": {}}
            cases.append(cur)
        else:
            head, rest = line.split(":")
            k = int(head.split()[1])
            idx, lab = rest.split("|")
            cur["wins"][k] = (list(map(int, idx.split())), list(map(int, lab.split())))
    return cases


@pytest.mark.parametrize("case", _parse_axis_rolls(), ids=lambda c: "N{N}w{w}s{s}p{periodic}".format(**c))
def test_hand_worked_axis(case):
    # embed the 1-D case as the lon axis (bit 2) of a 1 x 1 x N grid
    lay = O.window_layout(1, (1, 1, case["N"]), (1, 1, case["w"]), (0, 0, case["s"]), case["periodic"] << 2)
    for k, (idx, lab) in case["wins"].items():
        win = lay.windows[k]
        got = lay.perm[win.tok_off:win.tok_off + win.n]
        got_lab = (lay.labels[win.tok_off:win.tok_off + win.n] >> 2) & 1
        assert got.tolist() == idx
        assert got_lab.tolist() == lab


def _parse_counts():
    out = {}
    for line in open(os.path.join(GOLDEN, "window_counts.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        name, nwin, groups, split = (f.strip() for f in line.split("|"))
        g = {}
        for item in groups.split():
            c, t = item.split("x")
            g[int(t)] = int(c)
        out[name] = (int(nwin), g, int(split))
    return out


COUNT_CASES = [("tiny", 0, "tiny"), ("om4", 0, "om4"), ("ragged", 0, "ragged"), ("highres", 0, "highres0"),
               ("highres", 1, "highres1"), ("levels3d", 0, "levels3d")]


@pytest.mark.parametrize("name,module,key", COUNT_CASES)
def test_window_counts(name, module, key):
    nwin, groups, nsplit = _parse_counts()[key]
    lay = _layout(get_config(name), module)
    assert len(lay.windows) == nwin
    sizes = {}
    split = 0
    for w in lay.windows:
        sizes[w.n] = sizes.get(w.n, 0) + 1
        split += len(np.unique(lay.labels[w.tok_off:w.tok_off + w.n])) > 1
    assert sizes == groups
    assert split == nsplit


@pytest.mark.parametrize("name", ORDER)
def test_perm_is_permutation(name):
    cfg = get_config(name)
    for m in range(cfg.modules):
        lay = _layout(cfg, m)
        assert lay.n_tokens == cfg.n_tokens
        assert np.array_equal(np.sort(lay.perm), np.arange(cfg.n_tokens))


def _closed_form_slot(cfg, shift, t):
    """Window-major slot of original token t from the per-token formula (no roll, no slicing)."""
    B = cfg.batch
    D, H, W = cfg.grid
    w = cfg.window
    b, rem = divmod(t, D * H * W)
    d, rem = divmod(rem, H * W)
    h, x = divmod(rem, W)
    r = [(d - shift[0]) % D, (h - shift[1]) % H, (x - shift[2]) % W]
    k = [r[a] // w[a] for a in range(3)]
    ell = [r[a] % w[a] for a in range(3)]
    nk = [-(-N // wa) for N, wa in zip((D, H, W), w)]
    ext = [min(w[a], (D, H, W)[a] - k[a] * w[a]) for a in range(3)]

    def size_of(kk):  # tokens in window kk
        n = 1
        for a in range(3):
            n *= min(w[a], (D, H, W)[a] - kk[a] * w[a])
        return n
    # tokens before this window: full batches, then windows earlier in row-major order
    off = b * D * H * W
    for kd in range(nk[0]):
        for kh in range(nk[1]):
            for kw in range(nk[2]):
                if (kd, kh, kw) == tuple(k):
                    return off + (ell[0] * ext[1] + ell[1]) * ext[2] + ell[2]
                off += size_of((kd, kh, kw))
    raise AssertionError


@pytest.mark.parametrize("name", ORDER)
def test_closed_form_token_formula(name):
    cfg = get_config(name)
    rng = np.random.default_rng(1)
    for m in range(cfg.modules):
        lay = _layout(cfg, m)
        inv = np.empty_like(lay.perm)
        inv[lay.perm] = np.arange(lay.n_tokens)
        sample = np.concatenate([rng.integers(0, cfg.n_tokens, 40), [0, cfg.n_tokens - 1]])
        for t in sample:
            assert inv[t] == _closed_form_slot(cfg, cfg.shifts[m], int(t))


@pytest.mark.parametrize("name", ["tiny", "ragged", "levels3d"])
def test_roll_unroll_identity(name):
    cfg = get_config(name)
    lay = _layout(cfg)
    D, H, W = cfg.grid
    x = np.random.default_rng(2).standard_normal((cfg.batch, D, H, W, 3))
    assert np.array_equal(O.roll_unroll_grid(x, lay), x)
    assert np.array_equal(O.scatter(O.gather(x, lay), lay), x)


def test_labels_definition_3d():
    # level axis (bit 0) and lat (bit 1) masked, lon (bit 2) periodic: a token's label bits are set
    # exactly when its rolled index lies in the last s entries of a non-periodic axis
    cfg = get_config("levels3d")
    lay = _layout(cfg)
    D, H, W = cfg.grid
    s = cfg.shifts[0]
    for slot in [0, 17, 5000, 517000, lay.n_tokens - 1]:
        t = int(lay.perm[slot])
        d, rem = divmod(t, H * W)
        h, x = divmod(rem, W)
        rd, rh = (d - s[0]) % D, (h - s[1]) % H
        want = int(rd >= D - s[0]) | (int(rh >= H - s[1]) << 1)
        assert lay.labels[slot] == want


def test_rel_bins_worked():
    # 8x8 window, table 15x15: query (0,0) against key (7,7) -> bin (0,0); reverse -> bin (14,14)
    q = np.array([[0, 0, 0]])
    k = np.array([[0, 7, 7]])
    assert O.rel_bins(q, k, (1, 8, 8))[0, 0] == 0
    assert O.rel_bins(k, q, (1, 8, 8))[0, 0] == 14 * 15 + 14
    assert O.rel_bins(q, q, (1, 8, 8))[0, 0] == 7 * 15 + 7
