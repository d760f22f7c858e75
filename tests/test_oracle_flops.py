"""Pins of the oracle's work counters: allowed (query, key) pairs, module and block FLOPs.

Pair counts are worked out by hand below from each workload's window structure, not by
enumerating labels as the oracle does: a window whose tokens share one wrap label has n^2
allowed pairs; a window the shift mask splits has the sum of the squares of its label
classes. The FLOP totals are the hand-derived table of the measurement plan (per module
forward = 2 N C 3C + 2 N C C + 4 hd heads pairs; backward = 2 x forward), in GFLOP.
Sources: the window partition and row-major order (TERRA page, section IV-D; section V-A,
Eq. 4), the roll by half a window (BEAST page, "Model Architecture"), and the readings of
the ragged edge windows and the two-label mask on non-periodic axes.
"""
import pytest

from oracle import block_oracle as BO
from oracle import swin_oracle as O
from workloads import get_config


def _layout(cfg, shift):
    return O.window_layout(cfg.batch, cfg.grid, cfg.window, shift, cfg.periodic)


# Hand counts, per workload and module shift:
# tiny 32x64, w 8x8, s (4,4): 4 x 8 windows of 64; lat window 3 (rolled rows 24..31) splits at
#   local row 4 (rows with i' + 4 >= 32 carry label 1): 8 windows of 2 x 32 tokens.
#   24 * 64^2 + 8 * 2 * 32^2 = 114688.
# om4 2 x 180x360, w 6x12, s (3,6): 30 x 30 windows of 72 per batch; the last lat row splits
#   3/3 rows: 30 windows of 2 x 36.  2 * (870 * 72^2 + 30 * 2 * 36^2) = 9175680.
# ragged 181x361, w 8x16, s (4,8): lat windows 22 x 8 rows + 1 x 5 rows (rolled 176..180, label 1
#   from local row 1), lon (periodic) 22 x 16 + 1 x 9: 484 x 128, 22 x 72 (8 x 9), 22 x 80 split
#   1/4 rows into 16 + 64, one 5 x 9 corner split into 9 + 36.
#   484 * 128^2 + 22 * 72^2 + 22 * (16^2 + 64^2) + (9^2 + 36^2) = 8141025.
# highres 540x1080, w 12x12: W-MSA 45 x 90 windows of 144: 4050 * 144^2 = 83980800; SW-MSA
#   s (6,6): the last lat row of 90 windows splits 6/6 rows: 3960 * 144^2 + 90 * 2 * 72^2 = 83047680.
# levels3d 8x180x360, w 2x6x12, s (1,3,6): 4 x 30 x 30 windows of 144; the last level window
#   splits 1/1 levels, the last lat row 3/3 rows: 2610 unsplit, 870 + 90 split in two halves of
#   72, 30 split in four quarters of 36.
#   2610 * 144^2 + 960 * 2 * 72^2 + 30 * 4 * 36^2 = 64229760.
HAND_PAIRS = {
    "tiny": [24 * 64 ** 2 + 8 * 2 * 32 ** 2],
    "om4": [2 * (870 * 72 ** 2 + 30 * 2 * 36 ** 2)],
    "ragged": [484 * 128 ** 2 + 22 * 72 ** 2 + 22 * (16 ** 2 + 64 ** 2) + (9 ** 2 + 36 ** 2)],
    "highres": [4050 * 144 ** 2, 3960 * 144 ** 2 + 90 * 2 * 72 ** 2],
    "levels3d": [2610 * 144 ** 2 + 960 * 2 * 72 ** 2 + 30 * 4 * 36 ** 2],
}
HAND_MASK_SPLIT = {"tiny": 8, "om4": 60, "ragged": 23, "highres": 90, "levels3d": 990}

# (forward GFLOP of the whole pass, forward + backward GFLOP) from the measurement plan's table
PLAN_GFLOP = {"tiny": (0.096, None), "om4": (45.268, 135.80), "ragged": (42.594, 127.78),
              "highres": (2788.19, 8364.58), "levels3d": (202.21, 606.63)}


@pytest.mark.parametrize("name", list(HAND_PAIRS))
def test_allowed_pairs_match_hand_counts(name):
    cfg = get_config(name)
    for shift, want in zip(cfg.shifts, HAND_PAIRS[name]):
        assert O.allowed_pairs(_layout(cfg, shift)) == want


@pytest.mark.parametrize("name", list(HAND_MASK_SPLIT))
def test_mask_split_window_counts(name):
    cfg = get_config(name)
    lay = _layout(cfg, cfg.shifts[-1])
    split = sum(1 for w in lay.windows if len(set(lay.labels[w.tok_off:w.tok_off + w.n].tolist())) > 1)
    assert split == HAND_MASK_SPLIT[name]


@pytest.mark.parametrize("name", list(PLAN_GFLOP))
def test_module_flops_match_plan_table(name):
    cfg = get_config(name)
    fwd = fwd_bwd = 0
    for pairs in HAND_PAIRS[name]:
        f = O.module_flops(cfg.n_tokens, cfg.channels, cfg.heads, pairs)
        # the pieces, written out: QKV and proj GEMMs, the two attention products
        assert f["qkv"] == 2 * cfg.n_tokens * cfg.channels * 3 * cfg.channels
        assert f["proj"] == 2 * cfg.n_tokens * cfg.channels ** 2
        assert f["core"] == 4 * cfg.head_dim * cfg.heads * pairs
        assert f["bwd"] == 2 * f["fwd"] and f["fwd_bwd"] == 3 * f["fwd"]
        fwd += f["fwd"]
        fwd_bwd += f["fwd_bwd"]
    want_fwd, want_fb = PLAN_GFLOP[name]
    assert fwd / 1e9 == pytest.approx(want_fwd, abs=5e-3 if want_fwd < 1 else 0.006)
    if want_fb is not None:
        assert fwd_bwd / 1e9 == pytest.approx(want_fb, abs=0.006)


def test_block_flops_is_module_forward_plus_mlp():
    # one W-MSA block of the 540x1080 workload with hidden width 4C: attention forward
    # 1395.05 GFLOP (plan table) + two MLP products 2 * 2 N C 4C
    cfg = get_config("highres")
    n, c = cfg.n_tokens, cfg.channels
    got = BO.block_flops(n, c, 4 * c, cfg.heads, HAND_PAIRS["highres"][0])
    assert got / 1e9 == pytest.approx(1395.05 + 4 * n * c * 4 * c / 1e9, abs=0.006)
