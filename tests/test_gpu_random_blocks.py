"""A seeded sweep of random Swin-block shapes against the fp64 block oracle, through the C ABI
of include/swin_block.h: random grids (2-D and 3-D, ragged), head_dim 32/64/128, hidden widths
that are multiples of 64 (not only 4C), windows of the one-tile and the tiled kernels, one or two
chained blocks. Bars as in test_gpu_block.py (tests/bars.py): per-token outputs
|got - ref| <= 2e-2 + ulp_bf16(ref)/2; reduced gradients 2e-2 * max(1, |ref|_inf)."""
import numpy as np
import pytest

from tests.bars import reduced_excess, token_excess
from tests.gpu_util import log, run_block_chain
from tests.oracle_runner import block_chain_full
from workloads import BLOCK_BIAS_SCALE, make_block_extras, make_inputs
from workloads.configs import SwinConfig

pytestmark = pytest.mark.gpu

GRAD_KEYS = ("ln1_g", "ln1_b", "w_qkv", "b_qkv", "w_proj", "b_proj", "table", "ln2_g", "ln2_b", "w1", "b1", "w2",
             "b2")


def random_blocks(n=9, seed=23):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        hd = (32, 64, 128)[len(out) % 3]
        heads = int(rng.choice({32: [2, 4, 6], 64: [1, 2, 3], 128: [1, 2]}[hd]))
        C = hd * heads
        three_d = len(out) % 4 == 3
        D = int(rng.integers(2, 4)) if three_d else 1
        H, W = int(rng.integers(8, 40)), int(rng.integers(8, 48))
        wd = int(rng.integers(1, D + 1)) if three_d else 1
        wh, ww = int(rng.integers(4, min(H, 24) + 1)), int(rng.integers(4, min(W, 24) + 1))
        batch = int(rng.integers(1, 3))
        if batch * D * H * W > 2500:
            continue
        shift = tuple(int(rng.integers(0, w)) if g > w else 0 for g, w in zip((D, H, W), (wd, wh, ww)))
        shifts = ((0, 0, 0), shift) if rng.random() < 0.5 else (shift,)
        hidden = 64 * int(rng.integers(1, max(2, 4 * C // 64) + 1))
        name = "b%d_hd%d_C%d_h%d_g%dx%dx%d_w%dx%dx%d" % (len(out), hd, C, hidden, D, H, W, wd, wh, ww)
        cfg = SwinConfig(name=name, batch=batch, grid=(D, H, W), channels=C, heads=heads, window=(wd, wh, ww),
                         shifts=shifts, dtype="bf16", backward=True, periodic=int(rng.choice([0, 4, 6])),
                         description=name)
        out.append((cfg, hidden))
    return out


CASES = random_blocks()


@pytest.mark.parametrize("cfg,hidden", CASES, ids=lambda v: v.name if isinstance(v, SwinConfig) else str(v))
def test_random_block_vs_oracle(cfg, hidden):
    log("random block", cfg.name, "batch", cfg.batch, "shifts", cfg.shifts, "periodic", cfg.periodic)
    inp = make_inputs(cfg, bias_scale=BLOCK_BIAS_SCALE)
    extras = make_block_extras(cfg, hidden=hidden)
    got = run_block_chain(cfg, inp, extras)
    ref = block_chain_full(cfg, inp, extras)
    for key in ("y", "dx"):
        excess, err = token_excess(got[key], ref[key])
        log("  %s max-abs %.3e, worst excess over the bar %.3e" % (key, err, excess))
        assert excess <= 0, key
    for i, (gm, rm) in enumerate(zip(got["grads"], ref["grads"])):
        for k in GRAD_KEYS:
            ex, err = reduced_excess(gm[k], rm[k])
            assert ex <= 0, (cfg.name, i, k, err, ex)
