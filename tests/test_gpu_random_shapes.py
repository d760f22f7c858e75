"""A seeded sweep of random module shapes against the fp64 oracle, through the C ABI: 2-D and
3-D grids, ragged edges, head_dim 32/64/128, batch 1-2, every periodic combination of the lat
and lon axes, windows from 16 to over 1000 tokens (so both the one-tile and the tiled kernels,
tables held in LDS and in global memory), one or two chained modules; a second set with channels
256-1024 (the wide-tile QKV GEMM, whose output width 3C is a multiple of 256). Same bars as the other
parity tests (tests/bars.py): per-token outputs 2e-2 + ulp_bf16(ref)/2, reduced gradients 2e-2 * max(1, |ref|_inf)."""
import numpy as np
import pytest

from tests.bars import reduced_excess, token_excess
from tests.gpu_util import log, run_chain
from tests.oracle_runner import chain_full
from workloads import make_inputs
from workloads.configs import SwinConfig

pytestmark = pytest.mark.gpu



def random_configs(n=16, seed=11):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        hd = int(rng.choice([32, 64, 128]))
        heads = int(rng.choice({32: [2, 4], 64: [1, 2, 3], 128: [1, 2]}[hd]))
        three_d = rng.random() < 0.3
        D = int(rng.integers(2, 5)) if three_d else 1
        large = rng.random() < 0.35  # windows of 33-60 x 33-72: tables over 4096 bins, many over 8192
        if large:
            three_d = False
            D = 1
            H, W = int(rng.integers(33, 61)), int(rng.integers(33, 73))
        else:
            H, W = int(rng.integers(8, 64)), int(rng.integers(8, 72))
        wd = int(rng.integers(1, D + 1)) if three_d else 1
        if large:
            wh, ww = int(rng.integers(33, H + 1)), int(rng.integers(33, W + 1))
        else:
            wh, ww = int(rng.integers(4, min(H, 40) + 1)), int(rng.integers(4, min(W, 48) + 1))
        batch = int(rng.integers(1, 3))
        n_tok = batch * D * H * W
        if n_tok > 8000 or wd * wh * ww > 4400:
            continue
        shift = tuple(int(rng.integers(0, w)) if g > w else 0 for g, w in zip((D, H, W), (wd, wh, ww)))
        shifts = ((0, 0, 0), shift) if rng.random() < 0.4 else (shift,)
        periodic = int(rng.choice([0, 2, 4, 6]))
        name = "r%d_hd%d_g%dx%dx%d_w%dx%dx%d" % (len(out), hd, D, H, W, wd, wh, ww)
        out.append(SwinConfig(name=name, batch=batch, grid=(D, H, W), channels=hd * heads, heads=heads,
                              window=(wd, wh, ww), shifts=shifts, dtype="bf16", backward=True, periodic=periodic,
                              description=name))
    return out


def wide_configs(n=8, seed=5):
    """Channels 256-1024 with head_dim 32/64/128 (up to 32 heads), windows up to 16 x 16, grids of a
    few hundred to ~2400 tokens."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        hd = int(rng.choice([32, 64, 128]))
        C = int(rng.choice([256, 512, 768, 1024]))
        three_d = rng.random() < 0.25
        D = int(rng.integers(2, 4)) if three_d else 1
        H, W = int(rng.integers(6, 40)), int(rng.integers(6, 48))
        wd = int(rng.integers(1, D + 1))
        wh, ww = int(rng.integers(3, min(H, 16) + 1)), int(rng.integers(3, min(W, 16) + 1))
        batch = int(rng.integers(1, 3))
        n_tok = batch * D * H * W
        if n_tok > 3000 or n_tok * C > 1_500_000:
            continue
        shift = tuple(int(rng.integers(0, w)) if g > w else 0 for g, w in zip((D, H, W), (wd, wh, ww)))
        shifts = ((0, 0, 0), shift) if rng.random() < 0.3 else (shift,)
        periodic = int(rng.choice([0, 2, 4, 6]))
        name = "w%d_C%d_hd%d_g%dx%dx%d_w%dx%dx%d" % (len(out), C, hd, D, H, W, wd, wh, ww)
        out.append(SwinConfig(name=name, batch=batch, grid=(D, H, W), channels=C, heads=C // hd, window=(wd, wh, ww),
                              shifts=shifts, dtype="bf16", backward=True, periodic=periodic, description=name))
    return out


CASES = random_configs() + wide_configs()


@pytest.mark.parametrize("c", CASES, ids=lambda c: c.name)
def test_random_shape_vs_oracle(c):
    log("random shape", c.name, "batch", c.batch, "heads", c.heads, "shifts", c.shifts, "periodic", c.periodic)
    inp = make_inputs(c)
    got = run_chain(c, inp)
    ref = chain_full(c, inp)
    (exy, ey), (exd, edx) = token_excess(got["y"], ref["y"]), token_excess(got["dx"], ref["dx"])
    log("  y max-abs %.3e  dx max-abs %.3e (worst excess over the bar %.3e, %.3e)" % (ey, edx, exy, exd))
    assert exy <= 0.0 and exd <= 0.0
    for i, (gm, rm) in enumerate(zip(got["grads"], ref["grads"])):
        for k in ("w_qkv", "b_qkv", "w_proj", "b_proj", "table"):
            ex, err = reduced_excess(gm[k], rm[k], rm.get("abs", {}).get(k))
            assert ex <= 0.0, (c.name, i, k, err, ex)
