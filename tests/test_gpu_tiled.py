"""Parity of the tiled attention path (windows over 256 tokens, head_dim 64 and 128, bias
tables over 2048 bins) with the fp64 oracle, through the C ABI. Same bars as the one-tile
path (tests/bars.py): per-token outputs 2e-2 + ulp_bf16(ref)/2, reduced gradients 2e-2 * max(1, |ref|_inf)."""
import numpy as np
import pytest

from tests.bars import reduced_excess, token_excess
from tests.gpu_util import log, run_chain
from tests.oracle_runner import chain_full
from workloads import make_inputs
from workloads.configs import SwinConfig

pytestmark = pytest.mark.gpu



@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from shifted_window_attention_amd import native  # noqa: F401  (raises if the library is missing)


def cfg(name, grid, C, heads, window, shifts, periodic=4, batch=1):
    return SwinConfig(name=name, batch=batch, grid=grid, channels=C, heads=heads, window=window, shifts=shifts,
                      dtype="bf16", backward=True, periodic=periodic, description=name)


FWD_CASES = [
    # 768-token windows (24 x 32), W-MSA then SW-MSA, lon periodic
    cfg("w24x32", (1, 48, 96), 128, 4, (1, 24, 32), ((0, 0, 0), (0, 12, 16))),
    # ragged edges: 50 = 2*24 + 2 rows, 100 = 3*32 + 4 columns
    cfg("ragged24x32", (1, 50, 100), 128, 4, (1, 24, 32), ((0, 12, 16),)),
    # 3-D windows of 2 x 16 x 16 = 512 tokens, masked on level and lat
    cfg("levels_2x16x16", (4, 24, 48), 64, 2, (2, 16, 16), ((1, 8, 8),)),
    # a 32 x 32 window: 1024 tokens, 63 x 63 = 3969 bias bins
    cfg("w32", (1, 64, 96), 64, 2, (1, 32, 32), ((0, 16, 16),)),
    # global attention over 2400 tokens (window = grid), 79 x 119 bins
    cfg("global2400", (1, 40, 60), 64, 2, (1, 40, 60), ((0, 0, 0),), periodic=0),
    # head_dim 64 with 12 x 12 windows
    cfg("hd64", (1, 36, 48), 256, 4, (1, 12, 12), ((0, 0, 0), (0, 6, 6))),
    # head_dim 128 with 8 x 8 windows (TERRA Table V: w = 8, head_dim 128)
    cfg("hd128", (1, 32, 48), 512, 4, (1, 8, 8), ((0, 4, 4),)),
    # head_dim 128 and 576-token windows
    cfg("hd128_w24", (1, 48, 48), 256, 2, (1, 24, 24), ((0, 12, 12),)),
    # head_dim 128, ragged 16 x 16 windows: 40 = 2*16 + 8 rows, 52 = 3*16 + 4 columns (windows of 256, 128,
    # 64 and 32 tokens, so some end inside a 64-token block)
    cfg("hd128_ragged", (1, 40, 52), 256, 2, (1, 16, 16), ((0, 8, 8),)),
    # head_dim 64, ragged 12 x 20 windows (240, 80, 72 and 24 tokens)
    cfg("hd64_ragged", (1, 30, 44), 128, 2, (1, 12, 20), ((0, 6, 10),)),
    # 40 x 40 windows: 79 x 79 = 6241 bins, over the 4096 an LDS table holds (global-table kernels)
    cfg("w40_table6241", (1, 80, 80), 128, 2, (1, 40, 40), ((0, 20, 20),)),
    # global attention at head_dim 128 with the table in global memory (9401 bins)
    cfg("global2400_hd128", (1, 40, 60), 256, 2, (1, 40, 60), ((0, 0, 0),), periodic=0),
]


def _maxabs(a, b):
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b))))


def _check_grads(got, ref, label):
    for i, (gm, rm) in enumerate(zip(got, ref)):
        for k in ("w_qkv", "b_qkv", "w_proj", "b_proj", "table"):
            ex, err = reduced_excess(gm[k], rm[k], rm.get("abs", {}).get(k))
            log("  %s module %d d%s max-abs %.3e, worst excess over the bar %.3e" % (label, i, k, err, ex))
            assert ex <= 0.0, (label, i, k, err, ex)


# every forward case (the global ones have 9401 bins: dT through global atomics)
BWD_CASES = FWD_CASES + [
    # 256-token windows with head_dim 32 (over the one-tile backward's 160 tokens)
    cfg("w16x16", (1, 32, 48), 128, 4, (1, 16, 16), ((0, 0, 0), (0, 8, 8))),
    # 3-D windows with 4 levels: 4 x 12 x 12 = 576 tokens, 7 x 23 x 23 = 3703 bins, batch 2
    cfg("levels_4x12x12", (4, 24, 24), 128, 2, (4, 12, 12), ((2, 6, 6),), batch=2),
    # 60 x 90 windows (5400 tokens, the size of BEAST's smaller windows): 119 x 179 = 21301 bins
    cfg("w60x90_table21301", (1, 60, 180), 128, 2, (1, 60, 90), ((0, 0, 45),)),
]


@pytest.mark.parametrize("c", BWD_CASES, ids=lambda c: c.name)
def test_tiled_backward_vs_oracle(c):
    log("tiled fwd+bwd", c.name, c.grid, "window", c.window, "C", c.channels, "heads", c.heads)
    inp = make_inputs(c)
    got = run_chain(c, inp)
    ref = chain_full(c, inp)
    (exy, ey), (exd, edx) = token_excess(got["y"], ref["y"]), token_excess(got["dx"], ref["dx"])
    log("  y max-abs %.3e  dx max-abs %.3e (worst excess over the bar %.3e, %.3e)" % (ey, edx, exy, exd))
    assert exy <= 0.0 and exd <= 0.0
    _check_grads(got["grads"], ref["grads"], c.name)
    from shifted_window_attention_amd import native as N
    for m in got["mods"]:
        assert N.swin_attn_plan_flags(m.plan.handle) == 0   # no dT term left the fixed-point range


def test_tiled_backward_is_deterministic():
    import torch
    c = BWD_CASES[0]
    inp = make_inputs(c)
    got = run_chain(c, inp)
    m = got["mods"][-1]
    x, dy = got["xs"][-2], torch.ones_like(got["xs"][-1])
    m.fwd(x)
    dx1, g1 = m.bwd(dy, x)
    dx2, g2 = m.bwd(dy, x)
    torch.cuda.synchronize()
    assert torch.equal(dx1.view(torch.int16), dx2.view(torch.int16))
    for k in g1:
        assert torch.equal(g1[k], g2[k]), k


@pytest.mark.parametrize("c", FWD_CASES, ids=lambda c: c.name)
def test_tiled_forward_vs_oracle(c):
    log("tiled forward", c.name, c.grid, "window", c.window, "C", c.channels, "heads", c.heads)
    inp = make_inputs(c)
    got = run_chain(c, inp, with_bwd=False)
    ref = chain_full(c, inp, with_bwd=False)
    ex, err = token_excess(got["y"], ref["y"])
    log("  y max-abs %.3e (worst excess over the bar %.3e)" % (err, ex))
    assert ex <= 0.0


def test_tiled_dT_saturation_is_flagged():
    """A dS term of magnitude 2^11 or more does not fit the fixed-point dT accumulator: the call
    writes NaN over dbias_table and raises SWIN_FLAG_DT_SATURATED in the plan's sticky flags,
    which swin_attn_plan_flags reads and clears; the other gradients are still computed, and a
    later call in range gives the in-range result again, bit for bit."""
    import torch
    from shifted_window_attention_amd import native as N
    c = BWD_CASES[-3]          # w16x16: 256-token windows, tiled backward, table in LDS
    inp = make_inputs(c)
    got = run_chain(c, inp)
    m = got["mods"][-1]
    x = got["xs"][-2]
    dy = torch.randn(x.shape, generator=torch.Generator().manual_seed(5)).to(torch.bfloat16).cuda()
    assert N.swin_attn_plan_flags(m.plan.handle, clear=True) == 0
    dx1, g1 = m.bwd(dy, x)
    assert N.swin_attn_plan_flags(m.plan.handle) == 0
    assert bool(torch.isfinite(g1["table"]).all())
    log("  in range: max |dT| %.3e" % float(g1["table"].abs().max()))
    big = dy * (2.0 ** 20)     # dS ~ P (dP - D) grows with dy: far beyond 2^11
    dx2, g2 = m.bwd(big, x)
    flags = N.swin_attn_plan_flags(m.plan.handle)
    log("  saturating call: flags %#x" % flags)
    assert flags & N.SWIN_FLAG_DT_SATURATED
    assert bool(torch.isnan(g2["table"]).all())
    for k in ("w_qkv", "b_qkv", "w_proj", "b_proj"):
        assert bool(torch.isfinite(g2[k]).all()), k
    assert bool(torch.isfinite(dx2.float()).all())
    # the flag is sticky until cleared
    dx3, g3 = m.bwd(dy, x)
    assert N.swin_attn_plan_flags(m.plan.handle, clear=True) & N.SWIN_FLAG_DT_SATURATED
    assert N.swin_attn_plan_flags(m.plan.handle) == 0
    assert torch.equal(g3["table"], g1["table"])
    assert torch.equal(dx3.view(torch.int16), dx1.view(torch.int16))
