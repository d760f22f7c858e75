"""Edge cases of the HIP path against the fp64 oracle (through the C ABI).

Degenerate and boundary shapes of the method: a window covering the whole grid (global
attention), one-token windows, the largest windows of the one-tile kernels (256 tokens
forward, 160 backward; 161-256-token windows go to the tiled backward), a bias table over the
backward's 8192 LDS bins, axes that are all or none periodic, ragged 3-D windows, and the
smallest channel count. Same bars as the other parity tests (tests/bars.py): 2e-2 + ulp_bf16(ref)/2
(bf16) / 1e-5 (fp32) on per-token outputs, 2e-2 * max(1, |ref|_inf) on reduced gradients."""
import ctypes

import numpy as np
import pytest

from tests.bars import TOL_BF16, TOL_F32, reduced_excess, token_excess
from tests.gpu_util import log, run_chain, to_dev, ModuleOnDevice
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


def _cfg(name, grid, window, shifts, channels=64, heads=2, batch=1, periodic=0x4, dtype="bf16", backward=True):
    return SwinConfig(name=name, batch=batch, grid=grid, channels=channels, heads=heads, window=window,
                      shifts=shifts, dtype=dtype, backward=backward, periodic=periodic, description=name)


def _maxabs(a, b):
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b)))) if np.size(a) else 0.0


def _check(cfg, with_bwd=True, inp=None):
    inp = make_inputs(cfg) if inp is None else inp
    got = run_chain(cfg, inp, with_bwd=with_bwd)
    ref = chain_full(cfg, inp, with_bwd=with_bwd)
    tol = TOL_BF16 if cfg.dtype == "bf16" else TOL_F32
    if cfg.dtype == "bf16":
        ex, ey = token_excess(got["y"], ref["y"])
        log("  %s y max-abs %.3e, worst excess over the bar %.3e" % (cfg.name, ey, ex))
        assert ex <= 0.0
    else:
        ey = _maxabs(got["y"], ref["y"])
        log("  %s y max-abs %.3e" % (cfg.name, ey))
        assert ey <= tol
    if not with_bwd:
        return
    ex, edx = token_excess(got["dx"], ref["dx"])
    log("  %s dx max-abs %.3e, worst excess over the bar %.3e" % (cfg.name, edx, ex))
    assert ex <= 0.0
    for i, (gm, rm) in enumerate(zip(got["grads"], ref["grads"])):
        for k in ("w_qkv", "b_qkv", "w_proj", "b_proj", "table"):
            ex, err = reduced_excess(gm[k], rm[k], rm.get("abs", {}).get(k))
            assert ex <= 0.0, (cfg.name, i, k, err, ex)


BF16_CASES = [
    # the window is the whole grid: global attention over 128 tokens, two batch items
    _cfg("global_8x16", (1, 8, 16), (1, 8, 16), ((0, 0, 0),), batch=2),
    # one-token windows: every token attends only to itself (o = v)
    _cfg("window_1x1", (1, 6, 10), (1, 1, 1), ((0, 0, 0),)),
    # 160-token windows, the largest the backward pass supports, W-MSA then SW-MSA
    _cfg("window_10x16", (1, 20, 48), (1, 10, 16), ((0, 0, 0), (0, 5, 8)), channels=128, heads=4),
    # no periodic axis: both axes masked, ragged edges
    _cfg("periodic_none", (1, 21, 29), (1, 6, 8), ((0, 3, 4),), periodic=0x0),
    # both spatial axes periodic: shifted windows wrap without masks
    _cfg("periodic_lat_lon", (1, 21, 29), (1, 6, 8), ((0, 3, 4),), periodic=0x6),
    # 3-D with a ragged level axis (3 levels, 2-level windows) shifted on every axis
    _cfg("levels_ragged", (3, 13, 26), (2, 6, 12), ((1, 3, 6),), channels=64, heads=2),
]


@pytest.mark.parametrize("cfg", BF16_CASES, ids=lambda c: c.name)
def test_bf16_edge_case_vs_oracle(cfg):
    log("bf16 edge case", cfg.name, cfg.grid, cfg.window, cfg.shifts)
    _check(cfg)


def test_bf16_256_token_windows_forward_and_backward():
    """256-token windows: one-tile forward, tiled backward (over 160 tokens)."""
    cfg = _cfg("window_16x16", (1, 32, 40), (1, 16, 16), ((0, 8, 8),))
    log("bf16 256-token windows", cfg.grid, cfg.window)
    _check(cfg)


def test_bf16_backward_with_table_over_8192_bins():
    """Global attention over 40 x 60 tokens: 79 x 119 = 9401 bins, more than the backward's LDS bins
    hold, so dT is accumulated with global integer atomics."""
    cfg = _cfg("global_40x60", (1, 40, 60), (1, 40, 60), ((0, 0, 0),), periodic=0)
    log("bf16 global 40x60 forward and backward (9401 bins)", cfg.grid, cfg.window)
    _check(cfg)


@pytest.mark.parametrize("offset", [200.0, -200.0])
def test_bf16_constant_table_offset(offset):
    """A constant bias table adds the same amount to every unmasked logit of a row, which the
    softmax ignores. At +-200 (+-288.5 in log2 units) exp2 of the raw logits overflows or
    underflows, so the forward's offset-free first pass must fall back to the row-maximum offset
    (144-token windows, W-MSA then SW-MSA, ragged edge windows)."""
    cfg = _cfg("table_offset", (1, 30, 40), (1, 12, 12), ((0, 0, 0), (0, 6, 6)))
    inp = make_inputs(cfg)
    for m in inp.modules:
        m.table = np.full_like(m.table, offset)
        m.table_dev = np.full_like(m.table_dev, offset)
    log("bf16 constant bias table %+.0f" % offset, cfg.grid, cfg.window)
    _check(cfg, inp=inp)


F32_CASES = [
    _cfg("f32_ragged", (1, 21, 29), (1, 6, 8), ((0, 3, 4),), dtype="f32", backward=False),
    _cfg("f32_window_1x1", (1, 6, 10), (1, 1, 1), ((0, 0, 0),), dtype="f32", backward=False),
    _cfg("f32_global", (1, 8, 16), (1, 8, 16), ((0, 0, 0),), dtype="f32", backward=False, batch=2),
    # head_dim 16 and 48: the guarded variants of the fp32 attention kernel (head_dim below its bound)
    _cfg("f32_hd16", (1, 12, 20), (1, 4, 8), ((0, 2, 4),), channels=32, heads=2, dtype="f32", backward=False),
    _cfg("f32_hd48", (1, 12, 20), (1, 4, 8), ((0, 2, 4),), channels=96, heads=2, dtype="f32", backward=False),
]


@pytest.mark.parametrize("cfg", F32_CASES, ids=lambda c: c.name)
def test_f32_edge_case_forward_vs_oracle(cfg):
    log("fp32 edge case", cfg.name, cfg.grid, cfg.window, cfg.shifts)
    _check(cfg, with_bwd=False)
