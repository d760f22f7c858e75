"""Pins of the oracle's forward pass.

Checked against: an independent per-token brute-force loop; torch's
scaled_dot_product_attention in float64 (a library routine) for plain
per-window attention at shift 0 (windows formed by reshape, not slicing) and
for global attention when the window covers the grid; softmax row sums;
closed forms; translation equivariance; and a second formulation of masked
windows as unmasked sub-windows."""
import numpy as np
import pytest
import torch

from oracle import swin_oracle as O
from tests.oracle_cases import TINY, setup, tiny_cfg
from workloads import make_inputs


@pytest.mark.parametrize("case", TINY, ids=lambda c: c[0])
def test_brute_force_agrees(case):
    cfg, inp, p, lay = setup(case)
    y, _ = O.module_fwd(inp.x, p, lay, cfg.heads)
    yb = O.brute_force_fwd(inp.x, p, cfg.grid, cfg.window, cfg.shifts[0], cfg.periodic, cfg.heads)
    assert np.abs(y - yb).max() < 1e-12


def _sdpa(q, k, v, bias, scale):
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), attn_mask=torch.from_numpy(bias),
        scale=scale).numpy()


def _plain_window_attention_reshape(x, p, window, heads):
    """Shift 0, no mask: windows by reshape/transpose of the grid, attention by torch SDPA."""
    B, D, H, W, C = x.shape
    wd, wh, ww = window
    hd = C // heads
    xw = x.reshape(B, D // wd, wd, H // wh, wh, W // ww, ww, C).transpose(0, 1, 3, 5, 2, 4, 6, 7)
    xw = xw.reshape(-1, wd * wh * ww, C)
    qkv = xw @ p.w_qkv.T + p.b_qkv
    q, k, v = (qkv[..., i * C:(i + 1) * C].reshape(xw.shape[0], -1, heads, hd).transpose(0, 2, 1, 3)
               for i in range(3))
    # bias: offsets taken from explicit coordinates of the reshaped window
    cd, ch, cw = np.meshgrid(np.arange(wd), np.arange(wh), np.arange(ww), indexing="ij")
    coords = np.stack([cd.ravel(), ch.ravel(), cw.ravel()], 1)
    rel = coords[:, None, :] - coords[None, :, :] + np.array([wd - 1, wh - 1, ww - 1])
    bias = p.table[:, rel[..., 0], rel[..., 1], rel[..., 2]]           # [nh, n, n]
    o = _sdpa(q, k, v, np.broadcast_to(bias, (xw.shape[0],) + bias.shape).copy(), hd ** -0.5)
    yw = o.transpose(0, 2, 1, 3).reshape(xw.shape[0], -1, C) @ p.w_proj.T + p.b_proj
    yw = yw.reshape(B, D // wd, H // wh, W // ww, wd, wh, ww, C).transpose(0, 1, 4, 2, 5, 3, 6, 7)
    return yw.reshape(B, D, H, W, C)


@pytest.mark.parametrize("grid,window", [((1, 8, 12), (1, 4, 4)), ((4, 6, 8), (2, 3, 4)), ((1, 12, 24), (1, 6, 12))])
def test_shift0_equals_plain_window_attention(grid, window):
    case = ("plain", 2, grid, 16, 2, window, (0, 0, 0), 0x0)   # nothing periodic: still no mask at shift 0
    cfg, inp, p, lay = setup(case)
    y, _ = O.module_fwd(inp.x, p, lay, cfg.heads)
    y_ref = _plain_window_attention_reshape(inp.x, p, cfg.window, cfg.heads)
    assert np.abs(y - y_ref).max() < 1e-12


@pytest.mark.parametrize("grid", [(1, 6, 8), (2, 3, 4)])
def test_window_equals_grid_is_global_attention(grid):
    case = ("global", 1, grid, 16, 2, grid, (0, 0, 0), 0x4)
    cfg, inp, p, lay = setup(case)
    assert len(lay.windows) == 1
    y, _ = O.module_fwd(inp.x, p, lay, cfg.heads)
    x = inp.x.reshape(-1, cfg.channels)
    C, nh = cfg.channels, cfg.heads
    hd = C // nh
    qkv = x @ p.w_qkv.T + p.b_qkv
    q, k, v = (qkv[:, i * C:(i + 1) * C].reshape(-1, nh, hd).transpose(1, 0, 2)[None] for i in range(3))
    D, H, W = grid
    coords = np.stack(np.unravel_index(np.arange(D * H * W), (D, H, W)), 1)
    rel = coords[:, None, :] - coords[None, :, :] + np.array([D - 1, H - 1, W - 1])
    bias = p.table[:, rel[..., 0], rel[..., 1], rel[..., 2]][None].copy()
    o = _sdpa(q, k, v, bias, hd ** -0.5)[0].transpose(1, 0, 2).reshape(-1, C)
    y_ref = o @ p.w_proj.T + p.b_proj
    assert np.abs(y.reshape(-1, C) - y_ref).max() < 1e-12


@pytest.mark.parametrize("case", TINY, ids=lambda c: c[0])
def test_softmax_rows_sum_to_one_and_masked_exact_zero(case):
    cfg, inp, p, lay = setup(case)
    _, saved = O.windows_fwd(O.gather(inp.x, lay), p, lay, cfg.heads, keep=True)
    for g in saved["groups"]:
        P = g["P"]
        assert np.abs(P.sum(-1) - 1).max() < 1e-13
        assert np.all(P[~np.broadcast_to(g["allowed"][:, None], P.shape)] == 0.0)
        assert np.all(P[np.broadcast_to(g["allowed"][:, None], P.shape)] > 0.0)


@pytest.mark.parametrize("case", TINY[:4], ids=lambda c: c[0])
def test_closed_form_constant_values(case):
    # W_v = 0, b_v = c  =>  o == c for every token  =>  y == W_proj c + b_proj
    cfg, inp, p, lay = setup(case)
    C = cfg.channels
    p.w_qkv[2 * C:] = 0.0
    c = np.linspace(-1, 1, C)
    p.b_qkv[2 * C:] = c
    y, _ = O.module_fwd(inp.x, p, lay, cfg.heads)
    assert np.abs(y - (p.w_proj @ c + p.b_proj)).max() < 1e-12


@pytest.mark.parametrize("case", TINY, ids=lambda c: c[0])
def test_closed_form_uniform_weights(case):
    # W_q = 0, b_q = 0, T = 0  =>  all allowed logits equal  =>  o_i = mean of v over i's allowed keys
    cfg, inp, p, lay = setup(case)
    C, nh = cfg.channels, cfg.heads
    p.w_qkv[:C] = 0.0
    p.b_qkv[:C] = 0.0
    p.table[:] = 0.0
    xw = O.gather(inp.x, lay)
    _, saved = O.windows_fwd(xw, p, lay, nh)
    v = xw @ p.w_qkv[2 * C:].T + p.b_qkv[2 * C:]
    for win in lay.windows:
        rows = np.arange(win.tok_off, win.tok_off + win.n)
        lab = lay.labels[rows]
        for i, r in enumerate(rows):
            keys = rows[lab == lab[i]]
            assert np.abs(saved["o"][r] - v[keys].mean(0)).max() < 1e-12


@pytest.mark.parametrize("case", TINY[:3], ids=lambda c: c[0])
def test_key_bias_has_no_effect(case):
    cfg, inp, p, lay = setup(case)
    y0, _ = O.module_fwd(inp.x, p, lay, cfg.heads)
    C = cfg.channels
    p.b_qkv[C:2 * C] += 3.0 * np.cos(np.arange(C))
    y1, _ = O.module_fwd(inp.x, p, lay, cfg.heads)
    assert np.abs(y0 - y1).max() < 1e-11


def test_translation_equivariance_along_lon():
    # W divisible by ww, lon periodic: translating x by a multiple of ww translates y the same way
    case = ("transl", 1, (1, 8, 16), 16, 2, (1, 4, 4), (0, 2, 2), 0x4)
    cfg, inp, p, lay = setup(case)
    y, _ = O.module_fwd(inp.x, p, lay, cfg.heads)
    xs = np.roll(inp.x, 8, axis=3)
    ys, _ = O.module_fwd(xs, p, lay, cfg.heads)
    assert np.abs(np.roll(y, 8, axis=3) - ys).max() < 1e-12


@pytest.mark.parametrize("case", TINY, ids=lambda c: c[0])
def test_mask_equals_unmasked_subwindows(case):
    cfg, inp, p, lay = setup(case)
    xw = O.gather(inp.x, lay)
    y1, _ = O.windows_fwd(xw, p, lay, cfg.heads)
    y2 = O.windows_fwd_split(xw, p, lay, cfg.heads)
    assert np.abs(y1 - y2).max() < 1e-12


def test_window_subset_matches_full():
    cfg, inp, p, lay = setup(TINY[1])
    xw = O.gather(inp.x, lay)
    y_all, _ = O.windows_fwd(xw, p, lay, cfg.heads)
    ids = [0, 3, len(lay.windows) - 1]
    y_sub, _ = O.windows_fwd(xw, p, lay, cfg.heads, window_ids=ids, max_batch=2)
    for i in ids:
        w = lay.windows[i]
        assert np.array_equal(y_sub[w.tok_off:w.tok_off + w.n], y_all[w.tok_off:w.tok_off + w.n])
