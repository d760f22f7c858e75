"""Pins of the oracle's hand-derived backward.

Checked against: central finite differences of the oracle's own forward (in
float64, on sampled entries of every input), torch float64 autograd through
an independent torch formulation of the module (scaled_dot_product_attention
as the attention routine), and exact invariants (bias-table gradient sums to
zero per head, key-bias gradient is zero, proj-bias gradient is the sum of dy)."""
import numpy as np
import pytest
import torch

from oracle import swin_oracle as O
from tests.oracle_cases import TINY, setup


def _loss(x, p, lay, heads, dy):
    y, _ = O.module_fwd(x, p, lay, heads)
    return float((y * dy).sum())


FD_CASES = [TINY[0], TINY[1], TINY[3], TINY[4]]


@pytest.mark.parametrize("case", FD_CASES, ids=lambda c: c[0])
def test_finite_differences(case):
    cfg, inp, p, lay = setup(case)
    dy = inp.dy
    dx, g = O.module_bwd(dy, inp.x, p, lay, cfg.heads)
    rng = np.random.default_rng(5)
    eps = 1e-5
    targets = [("x", inp.x, dx), ("w_qkv", p.w_qkv, g.w_qkv), ("b_qkv", p.b_qkv, g.b_qkv),
               ("w_proj", p.w_proj, g.w_proj), ("b_proj", p.b_proj, g.b_proj), ("table", p.table, g.table)]
    for name, arr, grad in targets:
        flat = arr.reshape(-1)
        gflat = grad.reshape(-1)
        idx = rng.choice(flat.size, size=min(12, flat.size), replace=False)
        if name == "b_qkv":   # make sure q, k and v biases are all sampled
            C = cfg.channels
            idx = np.concatenate([idx, [0, C, 2 * C + 1]])
        for i in idx:
            old = flat[i]
            flat[i] = old + eps
            lp = _loss(inp.x, p, lay, cfg.heads, dy)
            flat[i] = old - eps
            lm = _loss(inp.x, p, lay, cfg.heads, dy)
            flat[i] = old
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - gflat[i]) <= 1e-7 * max(1.0, abs(fd)), (name, i, fd, gflat[i])


@pytest.mark.parametrize("case", TINY, ids=lambda c: c[0])
def test_exact_invariants(case):
    cfg, inp, p, lay = setup(case)
    dx, g = O.module_bwd(inp.dy, inp.x, p, lay, cfg.heads)
    C = cfg.channels
    # rows of dS sum to zero, so every head's table gradient sums to zero
    assert np.abs(g.table.reshape(cfg.heads, -1).sum(1)).max() < 1e-12
    # a key bias shifts each row of logits by a constant: no gradient
    assert np.abs(g.b_qkv[C:2 * C]).max() < 1e-12
    assert np.abs(g.b_proj - inp.dy.reshape(-1, C).sum(0)).max() < 1e-11


def _torch_module(x, wq, bq, wp, bp, tab, lay, heads):
    """Independent torch formulation: index_select gather, SDPA per extent group, index_copy scatter."""
    C = x.shape[-1]
    hd = C // heads
    xf = x.reshape(-1, C)
    perm = torch.from_numpy(lay.perm)
    xw = xf.index_select(0, perm)
    out = torch.zeros_like(xw)
    tflat = tab.reshape(heads, -1)
    for win in lay.windows:
        r = torch.arange(win.tok_off, win.tok_off + win.n)
        xt = xw.index_select(0, r)
        qkv = xt @ wq.T + bq
        q, k, v = (qkv[:, i * C:(i + 1) * C].reshape(win.n, heads, hd).transpose(0, 1) for i in range(3))
        loc = torch.from_numpy(lay.local[win.tok_off:win.tok_off + win.n])
        wd, wh, ww = lay.window
        rel = loc[:, None, :] - loc[None, :, :] + torch.tensor([wd - 1, wh - 1, ww - 1])
        bins = (rel[..., 0] * (2 * wh - 1) + rel[..., 1]) * (2 * ww - 1) + rel[..., 2]
        lab = torch.from_numpy(lay.labels[win.tok_off:win.tok_off + win.n].astype(np.int64))
        mask = torch.where(lab[:, None] == lab[None, :], 0.0, float("-inf")).to(torch.float64)
        bias = tflat[:, bins] + mask
        o = torch.nn.functional.scaled_dot_product_attention(q[None], k[None], v[None], attn_mask=bias[None],
                                                             scale=hd ** -0.5)[0]
        o = o.transpose(0, 1).reshape(win.n, C)
        out = out.index_copy(0, r, o @ wp.T + bp)
    y = torch.zeros_like(xf).index_copy(0, perm, out)
    return y.reshape(x.shape)


@pytest.mark.parametrize("case", TINY, ids=lambda c: c[0])
def test_torch_autograd_crosscheck(case):
    cfg, inp, p, lay = setup(case)
    dx, g = O.module_bwd(inp.dy, inp.x, p, lay, cfg.heads)
    y_np, _ = O.module_fwd(inp.x, p, lay, cfg.heads)
    ts = [torch.tensor(a, dtype=torch.float64, requires_grad=True)
          for a in (inp.x, p.w_qkv, p.b_qkv, p.w_proj, p.b_proj, p.table)]
    y = _torch_module(*ts, lay, cfg.heads)
    assert np.abs(y.detach().numpy() - y_np).max() < 1e-12
    (y * torch.from_numpy(inp.dy)).sum().backward()
    for t, ref in zip(ts, (dx, g.w_qkv, g.b_qkv, g.w_proj, g.b_proj, g.table)):
        assert np.abs(t.grad.numpy() - ref).max() < 1e-11 * max(1.0, np.abs(ref).max())


@pytest.mark.parametrize("case", FD_CASES, ids=lambda c: c[0])
def test_absolute_term_sums(case):
    """The absolute-term sums (a diagnostic of how much a reduced gradient's terms cancel) leave
    the gradients unchanged, bound them from above (|sum a| <= sum |a|), and for the proj bias
    are the sum of |dy| over the tokens."""
    cfg, inp, p, lay = setup(case)
    _, g0 = O.module_bwd(inp.dy, inp.x, p, lay, cfg.heads)
    _, g1 = O.module_bwd(inp.dy, inp.x, p, lay, cfg.heads, with_abs=True)
    assert g0.abs is None
    for k in ("w_qkv", "b_qkv", "w_proj", "b_proj", "table"):
        assert np.array_equal(getattr(g0, k), getattr(g1, k)), k
        assert np.all(g1.abs[k] >= np.abs(getattr(g1, k)) * (1 - 1e-12)), k
    np.testing.assert_allclose(g1.abs["b_proj"], np.abs(inp.dy).reshape(-1, cfg.channels).sum(0), rtol=1e-12)
