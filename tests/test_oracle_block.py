"""Pins of the Swin-block oracle (layer normalisation, GELU MLP, residuals around the
attention module).

Checked against: closed forms (normalised rows have mean 0 and unit biased variance; a
two-element row normalises to -1, +1; GELU(0) = 0 and GELU(1) = Phi(1)), torch float64
library routines (layer_norm, gelu and autograd through them), central finite differences
of the block forward for every input tensor, and blocks that reduce to simpler ones (zero
MLP weights leave y = h + b2; a zero attention projection leaves h = x + b_proj)."""
import math

import numpy as np
import pytest
import torch

from oracle import block_oracle as BO
from oracle import swin_oracle as O
from tests.oracle_cases import TINY, tiny_cfg
from workloads import make_block_extras, make_inputs


def _setup(case, hidden=None, norm_scale=0.1):
    cfg = tiny_cfg(case)
    inp = make_inputs(cfg)
    m = inp.modules[0]
    e = make_block_extras(cfg, hidden=hidden, norm_scale=norm_scale)[0]
    p = BO.BlockParams(ln1_g=e.ln1_g, ln1_b=e.ln1_b, attn=O.Params(m.w_qkv, m.b_qkv, m.w_proj, m.b_proj, m.table),
                       ln2_g=e.ln2_g, ln2_b=e.ln2_b, w1=e.w1, b1=e.b1, w2=e.w2, b2=e.b2)
    lay = O.window_layout(cfg.batch, cfg.grid, cfg.window, cfg.shifts[0], cfg.periodic)
    return cfg, inp, p, lay


def test_layer_norm_closed_forms():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 7, 16)) * 3 + 2
    y, mean, rstd = BO.layer_norm(x, np.ones(16), np.zeros(16), eps=0.0)
    assert np.abs(y.mean(-1)).max() < 1e-12
    assert np.abs((y ** 2).mean(-1) - 1).max() < 1e-12
    assert np.abs(mean - x.mean(-1)).max() < 1e-12
    # two channels: (a, b) -> (-1, +1) for a < b, whatever a and b
    y2, _, _ = BO.layer_norm(np.array([[3.0, 11.0]]), np.ones(2), np.zeros(2), eps=0.0)
    assert np.allclose(y2, [[-1.0, 1.0]], atol=1e-15)


def test_layer_norm_matches_torch():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((6, 24))
    g = 1 + 0.1 * rng.standard_normal(24)
    b = 0.1 * rng.standard_normal(24)
    dy = rng.standard_normal((6, 24))
    y, mean, rstd = BO.layer_norm(x, g, b, 1e-5)
    xt = torch.tensor(x, requires_grad=True)
    gt = torch.tensor(g, requires_grad=True)
    bt = torch.tensor(b, requires_grad=True)
    yt = torch.nn.functional.layer_norm(xt, (24,), gt, bt, 1e-5)
    assert np.abs(yt.detach().numpy() - y).max() < 1e-13
    (yt * torch.tensor(dy)).sum().backward()
    dx, dg, db = BO.layer_norm_bwd(dy, x, g, mean, rstd)
    assert np.abs(xt.grad.numpy() - dx).max() < 1e-12
    assert np.abs(gt.grad.numpy() - dg).max() < 1e-12
    assert np.abs(bt.grad.numpy() - db).max() < 1e-12


def test_gelu_closed_forms_and_torch():
    assert BO.gelu(np.array([0.0]))[0] == 0.0
    phi1 = 0.5 * (1 + math.erf(1 / math.sqrt(2)))     # standard normal CDF at 1
    assert abs(BO.gelu(np.array([1.0]))[0] - phi1) < 1e-15
    a = np.linspace(-6, 6, 97)
    at = torch.tensor(a, requires_grad=True)
    gt = torch.nn.functional.gelu(at)                 # exact (erf) form
    assert np.abs(gt.detach().numpy() - BO.gelu(a)).max() < 1e-14
    gt.sum().backward()
    assert np.abs(at.grad.numpy() - BO.gelu_grad(a)).max() < 1e-13
    # large |a|: a and 0
    assert abs(BO.gelu(np.array([30.0]))[0] - 30.0) < 1e-12 and abs(BO.gelu(np.array([-30.0]))[0]) < 1e-12


@pytest.mark.parametrize("case", [TINY[0], TINY[1], TINY[3]], ids=lambda c: c[0])
def test_block_backward_finite_differences(case):
    cfg, inp, p, lay = _setup(case, hidden=24)
    dy = inp.dy
    g = BO.block_bwd(dy, inp.x, p, lay, cfg.heads)

    def loss():
        y, _ = BO.block_fwd(inp.x, p, lay, cfg.heads)
        return float((y * dy).sum())

    rng = np.random.default_rng(9)
    eps = 1e-5
    targets = [("dx", inp.x), ("ln1_g", p.ln1_g), ("ln1_b", p.ln1_b), ("ln2_g", p.ln2_g), ("ln2_b", p.ln2_b),
               ("w1", p.w1), ("b1", p.b1), ("w2", p.w2), ("b2", p.b2), ("w_qkv", p.attn.w_qkv),
               ("w_proj", p.attn.w_proj), ("table", p.attn.table)]
    for name, arr in targets:
        flat = arr.reshape(-1)
        gflat = g[name].reshape(-1)
        for i in rng.choice(flat.size, size=min(8, flat.size), replace=False):
            old = flat[i]
            flat[i] = old + eps
            lp = loss()
            flat[i] = old - eps
            lm = loss()
            flat[i] = old
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - gflat[i]) <= 1e-7 * max(1.0, abs(fd)), (name, i, fd, gflat[i])


def test_block_reduces_to_simpler_blocks():
    cfg, inp, p, lay = _setup(TINY[0], hidden=24)
    C = cfg.channels
    # zero MLP input weights and bias: GELU(0) = 0, so the MLP adds exactly b2
    p0 = BO.BlockParams(**{**p.__dict__, "w1": np.zeros_like(p.w1), "b1": np.zeros_like(p.b1)})
    y, s = BO.block_fwd(inp.x, p0, lay, cfg.heads)
    assert np.abs(y - (s["h"] + p.b2)).max() < 1e-12
    # zero attention projection: the attention branch adds exactly b_proj
    a = p.attn
    p1 = BO.BlockParams(**{**p.__dict__, "attn": O.Params(a.w_qkv, a.b_qkv, np.zeros_like(a.w_proj), a.b_proj,
                                                          a.table)})
    _, s1 = BO.block_fwd(inp.x, p1, lay, cfg.heads)
    assert np.abs(s1["h"] - (inp.x + a.b_proj)).max() < 1e-12
    # the MLP bias gradient is the sum of dy, and the LN2 shift gradient the sum of dh at the MLP input
    g = BO.block_bwd(inp.dy, inp.x, p, lay, cfg.heads)
    assert np.abs(g["b2"] - inp.dy.reshape(-1, C).sum(0)).max() < 1e-11


def test_block_mlp_matches_torch_autograd():
    """The MLP half (LN2, W1, GELU, W2 and the residual) through torch float64 autograd."""
    cfg, inp, p, lay = _setup(TINY[1], hidden=24)
    _, s = BO.block_fwd(inp.x, p, lay, cfg.heads)
    C = cfg.channels
    h = torch.tensor(s["h"].reshape(-1, C), requires_grad=True)
    t = {k: torch.tensor(getattr(p, k), requires_grad=True) for k in ("ln2_g", "ln2_b", "w1", "b1", "w2", "b2")}
    xn2 = torch.nn.functional.layer_norm(h, (C,), t["ln2_g"], t["ln2_b"], 1e-5)
    y = h + torch.nn.functional.gelu(xn2 @ t["w1"].T + t["b1"]) @ t["w2"].T + t["b2"]
    y_or, _ = BO.block_fwd(inp.x, p, lay, cfg.heads)
    assert np.abs(y.detach().numpy() - y_or.reshape(-1, C)).max() < 1e-12
    (y * torch.tensor(inp.dy.reshape(-1, C))).sum().backward()
    g = BO.block_bwd(inp.dy, inp.x, p, lay, cfg.heads)
    for k in ("ln2_g", "ln2_b", "w1", "b1", "w2", "b2"):
        assert np.abs(t[k].grad.numpy() - g[k]).max() < 1e-10, k
