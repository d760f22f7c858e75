"""fp64 CPU oracle for a Swin Transformer block around the shifted-window attention module.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import or call this module: only
the tests use it. It shares no code with the HIP library; the attention part is the
attention oracle in oracle/swin_oracle.py.

What it computes, and from which passage:

* A block (TERRA page, section IV-A, Fig. 4: block 0 is W-MSA followed by an MLP, block 1
  is SW-MSA followed by an MLP, with layer normalisation in the block) is read as the
  pre-normalisation Swin block of the paper the page cites:
      h = x + A(LN1(x)),        y = h + W2 GELU(W1 LN2(h) + b1) + b2
  where A is the (shifted-)window attention module.
* Readings where the page is silent: layer normalisation over the C channels of a token
  with the biased variance and eps = 1e-5, then a per-channel scale and shift; GELU in its
  exact form 0.5 a (1 + erf(a / sqrt 2)); hidden width 4C (the usual MLP ratio).

Every function works in float64 on values the caller has already rounded to the run dtype.
The pins are in tests/test_oracle_block.py.
"""
from dataclasses import dataclass
from math import erf, pi, sqrt
from typing import Dict, Optional

import numpy as np

from . import swin_oracle as O

_erf = np.vectorize(erf, otypes=[np.float64])


def layer_norm(x: np.ndarray, g: np.ndarray, b: np.ndarray, eps: float = 1e-5):
    """y = (x - mean) / sqrt(var + eps) * g + b over the last axis (biased variance).
    Returns y, mean, rstd (the last two per row)."""
    mean = x.mean(axis=-1, keepdims=True)
    var = ((x - mean) ** 2).mean(axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + eps)
    return (x - mean) * rstd * g + b, mean[..., 0], rstd[..., 0]


def layer_norm_bwd(dy: np.ndarray, x: np.ndarray, g: np.ndarray, mean: np.ndarray, rstd: np.ndarray):
    """Gradients of layer_norm: with xhat = (x - mean) rstd and dxhat = dy g,
    dx = rstd (dxhat - mean(dxhat) - xhat mean(dxhat xhat)), dg = sum dy xhat, db = sum dy."""
    xhat = (x - mean[..., None]) * rstd[..., None]
    dxhat = dy * g
    dx = rstd[..., None] * (dxhat - dxhat.mean(axis=-1, keepdims=True)
                            - xhat * (dxhat * xhat).mean(axis=-1, keepdims=True))
    return dx, (dy * xhat).reshape(-1, x.shape[-1]).sum(axis=0), dy.reshape(-1, x.shape[-1]).sum(axis=0)


def gelu(a: np.ndarray) -> np.ndarray:
    """Exact GELU: a Phi(a) = 0.5 a (1 + erf(a / sqrt 2))."""
    return 0.5 * a * (1.0 + _erf(a / sqrt(2.0)))


def gelu_grad(a: np.ndarray) -> np.ndarray:
    """d/da of a Phi(a) = Phi(a) + a phi(a)."""
    return 0.5 * (1.0 + _erf(a / sqrt(2.0))) + a * np.exp(-0.5 * a * a) / sqrt(2.0 * pi)


@dataclass
class BlockParams:
    ln1_g: np.ndarray   # [C]
    ln1_b: np.ndarray   # [C]
    attn: O.Params
    ln2_g: np.ndarray   # [C]
    ln2_b: np.ndarray   # [C]
    w1: np.ndarray      # [H, C]   (H = hidden width)
    b1: np.ndarray      # [H]
    w2: np.ndarray      # [C, H]
    b2: np.ndarray      # [C]


def block_fwd(x: np.ndarray, p: BlockParams, layout: O.Layout, heads: int, eps: float = 1e-5,
              scale: Optional[float] = None):
    """y and the intermediates the backward uses, for x of shape [B, D, H, W, C]."""
    xn1, mean1, rstd1 = layer_norm(x, p.ln1_g, p.ln1_b, eps)
    att, asaved = O.module_fwd(xn1, p.attn, layout, heads, scale)
    h = x + att
    xn2, mean2, rstd2 = layer_norm(h, p.ln2_g, p.ln2_b, eps)
    a1 = xn2 @ p.w1.T + p.b1
    g1 = gelu(a1)
    y = h + g1 @ p.w2.T + p.b2
    saved = {"xn1": xn1, "mean1": mean1, "rstd1": rstd1, "h": h, "xn2": xn2, "mean2": mean2, "rstd2": rstd2,
             "a1": a1, "g1": g1, "attn": asaved}
    return y, saved


def block_bwd(dy: np.ndarray, x: np.ndarray, p: BlockParams, layout: O.Layout, heads: int, eps: float = 1e-5,
              scale: Optional[float] = None) -> Dict[str, np.ndarray]:
    """Hand-derived backward of block_fwd (forward recomputed). Returns dx and every parameter
    gradient (the attention ones under the attention oracle's names)."""
    _, s = block_fwd(x, p, layout, heads, eps, scale)
    C = x.shape[-1]
    dy2 = dy.reshape(-1, C)
    g1 = s["g1"].reshape(dy2.shape[0], -1)
    a1 = s["a1"].reshape(dy2.shape[0], -1)
    xn2 = s["xn2"].reshape(-1, C)
    out = {"w2": dy2.T @ g1, "b2": dy2.sum(axis=0)}
    dg1 = dy2 @ p.w2
    da1 = dg1 * gelu_grad(a1)
    out["w1"] = da1.T @ xn2
    out["b1"] = da1.sum(axis=0)
    dxn2 = (da1 @ p.w1).reshape(x.shape)
    dh_ln, out["ln2_g"], out["ln2_b"] = layer_norm_bwd(dxn2, s["h"], p.ln2_g, s["mean2"], s["rstd2"])
    dh = dy + dh_ln
    dxn1, ga = O.module_bwd(dh, s["xn1"], p.attn, layout, heads, scale)
    for k in ("w_qkv", "b_qkv", "w_proj", "b_proj", "table"):
        out[k] = getattr(ga, k)
    dx_ln, out["ln1_g"], out["ln1_b"] = layer_norm_bwd(dxn1, x, p.ln1_g, s["mean1"], s["rstd1"])
    out["dx"] = dh + dx_ln
    return out


def block_flops(n_tokens: int, channels: int, hidden: int, heads: int, pairs: int) -> int:
    """Algorithmic forward FLOPs of a block: the attention module plus the two MLP products
    (layer normalisation, GELU and residual adds are not counted)."""
    attn = O.module_flops(n_tokens, channels, heads, pairs)["fwd"]
    return attn + 2 * 2 * n_tokens * channels * hidden
