"""Seeded input generation.

Draws follow one fixed recipe so that every consumer sees identical values:
numpy ``default_rng(seed)`` (PCG64), all draws in float64, in the order
x, then per chained module (W_qkv, b_qkv, W_proj, b_proj, T), then dy.

Distributions: x ~ N(0,1) and dy ~ N(0,1); Xavier-normal weights with
std = sqrt(2/(fan_in+fan_out)) where W_qkv is one [3C, C] matrix and W_proj is
[C, C]; biases ~ N(0,1) times ``bias_scale``: 1 by default (the configurations
give no bias distribution; N(0,1) exercises the bias gradients with values of the
size of everything else), 0 for throughput runs; the relative-position table
T ~ N(0, 0.02^2) (0.02 read as the standard deviation).

Rounding: activations, weights, biases and dy are rounded to the run dtype
(float64 -> float32 -> bfloat16, round-to-nearest-even at each step); T is
kept in float32. Both the device path and the oracle consume the rounded
values (the oracle upcasts them to float64).
"""
from dataclasses import dataclass
from typing import List, Optional

import numpy as np

from .configs import SwinConfig


def round_bf16(a: np.ndarray) -> np.ndarray:
    """float array -> uint16 bfloat16 bit patterns, RNE via float32."""
    f = np.ascontiguousarray(a, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    u = bits.astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


@dataclass
class ModuleParams:
    """Weights of one attention module, as float64 values already rounded to the run dtype.

    ``*_dev`` hold the same values in the storage format the device consumes
    (uint16 bf16 bits or float32)."""
    w_qkv: np.ndarray   # [3C, C]
    b_qkv: np.ndarray   # [3C]
    w_proj: np.ndarray  # [C, C]
    b_proj: np.ndarray  # [C]
    table: np.ndarray   # [nh, 2wd-1, 2wh-1, 2ww-1] (float32 values)
    w_qkv_dev: np.ndarray = None
    b_qkv_dev: np.ndarray = None
    w_proj_dev: np.ndarray = None
    b_proj_dev: np.ndarray = None
    table_dev: np.ndarray = None


@dataclass
class Inputs:
    cfg: SwinConfig
    x: np.ndarray            # [B, D, H, W, C] float64 (rounded values)
    dy: Optional[np.ndarray]
    modules: List[ModuleParams]
    x_dev: np.ndarray = None
    dy_dev: np.ndarray = None


def _to_dtype(a64: np.ndarray, dtype: str):
    """-> (float64 view of rounded values, device storage array)."""
    if dtype == "bf16":
        bits = round_bf16(a64)
        return bf16_bits_to_f64(bits), bits
    if dtype == "f32":
        f = a64.astype(np.float32)
        return f.astype(np.float64), f
    raise ValueError(dtype)


def make_inputs(cfg: SwinConfig, seed: int = 0, bias_scale: float = 1.0,
                with_dy: Optional[bool] = None, keep_f64: bool = True) -> Inputs:
    rng = np.random.default_rng(seed)
    B = cfg.batch
    D, H, W = cfg.grid
    C = cfg.channels
    x64 = rng.standard_normal((B, D, H, W, C))
    x, x_dev = _to_dtype(x64, cfg.dtype)
    del x64
    mods = []
    for _ in range(cfg.modules):
        wq = rng.standard_normal((3 * C, C)) * np.sqrt(2.0 / (C + 3 * C))
        bq = rng.standard_normal(3 * C) * bias_scale
        wp = rng.standard_normal((C, C)) * np.sqrt(2.0 / (C + C))
        bp = rng.standard_normal(C) * bias_scale
        t = (rng.standard_normal(cfg.bias_table_shape()) * 0.02).astype(np.float32)
        (wq_r, wq_d), (bq_r, bq_d) = _to_dtype(wq, cfg.dtype), _to_dtype(bq, cfg.dtype)
        (wp_r, wp_d), (bp_r, bp_d) = _to_dtype(wp, cfg.dtype), _to_dtype(bp, cfg.dtype)
        m = ModuleParams(w_qkv=wq_r, b_qkv=bq_r, w_proj=wp_r, b_proj=bp_r,
                         table=t.astype(np.float64),
                         w_qkv_dev=wq_d, b_qkv_dev=bq_d, w_proj_dev=wp_d, b_proj_dev=bp_d,
                         table_dev=t)
        mods.append(m)
    want_dy = cfg.backward if with_dy is None else with_dy
    dy = dy_dev = None
    if want_dy:
        dy64 = rng.standard_normal((B, D, H, W, C))
        dy, dy_dev = _to_dtype(dy64, cfg.dtype)
        del dy64
    if not keep_f64:
        x = None
        dy = None
    return Inputs(cfg=cfg, x=x, dy=dy, modules=mods, x_dev=x_dev, dy_dev=dy_dev)


@dataclass
class BlockExtras:
    """The parts of one Swin block around its attention module: two layer normalisations and
    the MLP, as float64 values rounded to the run dtype, plus their device storage (``dev``)."""
    ln1_g: np.ndarray
    ln1_b: np.ndarray
    ln2_g: np.ndarray
    ln2_b: np.ndarray
    w1: np.ndarray   # [hidden, C]
    b1: np.ndarray   # [hidden]
    w2: np.ndarray   # [C, hidden]
    b2: np.ndarray   # [C]
    dev: dict = None


# Scale of every bias inside a Swin block (b1, b2 here, and the attention module's b_qkv, b_proj,
# which the block tests draw with make_inputs(cfg, bias_scale=BLOCK_BIAS_SCALE)).
BLOCK_BIAS_SCALE = 0.1


def make_block_extras(cfg: SwinConfig, hidden: Optional[int] = None, seed: int = 0,
                      bias_scale: float = BLOCK_BIAS_SCALE, norm_scale: float = 0.1) -> List[BlockExtras]:
    """Per chained block, drawn from numpy default_rng([seed, 1]) (a stream separate from
    make_inputs, whose draws stay unchanged) in float64, in the order ln1 scale, ln1 shift,
    ln2 scale, ln2 shift, W1, b1, W2, b2. Scales are 1 + norm_scale N(0,1) and shifts
    norm_scale N(0,1) (0 and 1 exactly when norm_scale = 0); W1, W2 Xavier-normal; biases
    bias_scale N(0,1). Hidden width 4C unless given."""
    rng = np.random.default_rng([seed, 1])
    C = cfg.channels
    H = 4 * C if hidden is None else hidden
    out = []
    for _ in range(cfg.modules):
        draws = {
            "ln1_g": 1.0 + norm_scale * rng.standard_normal(C),
            "ln1_b": norm_scale * rng.standard_normal(C),
            "ln2_g": 1.0 + norm_scale * rng.standard_normal(C),
            "ln2_b": norm_scale * rng.standard_normal(C),
            "w1": rng.standard_normal((H, C)) * np.sqrt(2.0 / (C + H)),
            "b1": bias_scale * rng.standard_normal(H),
            "w2": rng.standard_normal((C, H)) * np.sqrt(2.0 / (C + H)),
            "b2": bias_scale * rng.standard_normal(C),
        }
        vals, dev = {}, {}
        for k, v in draws.items():
            vals[k], dev[k] = _to_dtype(v, cfg.dtype)
        out.append(BlockExtras(dev=dev, **vals))
    return out
