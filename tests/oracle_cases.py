"""Tiny configurations for oracle pins (shapes only)."""
import numpy as np

from oracle import swin_oracle as O
from workloads.configs import SwinConfig
from workloads import make_inputs

# (name, batch, grid, C, heads, window, shift, periodic)
TINY = [
    ("masked2d", 1, (1, 8, 12), 16, 2, (1, 4, 4), (0, 2, 2), 0x4),
    ("ragged2d", 1, (1, 9, 11), 16, 2, (1, 4, 4), (0, 2, 2), 0x4),
    ("ragged_lat_periodic", 2, (1, 7, 10), 8, 1, (1, 3, 4), (0, 1, 2), 0x2),
    ("cube3d", 1, (4, 6, 8), 16, 2, (2, 3, 4), (1, 1, 2), 0x4),
    ("all_masked3d", 1, (5, 5, 6), 8, 2, (2, 3, 4), (1, 1, 2), 0x0),
    ("noshift", 1, (1, 8, 8), 16, 2, (1, 4, 4), (0, 0, 0), 0x4),
]


def tiny_cfg(case, dtype="f32"):
    name, b, grid, C, nh, win, sh, per = case
    return SwinConfig(name=name, batch=b, grid=grid, channels=C, heads=nh, window=win, shifts=(sh,),
                      dtype=dtype, backward=True, periodic=per)


def setup(case, seed=0, dtype="f32"):
    cfg = tiny_cfg(case, dtype)
    inp = make_inputs(cfg, seed=seed)
    m = inp.modules[0]
    p = O.Params(m.w_qkv, m.b_qkv, m.w_proj, m.b_proj, m.table)
    lay = O.window_layout(cfg.batch, cfg.grid, cfg.window, cfg.shifts[0], cfg.periodic)
    return cfg, inp, p, lay
