"""The five synthetic workloads of the shifted-window attention path.

Axis convention everywhere: the token grid is (D, H, W) = (level, lat, lon),
channels last, as the TERRA page describes its fields (section II-A: a
B x H x W x C tensor on a regular latitude-longitude grid). A 2-D grid has
D = 1, window depth 1 and level shift 0.

Periodicity is a bit mask over the three axes (bit 0 level, bit 1 lat,
bit 2 lon). Longitude wraps around the globe; latitude and level do not, so
their shift regions are masked.
"""
from dataclasses import dataclass, field
from typing import Tuple

PERIODIC_LON = 0x4


@dataclass(frozen=True)
class SwinConfig:
    name: str
    batch: int
    grid: Tuple[int, int, int]      # (D, H, W)
    channels: int
    heads: int
    window: Tuple[int, int, int]    # (wd, wh, ww)
    shifts: Tuple[Tuple[int, int, int], ...]  # one shift per chained module
    dtype: str                      # "f32" or "bf16"
    backward: bool
    periodic: int = PERIODIC_LON
    description: str = ""

    @property
    def ndim(self) -> int:
        return 2 if self.grid[0] == 1 and self.window[0] == 1 else 3

    @property
    def n_tokens(self) -> int:
        d, h, w = self.grid
        return self.batch * d * h * w

    @property
    def head_dim(self) -> int:
        return self.channels // self.heads

    @property
    def modules(self) -> int:
        return len(self.shifts)

    def bias_table_shape(self):
        wd, wh, ww = self.window
        return (self.heads, 2 * wd - 1, 2 * wh - 1, 2 * ww - 1)


CONFIGS = {
    "tiny": SwinConfig(
        name="tiny", batch=1, grid=(1, 32, 64), channels=64, heads=2,
        window=(1, 8, 8), shifts=((0, 4, 4),), dtype="f32", backward=False,
        description="32x64 lat-lon grid, C=64, 2 heads, 8x8 window, shift (4,4), fp32 forward"),
    "om4": SwinConfig(
        name="om4", batch=2, grid=(1, 180, 360), channels=192, heads=6,
        window=(1, 6, 12), shifts=((0, 3, 6),), dtype="bf16", backward=True,
        description="1-degree 180x360 grid, batch 2, C=192, 6 heads, 6x12 window, shift (3,6)"),
    "ragged": SwinConfig(
        name="ragged", batch=1, grid=(1, 181, 361), channels=256, heads=8,
        window=(1, 8, 16), shifts=((0, 4, 8),), dtype="bf16", backward=True,
        description="181x361 grid with ragged edge windows, C=256, 8 heads, 8x16 window, shift (4,8)"),
    "highres": SwinConfig(
        name="highres", batch=1, grid=(1, 540, 1080), channels=512, heads=16,
        window=(1, 12, 12), shifts=((0, 0, 0), (0, 6, 6)), dtype="bf16", backward=True,
        description="540x1080 tokens (2160x4320 field after 4x4 patch embedding), C=512, 16 heads, "
                    "12x12 window, W-MSA then SW-MSA shift (6,6)"),
    "levels3d": SwinConfig(
        name="levels3d", batch=1, grid=(8, 180, 360), channels=192, heads=6,
        window=(2, 6, 12), shifts=((1, 3, 6),), dtype="bf16", backward=True,
        description="8x180x360 level-lat-lon grid, C=192, 6 heads, 2x6x12 window, shift (1,3,6)"),
}

ORDER = ["tiny", "om4", "ragged", "highres", "levels3d"]


def get_config(name: str) -> SwinConfig:
    return CONFIGS[name]


def small_variant(cfg: SwinConfig, grid, batch=None, channels=None, heads=None) -> SwinConfig:
    """Same window/shift/periodicity/dtype as cfg on a smaller grid (for fast oracle runs)."""
    return SwinConfig(
        name=cfg.name + "_small", batch=cfg.batch if batch is None else batch, grid=tuple(grid),
        channels=cfg.channels if channels is None else channels,
        heads=cfg.heads if heads is None else heads, window=cfg.window, shifts=cfg.shifts,
        dtype=cfg.dtype, backward=cfg.backward, periodic=cfg.periodic,
        description="reduced grid of " + cfg.name)
