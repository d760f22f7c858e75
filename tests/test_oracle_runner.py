"""The sampled-window oracle runner used by the full-size GPU checks agrees with the full
oracle run (CPU only)."""
import numpy as np
import pytest

from tests.oracle_runner import chain_full, chain_sampled, layouts
from workloads import get_config, make_inputs
from workloads.configs import small_variant


@pytest.mark.parametrize("name,grid", [("highres", (1, 36, 48)), ("ragged", (1, 25, 41)), ("levels3d", (4, 12, 24))])
def test_sampled_equals_full(name, grid):
    cfg = small_variant(get_config(name), grid=grid, channels=64, heads=2)
    inp = make_inputs(cfg)
    full = chain_full(cfg, inp)
    nwin = len(layouts(cfg)[-1].windows)
    pick = sorted({0, 1, nwin // 2, nwin - 1})
    s = chain_sampled(cfg, inp, pick)
    C = cfg.channels
    assert np.abs(full["y"].reshape(-1, C)[s["y_tokens"]] - s["y"]).max() < 1e-12
    assert np.abs(full["dx"].reshape(-1, C)[s["dx_tokens"]] - s["dx"]).max() < 1e-12


@pytest.mark.parametrize("name,grid", [("highres", (1, 36, 48)), ("ragged", (1, 25, 41))])
def test_masked_dy_equals_full(name, grid):
    from tests.oracle_runner import chain_masked_dy
    cfg = small_variant(get_config(name), grid=grid, channels=64, heads=2)
    inp = make_inputs(cfg)
    lay = layouts(cfg)[-1]
    pick = [0, len(lay.windows) - 1]
    C = cfg.channels
    keep = np.zeros(cfg.n_tokens, dtype=bool)
    for i in pick:
        w = lay.windows[i]
        keep[lay.perm[w.tok_off:w.tok_off + w.n]] = True
    inp.dy = np.where(keep[:, None], inp.dy.reshape(-1, C), 0.0).reshape(inp.dy.shape)
    full = chain_full(cfg, inp)
    r = chain_masked_dy(cfg, inp, pick, inp.dy)
    assert np.abs(full["dx"].reshape(-1, C)[r["dx_tokens"]] - r["dx"]).max() < 1e-12
    for gf, gr in zip(full["grads"], r["grads"]):
        for k in ("w_qkv", "b_qkv", "w_proj", "b_proj", "table"):
            assert np.abs(gf[k] - gr[k]).max() < 1e-10 * max(1.0, np.abs(gf[k]).max()), k
            # the absolute-term sums reduce over the same windows, so they agree too
            assert np.abs(gf["abs"][k] - gr["abs"][k]).max() < 1e-10 * max(1.0, np.abs(gf["abs"][k]).max()), k
