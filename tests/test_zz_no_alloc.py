"""swin_attn_bwd_noalloc (the backward on the library's own per-GPU scratch array) against
swin_attn_bwd with a caller workspace, through the C ABI: outputs must be bitwise equal,
on consecutive calls of different sizes (the scratch keeps the previous call's contents),
including the tiled path whose bias-gradient accumulator must be cleared on every call."""
import ctypes

import numpy as np
import pytest

from tests.gpu_util import ModuleOnDevice, log, to_dev
from workloads import get_config, make_inputs
from workloads.configs import SwinConfig, small_variant

pytestmark = pytest.mark.gpu

GRADS = ("w_qkv", "b_qkv", "w_proj", "b_proj", "table")


def _case(cfg, module):
    import torch
    inp = make_inputs(cfg)
    m = ModuleOnDevice(cfg, module, inp.modules[module])
    x = to_dev(inp.x_dev, "bf16")
    dy = to_dev(inp.dy_dev, "bf16")
    m.fwd(x)
    torch.cuda.synchronize()
    return m, x, dy


def _noalloc_bwd(m, dy, x):
    import torch
    C = m.cfg.channels
    dx = torch.empty_like(dy)
    g = {"w_qkv": torch.empty(3 * C, C, dtype=torch.float32, device="cuda"),
         "b_qkv": torch.empty(3 * C, dtype=torch.float32, device="cuda"),
         "w_proj": torch.empty(C, C, dtype=torch.float32, device="cuda"),
         "b_proj": torch.empty(C, dtype=torch.float32, device="cuda"),
         "table": torch.empty_like(m.table)}
    m.N.swin_attn_bwd_noalloc(m.plan.handle, dy, x, m.w_qkv, m.w_proj, m.table, m.saved, dx, g["w_qkv"],
                              g["b_qkv"], g["w_proj"], g["b_proj"], g["table"])
    return dx, g


def _check_equal(m, x, dy, label):
    import torch
    want_dx, want = m.bwd(dy, x)
    got_dx, got = _noalloc_bwd(m, dy, x)
    torch.cuda.synchronize()
    log(label, "bwd workspace", m.plan.bwd_ws, "bytes")
    assert torch.equal(got_dx, want_dx), label
    for k in GRADS:
        assert torch.equal(got[k], want[k]), (label, k)


def test_noalloc_backward_matches_workspace_backward():
    # one-tile kernels on a 36x48 grid at C=512, then a smaller input on the tiled kernels
    # (head_dim 64), then the tiled case again on the scratch the previous call left behind
    big = small_variant(get_config("highres"), grid=(1, 36, 48))
    tiled = SwinConfig(name="tiled_hd64", batch=1, grid=(1, 24, 32), channels=128, heads=2, window=(1, 8, 8),
                       shifts=((0, 4, 4),), dtype="bf16", backward=True, description="24x32, C=128, head_dim 64")
    m1, x1, dy1 = _case(big, 1)
    assert m1.plan.bwd_ws <= 64 << 20
    _check_equal(m1, x1, dy1, "one-tile 36x48 C=512")
    m2, x2, dy2 = _case(tiled, 0)
    assert m2.plan.bwd_ws < m1.plan.bwd_ws
    _check_equal(m2, x2, dy2, "tiled 24x32 C=128")
    _check_equal(m2, x2, dy2, "tiled 24x32 C=128, again")
    for m in (m1, m2):
        m.plan.close()


def test_noalloc_refuses_a_workspace_beyond_its_scratch():
    import torch
    from shifted_window_attention_amd import native as N
    cfg = get_config("om4")   # 129,600 tokens at C = 192: a backward workspace of ~0.3 GB
    desc = N.make_desc(cfg.batch, cfg.grid, cfg.channels, cfg.heads, cfg.window, cfg.shifts[0], cfg.periodic,
                       N.SWIN_BF16)
    plan = N.Plan(desc)
    assert plan.bwd_ws > N.SWIN_NOALLOC_SCRATCH_BYTES
    # the size check runs before any launch: small distinct stand-ins for the buffers, never read
    ts = [torch.zeros(8, dtype=torch.float32, device="cuda") for _ in range(12)]
    ps = [ctypes.c_void_p(t.data_ptr()) for t in ts]
    st = N.lib.swin_attn_bwd_noalloc(plan.handle, *ps, None)
    assert st == 3, N.lib.swin_attn_last_error()
    assert b"scratch" in N.lib.swin_attn_last_error()
    plan.close()
