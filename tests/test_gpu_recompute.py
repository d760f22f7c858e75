"""The recomputing module calls (saved state o + LSE only, q/k/v rebuilt from x in the backward)
against swin_attn_fwd / swin_attn_bwd through the C ABI: y, dx and every gradient must be bitwise
equal, on the one-tile and the tiled backward, in a W-MSA -> SW-MSA chain; plus the sizes and the
argument errors."""
import ctypes

import pytest

from tests.gpu_util import ModuleOnDevice, log, to_dev
from workloads import get_config, make_inputs
from workloads.configs import SwinConfig, small_variant

pytestmark = pytest.mark.gpu

GRADS = ("w_qkv", "b_qkv", "w_proj", "b_proj", "table")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _grads(t, C, table):
    return {"w_qkv": t.empty(3 * C, C, dtype=t.float32, device="cuda"),
            "b_qkv": t.empty(3 * C, dtype=t.float32, device="cuda"),
            "w_proj": t.empty(C, C, dtype=t.float32, device="cuda"),
            "b_proj": t.empty(C, dtype=t.float32, device="cuda"),
            "table": t.empty_like(table)}


def _recompute_chain(mods, x, dy):
    """Forward through the chain with the recomputing calls, then backward in reverse."""
    import torch
    N = mods[0].N
    xs, saved = [x], []
    for m in mods:
        fwd_ws, _, sb = N.swin_attn_sizes_recompute(m.plan.handle)
        sv = torch.empty(sb, dtype=torch.uint8, device="cuda")
        ws = torch.empty(fwd_ws, dtype=torch.uint8, device="cuda")
        y = torch.empty_like(xs[-1])
        N.swin_attn_fwd_recompute(m.plan.handle, xs[-1], m.w_qkv, m.b_qkv, m.w_proj, m.b_proj, m.table, y, sv, ws)
        xs.append(y)
        saved.append(sv)
    d = dy
    grads = [None] * len(mods)
    for i in reversed(range(len(mods))):
        m = mods[i]
        _, bwd_ws, _ = N.swin_attn_sizes_recompute(m.plan.handle)
        ws = torch.empty(bwd_ws, dtype=torch.uint8, device="cuda")
        dx = torch.empty_like(d)
        g = _grads(torch, m.cfg.channels, m.table)
        N.swin_attn_bwd_recompute(m.plan.handle, d, xs[i], m.w_qkv, m.b_qkv, m.w_proj, m.table, saved[i], dx,
                                  g["w_qkv"], g["b_qkv"], g["w_proj"], g["b_proj"], g["table"], ws)
        d, grads[i] = dx, g
    torch.cuda.synchronize()
    return xs[-1], d, grads


CASES = [
    ("om4", small_variant(get_config("om4"), grid=(1, 36, 72))),
    ("highres_c512", small_variant(get_config("highres"), grid=(1, 36, 48))),
    ("tiled_w16", SwinConfig(name="tiled_w16", batch=1, grid=(1, 32, 48), channels=128, heads=4, window=(1, 16, 16),
                             shifts=((0, 0, 0), (0, 8, 8)), dtype="bf16", backward=True, periodic=4,
                             description="256-token windows: tiled backward")),
]


@pytest.mark.parametrize("name,cfg", CASES, ids=[c[0] for c in CASES])
def test_recompute_matches_saved_qkv(name, cfg):
    import torch
    log("recompute vs saved q/k/v", name, cfg.grid, "C", cfg.channels, "window", cfg.window)
    inp = make_inputs(cfg)
    mods = [ModuleOnDevice(cfg, i, p) for i, p in enumerate(inp.modules)]
    x = to_dev(inp.x_dev, "bf16")
    dy = to_dev(inp.dy_dev, "bf16")
    # reference: the saved-q/k/v calls
    xs = [x]
    for m in mods:
        xs.append(m.fwd(xs[-1]))
    d = dy
    ref = [None] * len(mods)
    for i in reversed(range(len(mods))):
        d, ref[i] = mods[i].bwd(d, xs[i])
    torch.cuda.synchronize()
    y_r, dx_r, g_r = _recompute_chain(mods, x, dy)
    assert torch.equal(y_r.view(torch.int16), xs[-1].view(torch.int16))
    assert torch.equal(dx_r.view(torch.int16), d.view(torch.int16))
    for i in range(len(mods)):
        for k in GRADS:
            assert torch.equal(g_r[i][k], ref[i][k]), (name, i, k)
    for m in mods:
        fwd_ws, bwd_ws, sb = m.N.swin_attn_sizes_recompute(m.plan.handle)
        assert sb < m.plan.saved_bytes and fwd_ws == m.plan.saved_bytes - sb   # q/k/v planes moved to the workspace
        assert bwd_ws == fwd_ws + m.plan.bwd_ws
        log("  saved bytes %d -> %d, backward workspace %d -> %d" % (m.plan.saved_bytes, sb, m.plan.bwd_ws, bwd_ws))


def test_recompute_argument_errors():
    import torch
    N = __import__("shifted_window_attention_amd.native", fromlist=["native"])
    cfg = small_variant(get_config("om4"), grid=(1, 36, 72))
    inp = make_inputs(cfg)
    m = ModuleOnDevice(cfg, 0, inp.modules[0])
    x = to_dev(inp.x_dev, "bf16")
    fwd_ws, bwd_ws, sb = N.swin_attn_sizes_recompute(m.plan.handle)
    y = torch.empty_like(x)
    sv = torch.empty(sb, dtype=torch.uint8, device="cuda")
    short = torch.empty(fwd_ws - 256, dtype=torch.uint8, device="cuda")
    L = N.lib
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    st = L.swin_attn_fwd_recompute(m.plan.handle, p(x), p(m.w_qkv), p(m.b_qkv), p(m.w_proj), p(m.b_proj), p(m.table),
                                   p(y), p(sv), p(short), short.numel(), None)
    assert st == 3 and b"workspace" in L.swin_attn_last_error()
    st = L.swin_attn_fwd_recompute(m.plan.handle, p(x), p(m.w_qkv), p(m.b_qkv), p(m.w_proj), p(m.b_proj), p(m.table),
                                   p(y), None, p(short), short.numel(), None)
    assert st == 1
    ws = torch.empty(fwd_ws, dtype=torch.uint8, device="cuda")
    N.swin_attn_fwd_recompute(m.plan.handle, x, m.w_qkv, m.b_qkv, m.w_proj, m.b_proj, m.table, y, sv, ws)
    g = _grads(torch, cfg.channels, m.table)
    dx = torch.empty_like(x)
    st = L.swin_attn_bwd_recompute(m.plan.handle, p(x), p(x), p(m.w_qkv), p(m.b_qkv), p(m.w_proj), p(m.table), p(sv),
                                   p(dx), p(g["w_qkv"]), p(g["b_qkv"]), p(g["w_proj"]), p(g["b_proj"]), p(g["table"]),
                                   p(ws), ws.numel(), None)
    assert st == 3   # bwd_ws > fwd_ws
    st = L.swin_attn_bwd_recompute(m.plan.handle, p(x), p(x), p(m.w_qkv), p(m.b_qkv), p(m.w_proj), p(m.table), p(sv),
                                   p(x), p(g["w_qkv"]), p(g["b_qkv"]), p(g["w_proj"]), p(g["b_proj"]), p(g["table"]),
                                   p(ws), ws.numel(), None)
    assert st == 1   # dx aliases x
    torch.cuda.synchronize()
    # fp32 plans have no recomputing calls
    f32 = N.Plan(N.make_desc(1, (1, 32, 64), 64, 2, (1, 8, 8), (0, 4, 4), 4, N.SWIN_F32))
    with pytest.raises(N.SwinError):
        N.swin_attn_sizes_recompute(f32.handle)
