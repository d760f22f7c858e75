"""The Python binding checks every tensor against the plan before a device call: a buffer
too small for the call, of the wrong element type, on the host or not contiguous raises in
Python and launches nothing, so the kernels never see a buffer shorter than their grid assumes.
Errors the library itself reports (NULL pointers, aliasing, workspace sizes, rank numbers) still
come back as SwinError with their status."""
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _module(N, torch, C=64, heads=2):
    desc = N.make_desc(1, (1, 12, 24), C, heads, (1, 6, 6), (0, 3, 3), N.SWIN_PERIODIC_LON, N.SWIN_BF16)
    plan = N.Plan(desc)
    T = plan.stats["n_tokens"]
    bf = dict(dtype=torch.bfloat16, device="cuda")
    m = {"x": torch.zeros(T, C, **bf), "y": torch.empty(T, C, **bf), "w_qkv": torch.zeros(3 * C, C, **bf),
         "b_qkv": torch.zeros(3 * C, **bf), "w_proj": torch.zeros(C, C, **bf), "b_proj": torch.zeros(C, **bf),
         "table": torch.zeros(heads, 1, 11, 11, dtype=torch.float32, device="cuda"), "saved": plan.alloc_saved()}
    return plan, m


def _fwd(N, plan, m, **over):
    a = {**m, **over}
    N.swin_attn_fwd(plan.handle, a["x"], a["w_qkv"], a["b_qkv"], a["w_proj"], a["b_proj"], a["table"], a["y"],
                    a["saved"])


def test_attention_forward_buffer_checks():
    import torch
    from shifted_window_attention_amd import native as N
    plan, m = _module(N, torch)
    _fwd(N, plan, m)  # the well-formed call runs
    torch.cuda.synchronize()
    with pytest.raises(ValueError, match="x:"):
        _fwd(N, plan, m, x=m["x"][:-1])                                   # one token short
    with pytest.raises(TypeError, match="y:"):
        _fwd(N, plan, m, y=torch.empty_like(m["y"], dtype=torch.float32))  # wrong element type
    with pytest.raises(ValueError, match="w_qkv:"):
        _fwd(N, plan, m, w_qkv=m["w_qkv"][:, :32])                        # not contiguous
    with pytest.raises(ValueError, match="w_proj:"):
        _fwd(N, plan, m, w_proj=m["w_proj"].cpu())                        # host memory
    with pytest.raises(TypeError, match="bias_table:"):
        _fwd(N, plan, m, table=m["table"].to(torch.bfloat16))            # the table is fp32
    with pytest.raises(ValueError, match="saved:"):
        _fwd(N, plan, m, saved=m["saved"][:-1])
    # a NULL input is still the library's error
    with pytest.raises(N.SwinError) as e:
        _fwd(N, plan, m, x=None)
    assert e.value.status == 1
    torch.cuda.synchronize()
    plan.close()


def test_attention_backward_and_gather_buffer_checks():
    import torch
    from shifted_window_attention_amd import native as N
    plan, m = _module(N, torch)
    _fwd(N, plan, m)
    C = 64
    f32 = dict(dtype=torch.float32, device="cuda")
    g = {"dw_qkv": torch.empty(3 * C, C, **f32), "db_qkv": torch.empty(3 * C, **f32),
         "dw_proj": torch.empty(C, C, **f32), "db_proj": torch.empty(C, **f32),
         "dtab": torch.empty_like(m["table"])}
    dx = torch.empty_like(m["x"])
    ws = plan.alloc_bwd_ws()

    def bwd(**over):
        a = {**g, **over}
        N.swin_attn_bwd(plan.handle, m["x"], m["x"], m["w_qkv"], m["w_proj"], m["table"], m["saved"], a.get("dx", dx),
                        a["dw_qkv"], a["db_qkv"], a["dw_proj"], a["db_proj"], a["dtab"], ws)
    bwd()
    torch.cuda.synchronize()
    with pytest.raises(ValueError, match="dw_proj:"):
        bwd(dw_proj=g["dw_proj"][:-1])
    with pytest.raises(TypeError, match="dbias_table:"):
        bwd(dtab=torch.empty(g["dtab"].shape, dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError, match="dx:"):
        bwd(dx=dx[:-1])
    with pytest.raises(ValueError, match="xw:"):
        N.swin_window_gather(plan.handle, m["x"], m["y"][:-1])
    torch.cuda.synchronize()
    plan.close()


def test_block_and_route_buffer_checks():
    import torch
    from shifted_window_attention_amd import native as N
    C, H = 64, 256
    desc = N.make_desc(1, (1, 12, 24), C, 2, (1, 6, 6), (0, 0, 0), N.SWIN_PERIODIC_LON, N.SWIN_BF16)
    plan = N.BlockPlan(N.make_block_desc(desc, hidden=H))
    bf = dict(dtype=torch.bfloat16, device="cuda")
    shapes = {"ln1_g": (C,), "ln1_b": (C,), "w_qkv": (3 * C, C), "b_qkv": (3 * C,), "w_proj": (C, C),
              "b_proj": (C,), "ln2_g": (C,), "ln2_b": (C,), "w1": (H, C), "b1": (H,), "w2": (C, H), "b2": (C,)}
    prm = {k: torch.zeros(s, **bf) for k, s in shapes.items()}
    prm["bias_table"] = torch.zeros(2, 1, 11, 11, dtype=torch.float32, device="cuda")
    x = torch.zeros(288, C, **bf)
    saved = plan.alloc_saved()
    N.swin_block_fwd(plan.handle, x, prm, torch.empty_like(x), saved)
    torch.cuda.synchronize()
    with pytest.raises(ValueError, match="w1:"):
        N.swin_block_fwd(plan.handle, x, {**prm, "w1": torch.zeros(H - 1, C, **bf)}, torch.empty_like(x), saved)
    with pytest.raises(TypeError, match="ln2_g:"):
        N.swin_block_fwd(plan.handle, x, {**prm, "ln2_g": torch.zeros(C, dtype=torch.float32, device="cuda")},
                         torch.empty_like(x), saved)
    g = {k: torch.empty(v.shape, dtype=torch.float32, device="cuda") for k, v in prm.items()}
    with pytest.raises(TypeError, match="grad w2:"):
        N.swin_block_bwd(plan.handle, x, x, prm, saved, torch.empty_like(x), {**g, "w2": torch.empty(C, H, **bf)},
                         plan.alloc_bwd_ws())
    plan.close()

    gdesc = N.make_desc(1, (1, 24, 36), 64, 1, (1, 6, 6), (0, 0, 0), 4, N.SWIN_BF16)
    rp = N.RoutePlan(gdesc, N.make_rank_layout(0, 3), N.make_rank_layout(1, 4))
    local = torch.zeros(int(rp.src_sizes[0]), 64, **bf)
    with pytest.raises(ValueError, match="send:"):
        N.swin_route_pack(rp, 0, local, torch.empty(int(rp.src_sizes[0]) - 1, 64, **bf))
    with pytest.raises(ValueError, match="2 send"):
        N.swin_route_loopback(rp, [None, None], [None] * 4)
    torch.cuda.synchronize()
    rp.close()
