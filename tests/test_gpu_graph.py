"""Module calls captured in a HIP graph (torch's graph API over the library's stream) and
replayed: a W-MSA -> SW-MSA chain forward and backward (bf16, C = 512) and the fp32 forward.
None of the calls records a memset or a host copy, and every kernel is deterministic, so each
replay must reproduce the eager results bitwise. Between replays the program clobbers the
outputs with eager work of its own and synchronises."""
import numpy as np
import pytest

from tests.gpu_util import ModuleOnDevice, log, to_dev
from workloads import get_config, make_inputs
from workloads.configs import small_variant

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from shifted_window_attention_amd import native  # noqa: F401  (raises if the library is missing)


def _chain(cfg):
    import torch
    from shifted_window_attention_amd import native as N
    inp = make_inputs(cfg)
    mods = [ModuleOnDevice(cfg, i, p) for i, p in enumerate(inp.modules)]
    x = to_dev(inp.x_dev, cfg.dtype)
    dy = to_dev(inp.dy_dev, cfg.dtype) if cfg.backward else None
    C = cfg.channels
    ys = [torch.empty_like(x) for _ in mods]
    dxs = [torch.empty_like(x) for _ in mods] if cfg.backward else []
    grads = [[torch.empty(3 * C, C, device="cuda"), torch.empty(3 * C, device="cuda"), torch.empty(C, C, device="cuda"),
              torch.empty(C, device="cuda"), torch.empty_like(m.table)] for m in mods] if cfg.backward else []

    def call(stream):
        xin = x
        for m, y in zip(mods, ys):
            N.swin_attn_fwd(m.plan.handle, xin, m.w_qkv, m.b_qkv, m.w_proj, m.b_proj, m.table, y, m.saved,
                            stream=stream)
            xin = y
        d = dy
        for i in reversed(range(len(dxs))):
            m, g = mods[i], grads[i]
            N.swin_attn_bwd(m.plan.handle, d, x if i == 0 else ys[i - 1], m.w_qkv, m.w_proj, m.table, m.saved,
                            dxs[i], g[0], g[1], g[2], g[3], g[4], m.ws, stream=stream)
            d = dxs[i]

    outs = ys + dxs + [t for g in grads for t in g]
    return call, outs


@pytest.mark.parametrize("name", ["highres_small", "tiny"])
def test_graph_replay_matches_eager(name):
    import torch
    cfg = small_variant(get_config("highres"), grid=(1, 24, 36)) if name == "highres_small" else get_config(name)
    call, outs = _chain(cfg)
    main = torch.cuda.current_stream()
    call(main)
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    side = torch.cuda.Stream()
    side.wait_stream(main)
    with torch.cuda.stream(side):
        call(side)
    main.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        call(side)
    torch.cuda.synchronize()
    for r in range(3):
        for t in outs:
            t.fill_(float("nan") if t.is_floating_point() else 0)
        call(main)  # eager work between replays
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        bad = [i for i, (a, b) in enumerate(zip(outs, ref)) if not torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                                                                                 b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))]
        log("graph replay %d of %s: %d of %d outputs differ from the eager call" % (r, name, len(bad), len(outs)))
        assert not bad, bad
