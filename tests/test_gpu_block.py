"""Parity of the Swin block (layer norms, attention module, GELU MLP, residuals) with the
fp64 block oracle, through the C ABI of include/swin_block.h.

Bars (tests/bars.py), as for the attention module: per-token outputs (y, dx) |got - ref| <=
2e-2 + ulp_bf16(ref)/2 element-wise; reduced gradients 2e-2 * max(1, |ref|_inf). The block keeps
its residual stream h (and its gradient) in fp32; tests/test_block_rounding.py shows on the CPU
that this is what brings the block's bf16 storage within the per-token bar."""
import numpy as np
import pytest

from tests.bars import reduced_excess, token_excess
from tests.gpu_util import log, run_block_chain
from tests.oracle_runner import block_chain_full
from workloads import BLOCK_BIAS_SCALE, get_config, make_block_extras, make_inputs
from workloads.configs import small_variant

pytestmark = pytest.mark.gpu

GRAD_KEYS = ("ln1_g", "ln1_b", "w_qkv", "b_qkv", "w_proj", "b_proj", "table", "ln2_g", "ln2_b", "w1", "b1", "w2",
             "b2")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from shifted_window_attention_amd import native  # noqa: F401  (raises if the library is missing)


def _check_tokens(got, ref, label):
    ex, err = token_excess(got, ref)
    log("  %s max-abs %.3e (|ref| %.3e), worst excess over the bar %.3e" %
        (label, err, float(np.abs(np.asarray(ref)).max()), ex))
    assert ex <= 0, label


def _check_grads(got, ref, label):
    for i, (gm, rm) in enumerate(zip(got, ref)):
        for k in GRAD_KEYS:
            ex, err = reduced_excess(gm[k], rm[k])
            log("  %s block %d d%s max-abs %.3e, worst excess over the bar %.3e" % (label, i, k, err, ex))
            assert ex <= 0, (label, i, k, err, ex)


BLOCK_CASES = [
    # W-MSA then SW-MSA blocks, C = 512, hidden 2048: the two-block pair on a reduced grid
    ("highres", dict(grid=(1, 36, 48)), None),
    # ragged edge windows and a token count that is not a multiple of the 256-row GEMM tile
    ("ragged", dict(grid=(1, 41, 57)), None),
    # hidden width 192 (partial 128-column tile in the GELU epilogue), batch 2
    ("om4", dict(grid=(1, 18, 36), batch=2, channels=64, heads=2), 192),
    # 3-D windows masked on level and lat
    ("levels3d", dict(grid=(4, 18, 36)), None),
    # C = 1024 (two 8-channel chunks per lane in the layer-norm kernels), 32 heads
    ("om4", dict(grid=(1, 12, 24), channels=1024, heads=32), 256),
    # head_dim 64 (the tiled attention kernels inside the block)
    ("highres", dict(grid=(1, 24, 36), channels=256, heads=4), None),
]


def _ids(v):
    if isinstance(v, dict):
        return "x".join(map(str, v["grid"])) + ("_c%d_h%d" % (v["channels"], v["heads"]) if "channels" in v else "")
    return str(v)


def test_block_with_large_windows():
    """A W->SW block pair with 16 x 16 windows (256 tokens: the tiled backward inside the block)."""
    from workloads.configs import SwinConfig
    cfg = SwinConfig(name="block_w16", batch=1, grid=(1, 32, 48), channels=128, heads=4, window=(1, 16, 16),
                     shifts=((0, 0, 0), (0, 8, 8)), dtype="bf16", backward=True, periodic=4, description="block_w16")
    log("block fwd+bwd with 256-token windows", cfg.grid)
    inp = make_inputs(cfg, bias_scale=BLOCK_BIAS_SCALE)
    extras = make_block_extras(cfg)
    got = run_block_chain(cfg, inp, extras)
    ref = block_chain_full(cfg, inp, extras)
    _check_tokens(got["y"], ref["y"], "y")
    _check_tokens(got["dx"], ref["dx"], "dx")
    _check_grads(got["grads"], ref["grads"], cfg.name)
    from shifted_window_attention_amd import native as N
    for b in got["blocks"]:
        assert N.swin_block_plan_flags(b.plan.handle) == 0   # dT stayed inside the fixed-point range


@pytest.mark.parametrize("name,kw,hidden", BLOCK_CASES, ids=_ids)
def test_block_chain_vs_oracle(name, kw, hidden):
    cfg = small_variant(get_config(name), **kw)
    log("block fwd+bwd", name, cfg.grid, "batch", cfg.batch, "C", cfg.channels, "hidden", hidden or 4 * cfg.channels)
    inp = make_inputs(cfg, bias_scale=BLOCK_BIAS_SCALE)
    extras = make_block_extras(cfg, hidden=hidden)
    got = run_block_chain(cfg, inp, extras)
    ref = block_chain_full(cfg, inp, extras)
    _check_tokens(got["y"], ref["y"], "y")
    _check_tokens(got["dx"], ref["dx"], "dx")
    _check_grads(got["grads"], ref["grads"], name)


def test_block_backward_is_deterministic():
    import torch
    cfg = small_variant(get_config("ragged"), grid=(1, 41, 57))
    inp = make_inputs(cfg, bias_scale=BLOCK_BIAS_SCALE)
    extras = make_block_extras(cfg)
    got = run_block_chain(cfg, inp, extras)
    b = got["blocks"][0]
    from tests.gpu_util import to_dev
    x = to_dev(inp.x_dev, "bf16")
    dy = to_dev(inp.dy_dev, "bf16")
    b.fwd(x)
    dx1, g1 = b.bwd(dy, x)
    dx2, g2 = b.bwd(dy, x)
    torch.cuda.synchronize()
    assert torch.equal(dx1.view(torch.int16), dx2.view(torch.int16))
    for k in g1:
        assert torch.equal(g1[k], g2[k]), k


def test_block_rejects_bad_calls():
    import torch
    from shifted_window_attention_amd import native as N
    cfg = small_variant(get_config("om4"), grid=(1, 12, 24), batch=1, channels=64, heads=2)
    inp = make_inputs(cfg, bias_scale=BLOCK_BIAS_SCALE)
    extras = make_block_extras(cfg)
    got = run_block_chain(cfg, inp, extras, with_bwd=False)
    b = got["blocks"][0]
    x = torch.zeros(cfg.n_tokens, cfg.channels, dtype=torch.bfloat16, device="cuda")
    # y aliasing x
    with pytest.raises(N.SwinError) as e:
        N.swin_block_fwd(b.plan.handle, x, b.params, x, b.saved)
    assert e.value.status == 1
    # a missing required parameter
    with pytest.raises(N.SwinError) as e:
        N.swin_block_fwd(b.plan.handle, x, {**b.params, "w1": None}, torch.empty_like(x), b.saved)
    assert e.value.status == 1
    # inference call without saved and without a workspace
    with pytest.raises(N.SwinError) as e:
        N.swin_block_fwd(b.plan.handle, x, b.params, torch.empty_like(x), None)
    assert e.value.status == 3
    # backward workspace one byte short
    g = b.grad_buffers()
    short = torch.empty(b.plan.bwd_ws - 1, dtype=torch.uint8, device="cuda")
    with pytest.raises(N.SwinError) as e:
        N.swin_block_bwd(b.plan.handle, x, x, b.params, b.saved, torch.empty_like(x), g, short)
    assert e.value.status == 3
    torch.cuda.synchronize()


def test_block_inference_call_matches_training_forward():
    """saved = NULL with a workspace of saved_bytes gives the same y as the training forward."""
    import torch
    from shifted_window_attention_amd import native as N
    cfg = small_variant(get_config("highres"), grid=(1, 24, 36))
    inp = make_inputs(cfg, bias_scale=BLOCK_BIAS_SCALE)
    extras = make_block_extras(cfg)
    got = run_block_chain(cfg, inp, extras, with_bwd=False)
    b = got["blocks"][0]
    from tests.gpu_util import to_dev
    x = to_dev(inp.x_dev, "bf16")
    y1 = b.fwd(x)
    y2 = torch.empty_like(x)
    ws = b.plan.alloc_saved()
    N.swin_block_fwd(b.plan.handle, x, b.params, y2, None, ws)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
