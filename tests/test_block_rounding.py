"""Why the Swin block keeps its residual stream in fp32: a CPU model of the block's storage.

The two-block W-MSA -> SW-MSA chain at C = 512, hidden 2048 (36 x 48 tokens) is evaluated in
float64 with bf16 rounding applied exactly where a bf16-MFMA block must store values: the
layer-norm outputs LN1(x) and LN2(h) and the GELU activation (GEMM operands) and the output y,
once with the residual stream h = x + A(LN1(x)) also rounded to bf16 and once with h kept in
fp32. Against the unrounded oracle, with the block's bias scale (0.1 N(0,1), every bias of a
block) and with N(0,1) linear biases, the bf16-h model exceeds the per-token bar
2e-2 + ulp_bf16(ref)/2 about twofold while the fp32-h model stays within it (at N(0,1) biases
only just: 0.98 of the bar, from GEMM-operand rounding alone, which the block tests' inputs
therefore draw at the block's bias scale). Pins the design choice, not the GPU; the oracle's
arithmetic is unchanged (only its inputs to each stage are rounded here)."""
import numpy as np
import pytest

from oracle import block_oracle as BO
from oracle import swin_oracle as O
from oracle.chains import block_chain_full, block_params_of, layouts
from tests.bars import half_ulp_bf16
from workloads import BLOCK_BIAS_SCALE, bf16_bits_to_f64, get_config, make_block_extras, make_inputs, round_bf16
from workloads.configs import small_variant


def _r(a):
    return bf16_bits_to_f64(round_bf16(a))


def _worst_ratio(bias_scale, h_bf16):
    cfg = small_variant(get_config("highres"), grid=(1, 36, 48))
    inp = make_inputs(cfg, bias_scale=bias_scale)
    ex = make_block_extras(cfg)
    ref = block_chain_full(cfg, inp, ex, with_bwd=False)["y"]
    x = inp.x
    for p, lay in zip([block_params_of(m, e) for m, e in zip(inp.modules, ex)], layouts(cfg)):
        xn1 = _r(BO.layer_norm(x, p.ln1_g, p.ln1_b)[0])
        att, _ = O.module_fwd(xn1, p.attn, lay, cfg.heads)
        h = x + att
        if h_bf16:
            h = _r(h)
        xn2 = _r(BO.layer_norm(h, p.ln2_g, p.ln2_b)[0])
        g1 = _r(BO.gelu(xn2 @ p.w1.T + p.b1))
        x = _r(h + g1 @ p.w2.T + p.b2)
    return float((np.abs(x - ref) / (2e-2 + half_ulp_bf16(ref))).max())


@pytest.mark.parametrize("bias_scale", [BLOCK_BIAS_SCALE, 1.0])
def test_fp32_residual_stream_meets_the_bar_and_bf16_does_not(bias_scale):
    r32 = _worst_ratio(bias_scale, h_bf16=False)
    r16 = _worst_ratio(bias_scale, h_bf16=True)
    print("bias scale %.1f: worst |model - ref| / bar  h fp32 %.3f  h bf16 %.3f" % (bias_scale, r32, r16))
    assert r32 <= 1.0
    assert r16 > 1.5
