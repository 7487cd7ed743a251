"""GPU parity of the unfused reference sequences against the oracle's unfused forms."""
import numpy as np
import pytest
import torch

import memory_bound_decode_add_amd as F
import oracle as O
import synth
from helpers import assert_close, assert_bits_equal, say
from test_gpu_mlp import dev_layers

pytestmark = pytest.mark.gpu


def test_unfused_product_decode_shape():
    say("[unfused product] M=1 K=9216 N=2560")
    inp = synth.make("swiglu_w4_gemv_1x9216x2560")
    g, u = F.from_bits(inp.g), F.from_bits(inp.u)
    W = F.W4Weight.from_numpy(inp.W.qweight, inp.W.scales)
    assert F.unfused_gemv_workspace_bytes(F.UNFUSED_PRODUCT, 1, 9216, 2560) == 94_371_840
    y = F.to_bits(F.unfused_swiglu_w4_gemv(F.UNFUSED_PRODUCT, g, u, W, F.scalar(1.0)))
    torch.cuda.synchronize()
    assert_close(y, O.unfused_product_gemv(inp.g, inp.u, inp.W.qweight, inp.W.scales, 1.0), "product")
    # and against the fused definition
    assert_close(y, O.swiglu_w4_gemv(inp.g, inp.u, inp.W.qweight, inp.W.scales, 1.0), "product vs fused")


def bf16_add(a_bits, b_bits):
    """Exact reference of a bf16 + bf16 -> bf16 add (the sum is exact in fp64; one rounding)."""
    return O.f64_to_bf16(O.bf16_to_f64(a_bits) + O.bf16_to_f64(b_bits))


@pytest.mark.parametrize("M,K,N", [(1, 1024, 512), (4, 2048, 264)])
def test_unfused_act(M, K, N):
    """The unfused sequence rounds the GEMV output to bf16 before its separate residual
    add, so where that add cancels, a one-step difference in the rounded GEMV output
    (fp32 against fp64 summation order) exceeds the relative bound of the small sum.
    So the scaled GEMV output is compared with the oracle, and the residual add stage
    is checked exactly against the GPU's own scaled output."""
    say(f"[unfused act] M={M} K={K} N={N}")
    inp = synth.swiglu_gemv_inputs(M, K, N, seed=2, with_residual=True)
    g, u = F.from_bits(inp.g), F.from_bits(inp.u)
    W = F.W4Weight.from_numpy(inp.W.qweight, inp.W.scales)
    res = F.from_bits(inp.residual)
    y0 = F.to_bits(F.unfused_swiglu_w4_gemv(F.UNFUSED_ACT, g, u, W, F.scalar(0.5)))
    y1 = F.to_bits(F.unfused_swiglu_w4_gemv(F.UNFUSED_ACT, g, u, W, F.scalar(0.5), res))
    torch.cuda.synchronize()
    assert_close(y0, O.unfused_act_gemv(inp.g, inp.u, inp.W.qweight, inp.W.scales, 0.5), "act")
    assert_bits_equal(y1, bf16_add(y0, inp.residual), "residual add stage")


def test_unfused_product_residual_stage():
    say("[unfused product] residual add stage, M=1 K=1024 N=512")
    inp = synth.swiglu_gemv_inputs(1, 1024, 512, seed=6, with_residual=True)
    g, u = F.from_bits(inp.g), F.from_bits(inp.u)
    W = F.W4Weight.from_numpy(inp.W.qweight, inp.W.scales)
    y0 = F.to_bits(F.unfused_swiglu_w4_gemv(F.UNFUSED_PRODUCT, g, u, W, F.scalar(0.5)))
    y1 = F.to_bits(F.unfused_swiglu_w4_gemv(F.UNFUSED_PRODUCT, g, u, W, F.scalar(0.5), F.from_bits(inp.residual)))
    torch.cuda.synchronize()
    assert_close(y0, O.unfused_product_gemv(inp.g, inp.u, inp.W.qweight, inp.W.scales, 0.5), "product")
    assert_bits_equal(y1, bf16_add(y0, inp.residual), "residual add stage")


def test_unfused_add_rmsnorm():
    say("[unfused norm] M=256 H=4096")
    inp = synth.add_rmsnorm_inputs(256, 4096, seed=3)
    h, y = F.unfused_add_rmsnorm(F.from_bits(inp.x), F.from_bits(inp.r), F.from_bits(inp.w), inp.eps)
    torch.cuda.synchronize()
    rh, ry = O.add_rmsnorm_eager(inp.x, inp.r, inp.w, inp.eps)
    assert_bits_equal(F.to_bits(h), rh, "h")
    assert_close(F.to_bits(y), ry, "y")


def test_unfused_mlp_layer():
    """Stage by stage against the oracle's unfused forms, each fed the bf16 inputs the
    stage read; the residual add stage exactly (see test_unfused_act)."""
    say("[unfused mlp] M=4 H=512 I=1024")
    inp = synth.mlp_inputs(4, 512, 1024, n_layers=1, seed=4)
    L = inp.layers[0]
    outs = {}
    for resid in (False, True):
        layer = dev_layers(inp, resid)[0]
        b = F.MlpBuffers.empty(4, 512, 1024)
        b.x.copy_(F.from_bits(inp.x))
        b.residual.copy_(F.from_bits(inp.r))
        F.unfused_mlp_decode(layer, b)
        torch.cuda.synchronize()
        outs[resid] = {"h": F.to_bits(b.residual), "y": F.to_bits(b.y_norm), "gu": F.to_bits(b.gate_up),
                       "out": F.to_bits(b.out)}
    h, y = O.add_rmsnorm_eager(inp.x, inp.r, L.norm_w, L.eps)
    got = outs[False]
    assert_bits_equal(got["h"], h, "h")
    assert_close(got["y"], y, "y")
    gu = got["gu"]
    assert_close(gu, O.w4_gemv(got["y"], L.gate_up.qweight, L.gate_up.scales), "gu")
    out = O.unfused_act_gemv(gu[:, :1024], gu[:, 1024:], L.down.qweight, L.down.scales, L.out_scale)
    assert_close(got["out"], out, "out")
    for k in ("h", "y", "gu"):
        assert_bits_equal(outs[True][k], got[k], f"{k} with residual")
    assert_bits_equal(outs[True]["out"], bf16_add(got["out"], got["h"]), "residual add stage")
