"""GPU parity of the matrix-core GEMV fed by direct-to-LDS loads of every operand (5..16
rows; selected with fdec_set_mfma_plan(3)) against the fp64 oracle, through the C ABI:
both prologues, ragged K slices and column tiles, several slices summed by the finish
kernels over a NaN-filled workspace, the pair-mode gate_up with the SwiGLU epilogue, and
the 16-row layer built on them."""
import numpy as np
import pytest
import torch

import memory_bound_decode_add_amd as F
import oracle as O
import synth
from helpers import assert_bits_equal, assert_close, say
from test_gpu_mlp import dev_layers
from test_gpu_mlp2 import check_layer2_mc

pytestmark = pytest.mark.gpu
BIG_WS = 64 << 20          # every plan here needs less


@pytest.fixture
def ring():
    F.set_mfma_plan(3)
    try:
        yield
    finally:
        F.set_mfma_plan(0)


def nan_ws(nbytes=BIG_WS):
    return torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")


# M, K, N: K = 4224 is 33 groups (odd slices, a step whose second group is past the end);
# N = 1000 and 264 end in a partial tile, 520 in a partial column range; 9216 x 2560 is
# the metric's shape at 16 rows (12 slices); 14336 x 4096 the 16-row layer's down (8).
SHAPES = [(5, 4224, 1000), (8, 1024, 264), (12, 4224, 520), (16, 9216, 2560), (16, 14336, 4096), (16, 256, 128),
          (7, 128, 1032), (16, 4096, 28672), (1, 2048, 776), (3, 4224, 264)]   # forced below 5 rows too


@pytest.mark.parametrize("M,K,N", SHAPES)
def test_ring_swiglu_gemv(ring, M, K, N):
    say(f"[ring] SwiGLU M={M} K={K} N={N}")
    inp = synth.swiglu_gemv_inputs(M, K, N, seed=M * 7 + K + N, out_scale=0.5, with_residual=True)
    g, u, W, res = F.from_bits(inp.g), F.from_bits(inp.u), F.W4Weight.from_numpy(inp.W.qweight, inp.W.scales), \
        F.from_bits(inp.residual)
    ws = nan_ws()
    y = F.to_bits(F.swiglu_w4_gemv(g, u, W, F.scalar(0.5), res, ws=ws))
    ref = O.swiglu_w4_gemv(inp.g, inp.u, inp.W.qweight, inp.W.scales, 0.5, inp.residual)
    say("  worst err/bound", assert_close(y, ref, "y"))
    assert_bits_equal(F.to_bits(F.swiglu_w4_gemv(g, u, W, F.scalar(0.5), res, ws=ws)), y, "repeat")


@pytest.mark.parametrize("M,K,N", SHAPES)
def test_ring_identity_gemv(ring, M, K, N):
    say(f"[ring] identity M={M} K={K} N={N}")
    inp = synth.swiglu_gemv_inputs(M, K, N, seed=M * 11 + K + N)
    x, W = F.from_bits(inp.g), F.W4Weight.from_numpy(inp.W.qweight, inp.W.scales)
    ws = nan_ws()
    for s in (None, 0.25):
        y = F.to_bits(F.w4_gemv(x, W, None if s is None else F.scalar(s), ws=ws))
        want = O.w4_gemv(inp.g, inp.W.qweight, inp.W.scales, s)
        say(f"  out_scale={s} worst err/bound", assert_close(y, want, "y"))
    # the residual epilogue of the identity prologue runs in the layer's down projection
    # (test_ring_layer_matrix_core)


def test_ring_strided_gate_up_halves(ring):
    say("[ring] SwiGLU prologue on the two halves of one [12, 2K] gate_up output")
    M, K, N = 12, 2048, 776
    inp = synth.swiglu_gemv_inputs(M, K, N, seed=5)
    gu = F.from_bits(np.concatenate([inp.g, inp.u], axis=1))
    W = F.W4Weight.from_numpy(inp.W.qweight, inp.W.scales)
    y = F.to_bits(F.swiglu_w4_gemv(gu[:, :K], gu[:, K:], W, None, None, ws=nan_ws()))
    say("  worst err/bound", assert_close(y, O.swiglu_w4_gemv(inp.g, inp.u, inp.W.qweight, inp.W.scales), "y"))


@pytest.mark.parametrize("M,K,I", [(16, 4096, 14336), (5, 1024, 520), (8, 9216, 1032), (16, 14336, 2048),
                                   (12, 4224, 264)])
def test_ring_pair_gate_up_swiglu(ring, M, K, I):
    say(f"[ring] pair-mode gate_up + SwiGLU M={M} K={K} I={I}")
    inp = synth.swiglu_gemv_inputs(M, K, 2 * I, seed=M * 31 + K + I)
    W = F.W4Weight.from_numpy(inp.W.qweight, inp.W.scales)
    x = F.from_bits(inp.g)
    ws = nan_ws()
    act = F.to_bits(F.w4_gemv_swiglu(x, W, ws=ws))
    say("  worst err/bound", assert_close(act, O.w4_gemv_swiglu(inp.g, inp.W.qweight, inp.W.scales), "act"))
    assert_bits_equal(F.to_bits(F.w4_gemv_swiglu(x, W, ws=ws)), act, "repeat")


@pytest.mark.parametrize("M,H,I", [(16, 4096, 14336), (8, 1024, 2048), (5, 512, 640)])
def test_ring_layer_matrix_core(ring, M, H, I):
    say(f"[ring] two-projection layer M={M} H={H} I={I}")
    inp = synth.mlp_inputs(M, H, I, n_layers=1, seed=M + H + I + 9)
    for resid in (True, False):
        layer = dev_layers(inp, resid)[0]
        b = F.Mlp2Buffers.empty(M, H, I)
        b.x.copy_(F.from_bits(inp.x))
        b.residual.copy_(F.from_bits(inp.r))
        ws = nan_ws()
        F.mlp_decode2(layer, b, ws)
        torch.cuda.synchronize()
        y = ws[: M * H * 2].view(torch.int16).view(torch.bfloat16).reshape(M, H)
        got = {"h": F.to_bits(b.residual), "y": F.to_bits(y), "act": F.to_bits(b.act), "out": F.to_bits(b.out)}
        say(f"  resid={resid} worst err/bound (y, act, out)", check_layer2_mc(inp.layers[0], inp.x, inp.r, got, resid))
