"""GPU parity of the prefill-size path (2,048 tokens at K = 9216, N = 2560): the fused SwiGLU
elementwise pass and the matrix-core W4 GEMM, against the fp64 oracle."""
import numpy as np
import pytest
import torch

import memory_bound_decode_add_amd as F
import oracle as O
import synth
from helpers import assert_bits_equal, assert_close, say

pytestmark = pytest.mark.gpu


def check_act(got, ref, what):
    """One rounding on both sides; the fp32 SiLU may land on the other side of a bf16
    rounding boundary where the fp64 one is within a few fp32 ulps of it."""
    g, r = O.bf16_to_f64(got), O.bf16_to_f64(ref)
    mism = g != r
    assert mism.mean() < 1e-3, f"{what}: {mism.mean():.2e} of the values differ"
    assert np.all(np.abs(g - r)[mism] <= np.abs(r[mism]) * 2.0 ** -7), f"{what}: more than one bf16 step"


@pytest.mark.parametrize("M,K,ld", [(3, 8, 8), (5, 1024, 1032), (2048, 9216, 9216)])
def test_swiglu_pass(M, K, ld):
    say(f"[swiglu pass] M={M} K={K} ld={ld}")
    rng = np.random.default_rng(M + K)
    gu = synth.f32_to_bf16_bits(rng.standard_normal((M, 2 * ld)).astype(np.float32))
    gd = F.from_bits(gu)
    g, u = gd[:, :K], gd[:, ld:ld + K]
    act = F.to_bits(F.swiglu(g, u))
    check_act(act, O.swiglu_act(gu[:, :K], gu[:, ld:ld + K]), "act")


@pytest.mark.parametrize("M,K,N", [(1, 128, 8), (130, 384, 168), (300, 1024, 520), (257, 4096, 2560)])
def test_w4_gemm_shapes_with_residual(M, K, N):
    say(f"[gemm] M={M} K={K} N={N}")
    inp = synth.swiglu_gemv_inputs(M, K, N, seed=M + K + N, out_scale=0.5, with_residual=True)
    W = F.W4Weight.from_numpy(inp.W.qweight, inp.W.scales)
    x, res = F.from_bits(inp.g), F.from_bits(inp.residual)
    y = F.to_bits(F.w4_gemm(x, W, F.scalar(0.5), res))
    ref = O.w4_gemm(inp.g, inp.W.qweight, inp.W.scales, 0.5, inp.residual)
    say("  worst err/bound", assert_close(y, ref, "y"))
    # no residual, NULL scale; and y in place of the residual
    y2 = F.to_bits(F.w4_gemm(x, W))
    assert_close(y2, O.w4_gemm(inp.g, inp.W.qweight, inp.W.scales), "y, no scale")
    F.w4_gemm(x, W, F.scalar(0.5), res, out=res)
    torch.cuda.synchronize()
    assert_bits_equal(F.to_bits(res), y, "in place")


def test_w4_gemm_exact_case_bit_exact():
    # small-integer activations, power-of-two scales: every product and partial sum is an
    # exact fp32 value, so any summation order gives the oracle's result bit for bit
    M, K, N = 200, 2048, 328
    rng = np.random.default_rng(9)
    x = synth.f32_to_bf16_bits(rng.integers(-4, 5, size=(M, K)).astype(np.float32))
    q = rng.integers(-8, 8, size=(K, N))
    s = synth.f32_to_bf16_bits(rng.choice([2.0 ** -6, 2.0 ** -7], size=(K // 128, N)).astype(np.float32))
    qw = synth.pack_int4(q)
    W = F.W4Weight.from_numpy(qw, s)
    y = F.to_bits(F.w4_gemm(F.from_bits(x), W, F.scalar(0.5)))
    assert_bits_equal(y, O.w4_gemm(x, qw, s, 0.5), "exact case")


def test_prefill_2048_tokens_swiglu_gemm():
    M, K, N = 2048, 9216, 2560
    say(f"[prefill] M={M} K={K} N={N}: SwiGLU pass, then the GEMM")
    inp = synth.swiglu_gemv_inputs(M, K, N, seed=2048, out_scale=1.0)
    W = F.W4Weight.from_numpy(inp.W.qweight, inp.W.scales)
    g, u = F.from_bits(inp.g), F.from_bits(inp.u)
    ws = F.workspace(F.swiglu_w4_gemm_workspace_bytes(M, K))
    y = F.to_bits(F.swiglu_w4_gemm(g, u, W, F.scalar(1.0), ws=ws))
    act = F.to_bits(ws[: M * K * 2].view(torch.int16).view(torch.bfloat16).reshape(M, K))
    check_act(act, O.swiglu_act(inp.g, inp.u), "act")
    ref = O.w4_gemm(act, inp.W.qweight, inp.W.scales, 1.0)
    say("  worst err/bound", assert_close(y, ref, "y"))
    y2 = F.to_bits(F.swiglu_w4_gemm(g, u, W, F.scalar(1.0), ws=ws))
    assert_bits_equal(y2, y, "repeat")
