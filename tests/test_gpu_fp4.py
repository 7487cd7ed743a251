"""GPU parity of the FP4 (E2M1) weight GEMV with E4M3 1x16 block scales against the fp64
oracle, through the C ABI: the in-register decode bit for bit, the SwiGLU and identity
GEMVs within the tolerance, an exact case bit for bit."""
import numpy as np
import pytest
import torch

import memory_bound_decode_add_amd as F
import oracle as O
import synth
from helpers import assert_bits_equal, assert_close, say

pytestmark = pytest.mark.gpu
UNSUP = -6


def dev_w(W: synth.FP4):
    return F.FP4Weight.from_numpy(W.qweight, W.scales)


# ---------------------------------------------------------------------------
# decode: bit-exact
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("K,N", [(1024, 512), (9216, 2560), (96, 8)])
def test_fp4_dequant_bit_exact(K, N):
    say(f"[fp4 dequant] K={K} N={N}")
    W = synth.fp4_weight(np.random.default_rng(K + N), K, N)
    w = F.fp4_dequant(dev_w(W)).cpu().numpy()
    want = O.fp4_dequant(W.qweight, W.scales).astype(np.float32)
    assert_bits_equal(w.view(np.uint32), want.view(np.uint32), "fp4 dequant")


def test_fp4_dequant_every_scale_code():
    say("[fp4 dequant] every E4M3 scale code (NaN codes replaced by 0) x every E2M1 code")
    K, N = 256, 16                                  # 16 x 16 = 256 block scales
    codes = np.arange(256, dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0
    sc = codes.reshape(N, K // 16)
    rng = np.random.default_rng(4)
    W = synth.FP4(rng.integers(0, 2**32, size=(N, K // 8), dtype=np.uint32), sc)
    w = F.fp4_dequant(dev_w(W)).cpu().numpy()
    want = O.fp4_dequant(W.qweight, W.scales).astype(np.float32)
    assert_bits_equal(w.view(np.uint32), want.view(np.uint32), "fp4 dequant, all scale codes")
    assert set(O.fp4_unpack(W.qweight).ravel().tolist()) == set(range(16))


# ---------------------------------------------------------------------------
# the GEMV: tolerance
# ---------------------------------------------------------------------------
def run(inp, out_scale, residual, swiglu=True):
    g, u = F.from_bits(inp.g), F.from_bits(inp.u)
    W = dev_w(inp.W)
    s = None if out_scale is None else F.scalar(out_scale)
    res = F.from_bits(inp.residual) if residual else None
    y = F.swiglu_fp4_gemv(g, u, W, s, res) if swiglu else F.fp4_gemv(g, W, s, res)
    torch.cuda.synchronize()
    return F.to_bits(y)


def want(inp, out_scale, residual, swiglu=True):
    res = inp.residual if residual else None
    if swiglu:
        return O.swiglu_fp4_gemv(inp.g, inp.u, inp.W.qweight, inp.W.scales, out_scale, res)
    return O.fp4_gemv(inp.g, inp.W.qweight, inp.W.scales, out_scale, res)


def test_fp4_gemv_decode_shape():
    say("[fp4 gemv] M=1 K=9216 N=2560 (the int4 metric's shape), out_scale 1.0")
    inp = synth.swiglu_fp4_gemv_inputs(1, 9216, 2560, seed=0, out_scale=1.0)
    say("  worst err/bound", assert_close(run(inp, 1.0, False), want(inp, 1.0, False), "y"))


@pytest.mark.parametrize("M,K,N", [(1, 1024, 512), (1, 32, 8), (2, 2080, 264), (3, 16384, 40), (4, 4096, 1000),
                                   (4, 96, 24), (2, 9216, 2560), (1, 1536, 17920)])
def test_fp4_gemv_shapes(M, K, N):
    say(f"[fp4 gemv] M={M} K={K} N={N}")
    inp = synth.swiglu_fp4_gemv_inputs(M, K, N, seed=M * 7 + K + N, out_scale=0.5, with_residual=True)
    for resid in (True, False):
        w = assert_close(run(inp, 0.5, resid), want(inp, 0.5, resid), f"y resid={resid}")
        say(f"  residual={resid}: worst err/bound {w:.3f}")
    assert_close(run(inp, None, False), want(inp, None, False), "y, NULL scale")
    assert_close(run(inp, 0.5, True, swiglu=False), want(inp, 0.5, True, swiglu=False), "identity prologue")


def test_fp4_gemv_exact_case_and_repeatability():
    say("[fp4 gemv] integer activations, power-of-two scales: bit-exact")
    rng = np.random.default_rng(12)
    M, K, N = 3, 4096, 520
    x = synth.f32_to_bf16_bits(rng.integers(-3, 4, size=(M, K)).astype(np.float32))
    sc = rng.choice(np.array([0x20, 0x28, 0x30], dtype=np.uint8), size=(N, K // 16))   # 2^-3, 2^-2, 2^-1
    W = synth.FP4(rng.integers(0, 2**32, size=(N, K // 8), dtype=np.uint32), sc)
    xd, Wd, s = F.from_bits(x), dev_w(W), F.scalar(0.5)
    y1 = F.fp4_gemv(xd, Wd, s)
    y2 = F.fp4_gemv(xd, Wd, s)
    torch.cuda.synchronize()
    assert_bits_equal(F.to_bits(y1), O.fp4_gemv(x, W.qweight, W.scales, 0.5), "exact case")
    assert_bits_equal(F.to_bits(y1), F.to_bits(y2), "repeat")


def test_fp4_gemv_rejects_what_it_cannot_do():
    inp = synth.swiglu_fp4_gemv_inputs(5, 96, 64, seed=1)          # 5..16 rows need K % 128 == 0
    g, u, W = F.from_bits(inp.g), F.from_bits(inp.u), dev_w(inp.W)
    with pytest.raises(F.FdecError) as e:
        F.swiglu_fp4_gemv(g, u, W)
    assert e.value.status == UNSUP
    inp = synth.swiglu_fp4_gemv_inputs(1, 16416, 8, seed=1)
    with pytest.raises(F.FdecError) as e:
        F.swiglu_fp4_gemv(F.from_bits(inp.g), F.from_bits(inp.u), dev_w(inp.W))
    assert e.value.status == UNSUP



# ---------------------------------------------------------------------------
# 5..64 rows: the matrix-core kernel with FP4 weights (two or four 16-row blocks
# per weight load past 16 rows)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("M,K,N", [(16, 14336, 4096), (16, 9216, 2560), (8, 4096, 1000), (5, 256, 24),
                                   (12, 1024, 512), (16, 4096, 28672), (17, 1024, 512), (32, 9216, 2560),
                                   (40, 256, 24), (64, 4096, 1000)])
def test_fp4_gemv_matrix_core_shapes(M, K, N):
    say(f"[fp4 gemv, matrix cores] M={M} K={K} N={N}")
    inp = synth.swiglu_fp4_gemv_inputs(M, K, N, seed=M * 5 + K + N, out_scale=0.5, with_residual=True)
    w = assert_close(run(inp, 0.5, True), want(inp, 0.5, True), "y with residual")
    say(f"  worst err/bound {w:.3f}")
    assert_close(run(inp, None, False), want(inp, None, False), "y, NULL scale")
    if K <= 4096:
        assert_close(run(inp, 0.5, False, swiglu=False), want(inp, 0.5, False, swiglu=False), "identity prologue")


@pytest.mark.parametrize("M", [16, 64])
def test_fp4_gemv_matrix_core_exact_case(M):
    say(f"[fp4 gemv, matrix cores] integer activations, power-of-two scales, M={M}: bit-exact")
    rng = np.random.default_rng(13)
    K, N = 9216, 264
    x = synth.f32_to_bf16_bits(rng.integers(-3, 4, size=(M, K)).astype(np.float32))
    sc = rng.choice(np.array([0x20, 0x28, 0x30], dtype=np.uint8), size=(N, K // 16))   # 2^-3, 2^-2, 2^-1
    W = synth.FP4(rng.integers(0, 2**32, size=(N, K // 8), dtype=np.uint32), sc)
    xd, Wd, s = F.from_bits(x), dev_w(W), F.scalar(0.5)
    y1 = F.fp4_gemv(xd, Wd, s)
    y2 = F.fp4_gemv(xd, Wd, s)
    torch.cuda.synchronize()
    assert_bits_equal(F.to_bits(y1), O.fp4_gemv(x, W.qweight, W.scales, 0.5), "exact case")
    assert_bits_equal(F.to_bits(y1), F.to_bits(y2), "repeat")


@pytest.mark.parametrize("M,K,N", [(3, 1536, 264), (8, 1024, 512)])
def test_fp4_gemv_strided_gate_up_halves(M, K, N):
    """g and u as the two halves of one [M, 2K] gate_up output (row stride 2K), on the
    chunk-owning kernel (M = 3) and the matrix-core kernel (M = 8)."""
    say(f"[fp4 gemv] strided g/u, M={M} K={K} N={N}")
    inp = synth.swiglu_fp4_gemv_inputs(M, K, N, seed=91 + M, out_scale=0.5)
    gu = torch.cat([F.from_bits(inp.g), F.from_bits(inp.u)], dim=1)      # [M, 2K]
    y = F.swiglu_fp4_gemv(gu[:, :K], gu[:, K:], dev_w(inp.W), F.scalar(0.5))
    torch.cuda.synchronize()
    assert_close(F.to_bits(y), want(inp, 0.5, False), "y")
