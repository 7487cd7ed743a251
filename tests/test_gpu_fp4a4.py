"""GPU parity of the GEMVs with both operands FP4 (the activation quantised at run time
with E4M3 1x16 block scales and a per-tensor scale) against the fp64 oracle, through the
C ABI: the quantiser bit for bit, the GEMVs within the tolerance and an exact case bit
for bit."""
import numpy as np
import pytest
import torch

import memory_bound_decode_add_amd as F
import oracle as O
import synth
from helpers import assert_bits_equal, assert_close, say

pytestmark = pytest.mark.gpu


def pack_codes(codes):
    """E2M1 codes [M, K] -> words [M, K/8] (code of k = 8 kb + j in bits [4j, 4j+4))."""
    c = codes.astype(np.uint32).reshape(codes.shape[0], -1, 8)
    return np.bitwise_or.reduce(c << (4 * np.arange(8, dtype=np.uint32)), axis=-1)


def calibrated(act64):
    """The per-tensor scale a calibration would pick: the largest magnitude over 6 * 448."""
    return np.float32(np.abs(act64).max() / (6.0 * 448.0))


def dev_w(W: synth.FP4):
    return F.FP4Weight.from_numpy(W.qweight, W.scales)


# ---------------------------------------------------------------------------
# the quantiser: bit-exact (the identity prologue: both sides quantise the same fp32 values)
# ---------------------------------------------------------------------------
def spread_bf16(rng, M, K):
    """bf16 values whose magnitudes span 2^-14 .. 2^6, so that block scales reach the E4M3
    subnormals, zero and the top of the range."""
    x = rng.standard_normal((M, K)) * np.exp2(rng.uniform(-14, 6, size=(M, K // 16, 1))).repeat(16, -1).reshape(M, K)
    return synth.f32_to_bf16_bits(x.astype(np.float32))


@pytest.mark.parametrize("M,K,case", [(1, 32, "normal"), (3, 9216, "normal"), (16, 4096, "spread"),
                                      (5, 14336, "spread"), (2, 1024, "saturated"), (4, 2048, "tiny")])
def test_quantize_bit_exact(M, K, case):
    say(f"[fp4 quantize] M={M} K={K} {case}")
    rng = np.random.default_rng(M * 31 + K)
    x = spread_bf16(rng, M, K) if case == "spread" else synth.f32_to_bf16_bits(
        (rng.standard_normal((M, K)) * 3).astype(np.float32))
    G = calibrated(O.bf16_to_f64(x))
    if case == "saturated":
        G = np.float32(G / 1000)        # block scales beyond 448: they saturate, and so do the codes
    if case == "tiny":
        G = np.float32(G * 1e4)         # block scales below E4M3's range: zero blocks
    codes, sc = F.nvfp4_quantize(F.from_bits(x), F.scalar(float(G)))
    want_c, want_s = O.nvfp4_quantize(O.bf16_to_f64(x).astype(np.float32), G)
    assert_bits_equal(sc.cpu().numpy(), want_s, "scale codes")
    assert_bits_equal(codes.cpu().numpy().view(np.uint32), pack_codes(want_c), "codes")
    say(f"  scale codes {int(want_s.min())}..{int(want_s.max())}, zero blocks {int((want_s == 0).sum())}")


def test_quantize_strided_rows():
    say("[fp4 quantize] strided rows (the second half of a [4, 2K] tensor)")
    rng = np.random.default_rng(8)
    K = 1024
    x = synth.f32_to_bf16_bits(rng.standard_normal((4, 2 * K)).astype(np.float32))
    G = calibrated(O.bf16_to_f64(x))
    codes, sc = F.nvfp4_quantize(F.from_bits(x)[:, K:], F.scalar(float(G)))
    want_c, want_s = O.nvfp4_quantize(O.bf16_to_f64(x[:, K:]).astype(np.float32), G)
    assert_bits_equal(sc.cpu().numpy(), want_s, "scale codes")
    assert_bits_equal(codes.cpu().numpy().view(np.uint32), pack_codes(want_c), "codes")


# ---------------------------------------------------------------------------
# the GEMVs: tolerance (the same tolerance as every GEMV here)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("M,K,N", [(1, 9216, 2560), (2, 1024, 520), (3, 4096, 1000), (4, 96, 24), (5, 1024, 264),
                                   (8, 9216, 2560), (16, 14336, 4096), (32, 2048, 776), (64, 9216, 2560)])
def test_fp4a4_gemv_identity(M, K, N):
    say(f"[fp4a4 gemv] identity M={M} K={K} N={N}")
    inp = synth.swiglu_fp4_gemv_inputs(M, K, N, seed=M + K + N, out_scale=0.5, with_residual=True)
    G = calibrated(O.bf16_to_f64(inp.g))
    x, W = F.from_bits(inp.g), dev_w(inp.W)
    ws = F.workspace(max(1, F.fp4_gemv_workspace_bytes(M, K, N)))
    for resid in (False, True):
        res = inp.residual if resid else None
        y = F.fp4a4_gemv(x, W, F.scalar(float(G)), F.scalar(0.5), F.from_bits(res) if resid else None, ws=ws)
        want = O.fp4a4_gemv(inp.g, inp.W.qweight, inp.W.scales, G, 0.5, res)
        say(f"  residual={resid}: worst err/bound", assert_close(F.to_bits(y), want, "y"))


@pytest.mark.parametrize("M,K,N", [(1, 9216, 2560), (1, 8960, 1536), (4, 2048, 264), (16, 9216, 2560),
                                   (64, 4096, 520)])
def test_swiglu_fp4a4_gemv(M, K, N):
    say(f"[fp4a4 gemv] SwiGLU M={M} K={K} N={N}")
    inp = synth.swiglu_fp4_gemv_inputs(M, K, N, seed=M * 3 + K + N, out_scale=1.0)
    act = O.silu_mul(O.bf16_to_f64(inp.g), O.bf16_to_f64(inp.u))
    G = calibrated(act)
    ws = F.workspace(max(1, F.fp4_gemv_workspace_bytes(M, K, N)))
    y = F.swiglu_fp4a4_gemv(F.from_bits(inp.g), F.from_bits(inp.u), dev_w(inp.W), F.scalar(float(G)), None, ws=ws)
    want = O.swiglu_fp4a4_gemv(inp.g, inp.u, inp.W.qweight, inp.W.scales, G, None)
    say("  worst err/bound", assert_close(F.to_bits(y), want, "y"))
    # the fp32 SiLU may put a value on the other side of a rounding boundary from the
    # oracle's; the quantised activations agree almost everywhere
    y2 = F.swiglu_fp4a4_gemv(F.from_bits(inp.g), F.from_bits(inp.u), dev_w(inp.W), F.scalar(float(G)), None, ws=ws)
    assert_bits_equal(F.to_bits(y2), F.to_bits(y), "repeat")


def test_swiglu_fp4a4_strided_halves():
    say("[fp4a4 gemv] g and u as the two halves of one [3, 2K] gate_up output")
    M, K, N = 3, 2048, 520
    inp = synth.swiglu_fp4_gemv_inputs(M, K, N, seed=77)
    gu = np.concatenate([inp.g, inp.u], axis=1)
    gud = F.from_bits(gu)
    G = calibrated(O.silu_mul(O.bf16_to_f64(inp.g), O.bf16_to_f64(inp.u)))
    y = F.swiglu_fp4a4_gemv(gud[:, :K], gud[:, K:], dev_w(inp.W), F.scalar(float(G)), F.scalar(0.5))
    want = O.swiglu_fp4a4_gemv(inp.g, inp.u, inp.W.qweight, inp.W.scales, G, 0.5)
    say("  worst err/bound", assert_close(F.to_bits(y), want, "y"))


# ---------------------------------------------------------------------------
# an exact case: every activation block is an E2M1 vector times a power of two with a
# largest magnitude of 6 times it, so quantisation is lossless with G = 1; power-of-two
# weight scales make every product and partial sum exact
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("M,K,N", [(3, 4096, 264), (16, 9216, 520)])
def test_fp4a4_exact_case_bit_exact(M, K, N):
    say(f"[fp4a4 gemv] exact case M={M} K={K} N={N}")
    rng = np.random.default_rng(M + N)
    codes = rng.integers(0, 16, size=(M, K))
    codes[:, ::16] = 7 | (rng.integers(0, 2, size=(M, K // 16)) << 3)      # a +-6 in every block
    e = rng.integers(-2, 3, size=(M, K // 16)).repeat(16, axis=1)
    x = synth.f32_to_bf16_bits((O.e2m1_decode(codes) * np.exp2(e)).astype(np.float32))
    W = synth.fp4_weight(rng, K, N)
    W = synth.FP4(W.qweight, O.e4m3_encode(np.exp2(rng.integers(-8, -5, size=W.scales.shape)).astype(np.float32)))
    y = F.fp4a4_gemv(F.from_bits(x), dev_w(W), F.scalar(1.0), F.scalar(0.5),
                     ws=F.workspace(max(1, F.fp4_gemv_workspace_bytes(M, K, N))))
    qc, sc = O.nvfp4_quantize(O.bf16_to_f64(x).astype(np.float32), 1.0)
    assert np.array_equal(O.nvfp4_dequant(qc, sc), O.bf16_to_f64(x))   # lossless, as built
    assert_bits_equal(F.to_bits(y), O.fp4a4_gemv(x, W.qweight, W.scales, 1.0, 0.5), "exact case")
