"""Pins of the oracle's FP4 weight path (E2M1 values, E4M3 block scales of 16 along K,
fp32 output multiplier): the decodings against their bit-field definitions and a
library, the GEMV against a brute-force loop, exact rational arithmetic and special
cases.  CPU only."""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
import synth


def e2m1_from_fields(c):
    """E2M1 from its fields: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0;
    exponent 0 is subnormal (m * 2**-1)."""
    s, e, m = (c >> 3) & 1, (c >> 1) & 3, c & 1
    mag = m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1 + m / 2)
    return -mag if s else mag


def test_e2m1_every_code_matches_its_fields():
    got = O.e2m1_decode(np.arange(16))
    want = np.array([e2m1_from_fields(c) for c in range(16)])
    assert np.array_equal(got, want)
    assert np.signbit(got[8]) and got[8] == 0          # code 8 is -0
    mags = got[:8]
    assert np.all(np.diff(mags) > 0) and mags.max() == 6.0 and mags[1] == 0.5
    assert np.array_equal(got[8:], -got[:8])


def test_e2m1_values_lie_on_the_e4m3_grid():
    # every E2M1 value is exactly representable in E4M3 (checked with torch's fp8 type)
    v = torch.tensor(O.e2m1_decode(np.arange(16)), dtype=torch.float32)
    assert torch.equal(v.to(torch.float8_e4m3fn).float(), v)


def test_e4m3_every_code_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    got = O.e4m3_decode(codes)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().double().numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2
    assert np.array_equal(got[~nan], want[~nan])
    assert np.nanmax(got) == 448.0 and got[1] == 2.0 ** -9


def test_fp4_unpack_round_trip():
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 16, size=(64, 7))
    words = synth.pack_int4(np.where(codes >= 8, codes - 16, codes))    # same nibble layout
    assert np.array_equal(O.fp4_unpack(words), codes)


def test_fp4_dequant_block_layout():
    K, N = 64, 3
    codes = np.full((K, N), 2)                       # E2M1 code 2 = 1.0
    words = synth.pack_int4(codes)
    sc = np.zeros((N, K // 16), dtype=np.uint8)
    for b in range(K // 16):
        sc[:, b] = 0x38 + b                          # E4M3 1.0, 1.125, 1.25, 1.375
    w = O.fp4_dequant(words, sc)
    for k in range(K):
        assert np.all(w[k] == 1.0 + (k // 16) / 8)


def brute_fp4(g, u, words, sc, out_scale, residual=None):
    """Pure-Python triple loop over (m, n, k) from the decoded fields."""
    gf, uf = O.bf16_to_f64(g), O.bf16_to_f64(u)
    M, K = gf.shape
    N = words.shape[0]
    y = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                code = (int(words[n, k // 8]) >> (4 * (k % 8))) & 0xF
                sb = int(sc[n, k // 16])
                e, mm = (sb >> 3) & 0xF, sb & 7
                s = (mm / 8 * 2.0 ** -6 if e == 0 else (1 + mm / 8) * 2.0 ** (e - 7)) * (-1 if sb & 0x80 else 1)
                a = gf[m, k] / (1 + math.exp(-gf[m, k])) * uf[m, k]
                acc += a * e2m1_from_fields(code) * s
            y[m, n] = acc * out_scale + (O.bf16_to_f64(residual)[m, n] if residual is not None else 0.0)
    return y


@pytest.mark.parametrize("M,K,N", [(1, 32, 3), (2, 64, 5), (3, 96, 2)])
def test_fp4_gemv_matches_brute_force(M, K, N):
    inp = synth.swiglu_fp4_gemv_inputs(M, K, N, seed=K + N, out_scale=0.75, with_residual=True)
    got, f = O.swiglu_fp4_gemv(inp.g, inp.u, inp.W.qweight, inp.W.scales, 0.75, inp.residual, return_f64=True)
    want = brute_fp4(inp.g, inp.u, inp.W.qweight, inp.W.scales, 0.75, inp.residual)
    assert np.allclose(f, want, rtol=1e-12, atol=1e-12 * np.abs(want).max())
    assert np.array_equal(got, O.f64_to_bf16(want)) or np.abs(O.bf16_to_f64(got) - want).max() <= \
        2.0 ** -7 * np.abs(want).max()


def test_fp4_gemv_exact_rational():
    # integer activations: every term is a dyadic rational and the fp64 sum is exact
    rng = np.random.default_rng(9)
    K, N = 256, 6
    x = synth.f32_to_bf16_bits(rng.integers(-3, 4, size=(1, K)).astype(np.float32))
    W = synth.fp4_weight(rng, K, N)
    got = O.fp4_gemv(x, W.qweight, W.scales, out_scale=0.5, return_f64=True)[1]
    codes = O.fp4_unpack(W.qweight)
    for n in range(N):
        exact = Fraction(0)
        for k in range(K):
            s = Fraction(float(O.e4m3_decode(W.scales[n, k // 16])))
            exact += Fraction(float(O.bf16_to_f64(x[0, k]))) * Fraction(e2m1_from_fields(int(codes[k, n]))) * s
        assert Fraction(float(got[0, n])) == exact / 2


def test_fp4_gemv_one_hot_and_linearity():
    rng = np.random.default_rng(3)
    K, N = 128, 9
    W = synth.fp4_weight(rng, K, N)
    w = O.fp4_dequant(W.qweight, W.scales)
    for k in (0, 17, 127):
        x = np.zeros((1, K), dtype=np.float32)
        x[0, k] = 1.0
        y = O.fp4_gemv(synth.f32_to_bf16_bits(x), W.qweight, W.scales, return_f64=True)[1]
        assert np.array_equal(y[0], w[k])
    inp = synth.swiglu_fp4_gemv_inputs(2, K, N, seed=1)
    a = O.swiglu_fp4_gemv(inp.g, inp.u, inp.W.qweight, inp.W.scales, 1.0, return_f64=True)[1]
    b = O.swiglu_fp4_gemv(inp.g, inp.u, inp.W.qweight, inp.W.scales, 2.0, return_f64=True)[1]
    assert np.array_equal(b, 2 * a)
