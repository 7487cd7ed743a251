"""Pins of the oracle's FP4 activation path (both operands FP4): the E2M1 and E4M3
encoders against independent formulations and a library, the quantiser against a block
worked out by hand and its invariants, and the GEMV against a brute-force loop.  CPU
only."""
import numpy as np
import pytest
import torch

import oracle as O
import synth


def e2m1_by_local_ulp(a):
    """Round a magnitude to E2M1 by its local spacing: 0.5 below 2, 1 in [2, 4), 2 from 4
    on; Python's round() breaks ties to the even multiple, which is the even mantissa bit;
    6 is the largest value."""
    ulp = 0.5 if a < 2 else 1.0 if a < 4 else 2.0
    return min(round(a / ulp) * ulp, 6.0)


def magnitude_of(code):
    return float(abs(O.e2m1_decode(np.array([code]))[0]))


def test_e2m1_encode_matches_rounding_by_local_spacing():
    # a grid through every spacing, every tie point and its fp32 neighbours, beyond 6
    grid = np.arange(0, 9, 1 / 64, dtype=np.float32)
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float32)
    near = np.concatenate([ties, np.nextafter(ties, 0), np.nextafter(ties, 10)])
    vals = np.concatenate([grid, near, np.float32([6.0, 6.5, 100.0, 3e38])])
    codes = O.e2m1_encode(vals)
    for v, c in zip(vals, codes):
        assert c < 8 and magnitude_of(c) == e2m1_by_local_ulp(float(v)), (v, c)
    # signs: the sign bit follows the input's, -0 included
    neg = O.e2m1_encode(-vals)
    assert np.array_equal(neg & 7, codes) and np.all(neg >= 8)
    assert O.e2m1_encode(np.float32([-0.0]))[0] == 8 and O.e2m1_encode(np.float32([0.0]))[0] == 0


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(3)
    vals = np.exp2(rng.uniform(-12, 8.8, size=20000)).astype(np.float32)
    vals = vals[vals <= 448]
    # every tie point between neighbouring codes, and its fp32 neighbours
    fin = O.e4m3_decode(np.arange(127))
    mids = ((fin[:-1] + fin[1:]) / 2).astype(np.float32)
    vals = np.concatenate([vals, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9), fin.astype(np.float32)])
    got = O.e4m3_encode(vals)
    want = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, want)


def test_e4m3_encode_saturates():
    assert np.all(O.e4m3_encode(np.float32([448, 449, 464, 480, 1e6, 3e38])) == 126)
    assert O.e4m3_decode(126) == 448.0
    assert O.e4m3_encode(np.float32([0.0]))[0] == 0


def test_quantize_block_worked_by_hand():
    # G = 1, block 0..15: amax 15, 15 / 6 = 2.5 = 1.25 * 2 (E4M3 code 66, exact); the values
    # / 2.5 are 0, 0.4, 0.8, ..., 6.0, each to the nearest E2M1 magnitude (no ties)
    x = np.arange(16, dtype=np.float32)[None, :]
    codes, sc = O.nvfp4_quantize(x, 1.0)
    assert sc.tolist() == [[66]] and O.e4m3_decode(66) == 2.5
    assert codes[0].tolist() == [0, 1, 2, 2, 3, 4, 4, 5, 5, 6, 6, 6, 6, 7, 7, 7]
    # negated: the same codes with the sign bit
    c2, s2 = O.nvfp4_quantize(-x, 1.0)
    assert np.array_equal(s2, sc) and np.array_equal(c2[0, 1:], codes[0, 1:] | 8)
    # G scales out: x * 2^k with G * 2^k gives the same codes (every step exact by powers of 2)
    c3, s3 = O.nvfp4_quantize(x * np.float32(8), 8.0)
    assert np.array_equal(c3, codes) and np.array_equal(s3, sc)


def test_quantize_zero_and_saturated_blocks():
    x = np.zeros((2, 32), dtype=np.float32)
    x[1, 16:] = np.float32(1e6)                  # block scale saturates at 448 with G = 1
    codes, sc = O.nvfp4_quantize(x, 1.0)
    assert np.all(codes[0] == 0) and np.all(sc[0] == 0)
    assert sc[1, 1] == 126 and np.all(codes[1, 16:] == 7)
    # a block too small for any E4M3 scale quantises to zeros
    tiny = np.full((1, 16), 1e-6, dtype=np.float32)
    c4, s4 = O.nvfp4_quantize(tiny, 1.0)
    assert s4[0, 0] == 0 and np.all(c4 == 0)


def test_quantize_error_within_half_a_step():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((8, 1024)).astype(np.float32) * np.float32(3.0)
    G = np.float32(np.abs(x).max() / (6 * 448))
    codes, sc = O.nvfp4_quantize(x, G)
    xq = O.nvfp4_dequant(codes, sc) * np.float64(G)
    s = np.repeat(O.e4m3_decode(sc), 16, axis=-1) * np.float64(G)
    a = np.abs(x.astype(np.float64)) / s
    step = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))
    # unsaturated values: within half a local step (plus fp32 rounding of the quotient)
    ok = a <= 6
    err = np.abs(xq - x) / s
    assert np.all(err[ok] <= step[ok] / 2 * (1 + 1e-6) + 1e-6)
    # the block scale puts each block's largest magnitude near 6
    amax = np.abs(x.reshape(8, 64, 16)).max(-1)
    ratio = amax / (O.e4m3_decode(sc) * G)
    assert np.all((ratio > 5.2) & (ratio < 7.0))


def brute_fp4a4(x_bits, qweight, scales, G, out_scale):
    """Loop over (m, n, k) with both operands decoded from their fields."""
    x = O.bf16_to_f64(x_bits).astype(np.float32)
    codes, sc = O.nvfp4_quantize(x, G)
    wc = O.fp4_unpack(qweight)
    M, K = x.shape
    N = qweight.shape[0]
    ws = O.e4m3_decode(scales)
    out = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                a = O.e2m1_decode(codes[m, k]) * O.e4m3_decode(sc[m, k // 16])
                w = O.e2m1_decode(wc[k, n]) * ws[n, k // 16]
                acc += float(a) * float(w)
            out[m, n] = out_scale * acc
    return out


@pytest.mark.parametrize("M,K,N", [(1, 32, 8), (3, 64, 5)])
def test_fp4a4_gemv_matches_brute_force(M, K, N):
    inp = synth.swiglu_fp4_gemv_inputs(M, K, N, seed=M + K + N)
    G = np.float32(0.01)
    _, y64 = O.fp4a4_gemv(inp.g, inp.W.qweight, inp.W.scales, G, 0.75, return_f64=True)
    np.testing.assert_allclose(y64, brute_fp4a4(inp.g, inp.W.qweight, inp.W.scales, G, 0.75), rtol=1e-12, atol=1e-12)


def test_swiglu_fp4a4_quantises_the_fp32_activation():
    inp = synth.swiglu_fp4_gemv_inputs(2, 64, 8, seed=4)
    G = np.float32(0.003)
    act = O.silu_mul(O.bf16_to_f64(inp.g), O.bf16_to_f64(inp.u)).astype(np.float32)
    codes, sc = O.nvfp4_quantize(act, G)
    want = O.nvfp4_dequant(codes, sc) @ O.fp4_dequant(inp.W.qweight, inp.W.scales)
    _, y64 = O.swiglu_fp4a4_gemv(inp.g, inp.u, inp.W.qweight, inp.W.scales, G, 1.0, return_f64=True)
    np.testing.assert_allclose(y64, want, rtol=1e-12, atol=1e-12)
    # the quantised activation is a coarse copy of the exact one: within a quarter of it
    err = np.abs(O.nvfp4_dequant(codes, sc) * np.float64(G) - act)
    assert err.max() <= 0.25 * np.abs(act).max()
