"""Pins for the fp64 oracle: each test checks it against something other than itself.

What pins what:

* bf16 decoding: exhaustive over all 65,536 patterns against PyTorch's bf16 -> fp32.
* bf16 rounding: PyTorch's fp32 -> bf16 on fp32-representable values (ties, subnormals,
  overflow), and hand-built float64 values where rounding through fp32 would differ.
* int4 unpacking: all 16 codes in all 8 nibble positions against the two's-complement
  table; round trip against the independent packer in ``synth``.
* dequantisation: exact in fp32 (12-bit products).
* the GEMV: a pure-Python brute-force triple loop with its own bf16 decoding (struct),
  the materialised-product form and the group-factored form, on tiny shapes; closed
  forms (one-hot activation, zero scale, linearity, odd symmetry in u).
* the product buffer: the closed form 1*K*N*4 bytes, about 94 MB at K=9216, N=2560.
* RMSNorm: PyTorch's ``rms_norm`` in float64, unit RMS for an all-ones weight, the
  constant-row closed form, and h bit-identical to PyTorch's bf16 addition.
* SiLU: PyTorch's ``silu`` in float64.
* the layer: a pure-Python brute force of the whole add_rmsnorm -> gate_up -> SwiGLU
  -> down chain, with an independent bit-level bf16 rounding.
"""
import json
import math
import os
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------
# independent helpers (pure Python, no oracle code)
# ----------------------------------------------------------------------------
def bf16_bits_to_float(b: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(b) & 0xFFFF) << 16))[0]


def f64_to_bf16_bits_bitwise(x: float) -> int:
    """RNE float64 -> bf16 working on the float64 bit pattern (normal bf16 range only)."""
    u = struct.unpack("<Q", struct.pack("<d", x))[0]
    sign = u >> 63
    exp = (u >> 52) & 0x7FF
    man = u & ((1 << 52) - 1)
    if exp == 0 and man == 0:
        return sign << 15
    e = exp - 1023
    assert -126 <= e <= 127, "helper covers the normal bf16 range only"
    full = (1 << 52) | man                        # 53-bit significand
    keep = full >> 45                             # 8 bits kept
    rest = full & ((1 << 45) - 1)
    half = 1 << 44
    if rest > half or (rest == half and (keep & 1)):
        keep += 1
    if keep == 1 << 8:                            # carry into the next binade
        keep >>= 1
        e += 1
    assert e <= 127
    return (sign << 15) | ((e + 127) << 7) | (keep & 0x7F)


def to_bits_t(a):
    return torch.from_numpy(np.asarray(a, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)


def from_bits_t(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def brute_force_gemv(g, u, qw, sc, out_scale, residual=None):
    M, K = g.shape
    N = qw.shape[0]
    out = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            tot = 0.0
            for k in range(K):
                gv, uv = bf16_bits_to_float(g[m, k]), bf16_bits_to_float(u[m, k])
                a = gv / (1.0 + math.exp(-gv)) * uv
                code = (int(qw[n, k // 8]) >> (4 * (k % 8))) & 0xF
                qv = code - 16 if code >= 8 else code
                tot += a * qv * bf16_bits_to_float(sc[k // 128, n])
            v = tot * out_scale
            if residual is not None:
                v += bf16_bits_to_float(residual[m, n])
            out[m, n] = v
    return out


# ----------------------------------------------------------------------------
# bf16
# ----------------------------------------------------------------------------
def test_bf16_decode_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = O.bf16_to_f64(bits)
    ref = to_bits_t(bits).to(torch.float64).numpy()
    both_nan = np.isnan(ours) & np.isnan(ref)
    assert np.all((ours == ref) | both_nan)
    assert np.array_equal(np.signbit(ours[~both_nan]), np.signbit(ref[~both_nan]))


def test_bf16_round_matches_torch_on_fp32_values():
    rng = np.random.default_rng(1)
    # random fp32 bit patterns (finite), plus exact ties and near-ties
    pats = rng.integers(0, 2**32, size=400_000, dtype=np.uint64).astype(np.uint32)
    f = pats.view(np.float32)
    f = f[np.isfinite(f)]
    base = rng.integers(0, 2**16, size=20_000, dtype=np.uint32) << 16
    ties = (base | 0x8000).view(np.float32)
    near = np.concatenate([(base | 0x7FFF).view(np.float32), (base | 0x8001).view(np.float32)])
    sub = (rng.integers(1, 2**23, size=20_000, dtype=np.uint32)).view(np.float32)
    big = np.array([3.3895e38, 3.39e38, 3.4e38, -3.4e38, 1.0e-45, -1.0e-45, 0.0, -0.0],
                   dtype=np.float32)
    allv = np.concatenate([f, ties[np.isfinite(ties)], near[np.isfinite(near)], sub, big])
    ours = O.f64_to_bf16(allv.astype(np.float64))
    ref = from_bits_t(torch.from_numpy(allv).to(torch.bfloat16))
    assert np.array_equal(ours, ref)


def test_bf16_round_is_direct_from_f64():
    # Values where fp64 -> fp32 -> bf16 would differ from one rounding.
    one = 1.0
    cases = {
        one + 2**-8 + 2**-40: 0x3F81,   # just above the tie -> up (via fp32 it would tie -> even = 1.0)
        one + 2**-8 - 2**-40: 0x3F80,   # just below the tie -> down
        one + 2**-8: 0x3F80,            # exact tie -> even (1.0)
        one + 3 * 2**-8: 0x3F82,        # exact tie -> even (up)
        -(one + 2**-8 + 2**-40): 0xBF81,
    }
    for x, want in cases.items():
        assert int(O.f64_to_bf16(np.array([x]))[0]) == want, x
        assert f64_to_bf16_bits_bitwise(x) == want, x


def test_bf16_round_matches_bitwise_rounding_on_random_f64():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(20_000) * np.exp2(rng.integers(-100, 100, 20_000))
    ours = O.f64_to_bf16(x)
    ref = np.array([f64_to_bf16_bits_bitwise(float(v)) for v in x], dtype=np.uint16)
    assert np.array_equal(ours, ref)


# ----------------------------------------------------------------------------
# int4
# ----------------------------------------------------------------------------
def test_unpack_every_code_every_position():
    for j in range(8):
        for code in range(16):
            w = np.zeros((3, 1), dtype=np.uint32)          # [N = 3, K/8 = 1]
            w[1, 0] = np.uint32(code << (4 * j))
            q = O.w4_unpack(w)
            want = code - 16 if code >= 8 else code
            assert q.shape == (8, 3)
            assert q[j, 1] == want
            mask = np.ones_like(q, dtype=bool)
            mask[j, 1] = False
            assert np.all(q[mask] == 0)


def test_pack_unpack_round_trip():
    rng = np.random.default_rng(3)
    q = rng.integers(-8, 8, size=(256, 24)).astype(np.int8)
    assert np.array_equal(O.w4_unpack(synth.pack_int4(q)), q)
    words = rng.integers(0, 2**32, size=(5, 16), dtype=np.uint32)
    assert np.array_equal(synth.pack_int4(O.w4_unpack(words)), words)


def test_random_words_give_uniform_int4():
    rng = np.random.default_rng(4)
    q = O.w4_unpack(synth._qweight(rng, 1024, 512))
    counts = np.bincount(q.ravel().astype(np.int64) + 8, minlength=16)
    assert q.min() == -8 and q.max() == 7
    exp = q.size / 16
    assert np.all(np.abs(counts - exp) < 6 * math.sqrt(exp))


def test_dequant_is_exact_in_fp32():
    rng = np.random.default_rng(5)
    s_bits = synth._scales_bf16(rng, (4, 64))
    q = np.arange(-8, 8)
    s = O.bf16_to_f64(s_bits).ravel()
    prod64 = q[:, None].astype(np.float64) * s[None, :]
    prod32 = q[:, None].astype(np.float32) * s[None, :].astype(np.float32)
    assert np.array_equal(prod64, prod32.astype(np.float64))
    # and the oracle's dequant places scale g on rows [128 g, 128 g + 128)
    qw = synth.pack_int4(np.ones((256, 2), dtype=np.int8))
    sc = synth.f32_to_bf16_bits(np.array([[0.5, 0.25], [2.0, 4.0]], dtype=np.float32))
    d = O.w4_dequant(qw, sc)
    assert np.all(d[:128, 0] == 0.5) and np.all(d[128:, 0] == 2.0)
    assert np.all(d[:128, 1] == 0.25) and np.all(d[128:, 1] == 4.0)


# ----------------------------------------------------------------------------
# the GEMV
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("M,K,N", [(1, 128, 1), (2, 256, 3), (16, 128, 8), (1, 256, 8)])
def test_gemv_forms_agree_with_brute_force(M, K, N):
    inp = synth.swiglu_gemv_inputs(M, K, N, seed=7, out_scale=0.75, with_residual=True)
    args = (inp.g, inp.u, inp.W.qweight, inp.W.scales)
    _, fused = O.swiglu_w4_gemv(*args, 0.75, inp.residual, return_f64=True)
    prod = O.product_form_gemv(*args, 0.75, inp.residual)
    fact = O.factored_form_gemv(*args, 0.75, inp.residual)
    brute = brute_force_gemv(*args, 0.75, inp.residual)
    scale = np.max(np.abs(brute))
    for other in (prod, fact, fused):
        assert np.max(np.abs(other - brute)) <= 1e-12 * scale
    # no residual
    _, f2 = O.swiglu_w4_gemv(*args, 0.75, return_f64=True)
    b2 = brute_force_gemv(*args, 0.75)
    assert np.max(np.abs(f2 - b2)) <= 1e-12 * np.max(np.abs(b2))


def test_gemv_one_hot_activation_picks_a_weight_row():
    K, N = 256, 16
    rng = np.random.default_rng(8)
    q = rng.integers(-8, 8, size=(K, N)).astype(np.int8)
    qw = synth.pack_int4(q)
    sc = synth.f32_to_bf16_bits(np.full((K // 128, N), 2.0**-6, dtype=np.float32))
    g = np.zeros((1, K), dtype=np.float32)
    u = np.zeros((1, K), dtype=np.float32)
    k0 = 133
    g[0, k0] = 64.0            # silu(64) = 64 to within 1e-26 relative
    u[0, k0] = 3.0
    gb, ub = synth.f32_to_bf16_bits(g), synth.f32_to_bf16_bits(u)
    y, yf = O.swiglu_w4_gemv(gb, ub, qw, sc, 0.5, return_f64=True)
    want = 0.5 * 64.0 * 3.0 * q[k0].astype(np.float64) * 2.0**-6
    assert np.max(np.abs(yf[0] - want)) <= 1e-12 * np.max(np.abs(want))
    assert np.array_equal(O.bf16_to_f64(y[0]), want)          # small dyadic values: exact in bf16


def test_gemv_zero_scale_and_linearity_and_symmetry():
    inp = synth.swiglu_gemv_inputs(2, 256, 24, seed=9, with_residual=True)
    args = (inp.g, inp.u, inp.W.qweight, inp.W.scales)
    y0 = O.swiglu_w4_gemv(*args, 0.0)
    assert np.all(O.bf16_to_f64(y0) == 0)                    # +-0: 0 * acc keeps acc's sign
    yr = O.swiglu_w4_gemv(*args, 0.0, inp.residual)
    assert np.array_equal(O.bf16_to_f64(yr), O.bf16_to_f64(inp.residual))
    _, a = O.swiglu_w4_gemv(*args, 1.0, return_f64=True)
    _, b = O.swiglu_w4_gemv(*args, 2.0, return_f64=True)
    assert np.array_equal(2 * a, b)
    neg_u = inp.u ^ np.uint16(0x8000)
    _, c = O.swiglu_w4_gemv(inp.g, neg_u, inp.W.qweight, inp.W.scales, 1.0, return_f64=True)
    assert np.array_equal(c, -a)


def test_gemv_exact_special_case_integer_arithmetic():
    """g in {0, 32, 64}, u small integers, power-of-two scales: with exact rationals
    the result is sum_k g_k u_k q_k s; the fp64 oracle lies within 1e-12 of it."""
    rng = np.random.default_rng(10)
    M, K, N = 1, 512, 32
    g = rng.choice([0.0, 32.0, 64.0], size=(M, K)).astype(np.float32)
    u = rng.integers(-3, 4, size=(M, K)).astype(np.float32)
    q = rng.integers(-8, 8, size=(K, N)).astype(np.int8)
    s = rng.choice([2.0**-6, 2.0**-7], size=(K // 128, N)).astype(np.float32)
    gb, ub = synth.f32_to_bf16_bits(g), synth.f32_to_bf16_bits(u)
    qw, sb = synth.pack_int4(q), synth.f32_to_bf16_bits(s)
    _, yf = O.swiglu_w4_gemv(gb, ub, qw, sb, 0.5, return_f64=True)
    for n in range(N):
        exact = sum(Fraction(int(g[0, k])) * int(u[0, k]) * int(q[k, n]) * Fraction(float(s[k // 128, n]))
                    for k in range(K)) * Fraction(1, 2)
        assert abs(yf[0, n] - float(exact)) <= 1e-12 * max(1.0, abs(float(exact)))


def test_product_buffer_closed_form_matches_page():
    fig = json.load(open(os.path.join(GOLDEN, "page_figures.json")))["product_buffer"]
    nbytes = O.product_buffer_bytes(fig["M"], fig["K"], fig["N"])
    assert nbytes == 1 * 9216 * 2560 * 4 == 94_371_840
    assert round(nbytes / 1e6) == fig["approx_megabytes"]
    # and the explicit product array in the oracle's product form has that size
    M, K, N = 1, 256, 8
    assert np.empty((M, K, N), dtype=np.float32).nbytes == O.product_buffer_bytes(M, K, N)


# ----------------------------------------------------------------------------
# SiLU and RMSNorm
# ----------------------------------------------------------------------------
def test_silu_matches_torch():
    x = np.linspace(-40, 40, 10001)
    ref = torch.nn.functional.silu(torch.from_numpy(x)).numpy()
    assert np.max(np.abs(O.silu(x) - ref)) <= 1e-14 * np.max(np.abs(ref))
    assert O.silu(np.float64(0.0)) == 0.0
    assert abs(O.silu(np.float64(64.0)) - 64.0) < 1e-20


def test_h_bit_identical_to_torch_bf16_add():
    inp = synth.add_rmsnorm_inputs(64, 1024, seed=11)
    h, _ = O.add_rmsnorm(inp.x, inp.r, inp.w, inp.eps)
    ref = from_bits_t(to_bits_t(inp.x) + to_bits_t(inp.r))
    assert np.array_equal(h, ref)


def test_rmsnorm_matches_torch_rms_norm_f64():
    inp = synth.add_rmsnorm_inputs(32, 1536, seed=12)
    h, _, yf = O.add_rmsnorm(inp.x, inp.r, inp.w, 1e-6, return_f64=True)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(O.bf16_to_f64(h)), (1536,),
                                       torch.from_numpy(O.bf16_to_f64(inp.w)), 1e-6).numpy()
    assert np.max(np.abs(yf - ref)) <= 1e-13 * np.max(np.abs(ref))


def test_rmsnorm_unit_rms_with_unit_weight():
    inp = synth.add_rmsnorm_inputs(16, 4096, seed=13)
    ones = synth.f32_to_bf16_bits(np.ones(4096, dtype=np.float32))
    eps = 1e-6
    h, y, yf = O.add_rmsnorm(inp.x, inp.r, ones, eps, return_f64=True)
    hf = O.bf16_to_f64(h)
    ms = np.mean(hf * hf, axis=1)
    rms = np.sqrt(np.mean(yf * yf, axis=1))
    assert np.max(np.abs(rms - np.sqrt(ms / (ms + eps)))) < 1e-12
    assert np.max(np.abs(rms - 1.0)) < 1e-6
    yb = O.bf16_to_f64(y)
    assert np.max(np.abs(np.sqrt(np.mean(yb * yb, axis=1)) - 1.0)) < 2.0**-8


def test_rmsnorm_constant_row_closed_form():
    H, eps = 512, 1e-6
    for c in (0.75, -3.0, 1e-3):
        x = synth.f32_to_bf16_bits(np.full((1, H), c, dtype=np.float32))
        z = np.zeros((1, H), dtype=np.uint16)
        w = synth.f32_to_bf16_bits(np.linspace(0.5, 1.5, H).astype(np.float32))
        h, _, yf = O.add_rmsnorm(x, z, w, eps, return_f64=True)
        cb = O.bf16_to_f64(h)[0, 0]
        want = np.sign(cb) * O.bf16_to_f64(w) * abs(cb) / math.sqrt(cb * cb + eps)
        assert np.max(np.abs(yf[0] - want)) <= 1e-14


def test_eager_rmsnorm_close_to_torch_eager_sequence():
    """The oracle's eager variant against the eager PyTorch spelling (fp32 compute,
    bf16 round trips): equal except for rare one-step differences from fp32 rounding."""
    inp = synth.add_rmsnorm_inputs(64, 2048, seed=14)
    h, y = O.add_rmsnorm_eager(inp.x, inp.r, inp.w, 1e-6)
    xt, rt, wt = to_bits_t(inp.x), to_bits_t(inp.r), to_bits_t(inp.w)
    ht = xt + rt
    hf = ht.to(torch.float32)
    var = hf.pow(2).mean(-1, keepdim=True)
    yt = wt * (hf * torch.rsqrt(var + 1e-6)).to(torch.bfloat16)
    assert np.array_equal(h, from_bits_t(ht))
    diff = np.abs(O.bf16_to_f64(y) - O.bf16_to_f64(from_bits_t(yt)))
    step = np.abs(O.bf16_to_f64(from_bits_t(yt))) * 2.0**-7
    assert np.all(diff <= step + 1e-30)
    assert np.mean(diff > 0) < 0.01


# ----------------------------------------------------------------------------
# the layer, against a pure-Python brute force
# ----------------------------------------------------------------------------
def _py_round(x):
    return bf16_bits_to_float(f64_to_bf16_bits_bitwise(x))


def _py_layer(x, r, nw, guq, gus, dq, ds, s, eps, residual_in_epilogue):
    M, H = x.shape
    I = guq.shape[0] // 2

    def wq(qw, sc, k, n):
        code = (int(qw[n, k // 8]) >> (4 * (k % 8))) & 0xF
        return (code - 16 if code >= 8 else code) * bf16_bits_to_float(sc[k // 128, n])

    outs = {"h": [], "y": [], "gu": [], "out": []}
    for m in range(M):
        h = [_py_round(bf16_bits_to_float(x[m, j]) + bf16_bits_to_float(r[m, j])) for j in range(H)]
        ms = sum(v * v for v in h) / H
        inv = 1.0 / math.sqrt(ms + eps)
        y = [_py_round(h[j] * inv * bf16_bits_to_float(nw[j])) for j in range(H)]
        gu = [_py_round(sum(y[k] * wq(guq, gus, k, n) for k in range(H))) for n in range(2 * I)]
        act = [gu[k] / (1.0 + math.exp(-gu[k])) * gu[I + k] for k in range(I)]
        out = []
        for n in range(H):
            v = s * sum(act[k] * wq(dq, ds, k, n) for k in range(I))
            if residual_in_epilogue:
                v += h[n]
            out.append(_py_round(v))
        outs["h"].append(h); outs["y"].append(y); outs["gu"].append(gu); outs["out"].append(out)
    return {k: np.array(v) for k, v in outs.items()}


@pytest.mark.parametrize("resid", [True, False])
def test_mlp_layer_matches_brute_force(resid):
    inp = synth.mlp_inputs(2, 128, 128, n_layers=1, seed=15, out_scale=0.5)
    L = inp.layers[0]
    d = O.mlp_decode(inp.x, inp.r, L.norm_w, L.gate_up.qweight, L.gate_up.scales,
                     L.down.qweight, L.down.scales, L.out_scale, L.eps,
                     residual_in_epilogue=resid)
    ref = _py_layer(inp.x, inp.r, L.norm_w, L.gate_up.qweight, L.gate_up.scales,
                    L.down.qweight, L.down.scales, L.out_scale, L.eps, resid)
    for k in ("h", "y", "gu", "out"):
        ours = O.bf16_to_f64(d[k])
        # identical except where fp64 summation order lands within 1e-12 of a bf16 tie
        mism = ours != ref[k]
        assert mism.mean() < 0.02, k
        assert np.all(np.abs(ours - ref[k])[mism] <= np.abs(ref[k][mism]) * 2.0**-7), k


def test_mlp_chain_defers_residual():
    inp = synth.mlp_inputs(1, 128, 128, n_layers=2, seed=16)
    x2, r2, tr = O.mlp_chain(inp.x, inp.r, inp.layers, keep=True)
    L0, L1 = inp.layers
    d0 = O.mlp_decode(inp.x, inp.r, L0.norm_w, L0.gate_up.qweight, L0.gate_up.scales,
                      L0.down.qweight, L0.down.scales, 0.5, 1e-6, residual_in_epilogue=False)
    # layer 1's residual input is layer 0's h; its x input is layer 0's down output
    h1, _ = O.add_rmsnorm(d0["out"], d0["h"], L1.norm_w, 1e-6)
    assert np.array_equal(r2, h1)
    assert np.array_equal(tr[1]["h"], h1)
    assert np.array_equal(tr[0]["out"], d0["out"])


# ----------------------------------------------------------------------------
# the two-kernel layer (norm as the gate_up prologue, SwiGLU as its epilogue)
# ----------------------------------------------------------------------------
def _py_layer2(x, r, nw, guq, gus, dq, ds, s, eps, residual_in_epilogue, round_y=False):
    """Pure-Python loops: gate/up are not rounded (never written), act is; y is rounded only
    with round_y (the form whose norm runs as its own kernel and writes y)."""
    M, H = x.shape
    I = guq.shape[0] // 2

    def wq(qw, sc, k, n):
        code = (int(qw[n, k // 8]) >> (4 * (k % 8))) & 0xF
        return (code - 16 if code >= 8 else code) * bf16_bits_to_float(sc[k // 128, n])

    outs = {"h": [], "act": [], "out": []}
    for m in range(M):
        h = [_py_round(bf16_bits_to_float(x[m, j]) + bf16_bits_to_float(r[m, j])) for j in range(H)]
        inv = 1.0 / math.sqrt(sum(v * v for v in h) / H + eps)
        y = [h[j] * inv * bf16_bits_to_float(nw[j]) for j in range(H)]
        if round_y:
            y = [_py_round(v) for v in y]
        g = [sum(y[k] * wq(guq, gus, k, n) for k in range(H)) for n in range(I)]
        u = [sum(y[k] * wq(guq, gus, k, I + n) for k in range(H)) for n in range(I)]
        act = [_py_round(g[n] / (1.0 + math.exp(-g[n])) * u[n]) for n in range(I)]
        out = []
        for n in range(H):
            v = s * sum(act[k] * wq(dq, ds, k, n) for k in range(I))
            out.append(_py_round(v + (h[n] if residual_in_epilogue else 0.0)))
        outs["h"].append(h); outs["act"].append(act); outs["out"].append(out)
    return {k: np.array(v) for k, v in outs.items()}


@pytest.mark.parametrize("round_y", [False, True])
@pytest.mark.parametrize("resid", [True, False])
def test_mlp_layer2_matches_brute_force(resid, round_y):
    inp = synth.mlp_inputs(2, 128, 128, n_layers=1, seed=17, out_scale=0.5)
    L = inp.layers[0]
    d = O.mlp_decode2(inp.x, inp.r, L.norm_w, L.gate_up.qweight, L.gate_up.scales,
                      L.down.qweight, L.down.scales, L.out_scale, L.eps, residual_in_epilogue=resid,
                      y_rounded=round_y)
    ref = _py_layer2(inp.x, inp.r, L.norm_w, L.gate_up.qweight, L.gate_up.scales,
                     L.down.qweight, L.down.scales, L.out_scale, L.eps, resid, round_y)
    for k in ("h", "act", "out"):
        ours = O.bf16_to_f64(d[k])
        mism = ours != ref[k]
        assert mism.mean() < 0.02, k
        assert np.all(np.abs(ours - ref[k])[mism] <= np.abs(ref[k][mism]) * 2.0**-7), k


def test_layer2_gate_up_is_norm_invariant_to_input_scale():
    # RMSNorm with eps = 0 divides out any common factor of the row: doubling x and r
    # (exact in bf16) doubles h and leaves y, and so act, bit-identical.
    inp = synth.mlp_inputs(2, 256, 128, n_layers=1, seed=18)
    L = inp.layers[0]
    x2 = O.f64_to_bf16(2.0 * O.bf16_to_f64(inp.x))
    r2 = O.f64_to_bf16(2.0 * O.bf16_to_f64(inp.r))
    h1, a1 = O.add_rmsnorm_gemv_swiglu(inp.x, inp.r, L.norm_w, L.gate_up.qweight, L.gate_up.scales, 0.0)
    h2, a2 = O.add_rmsnorm_gemv_swiglu(x2, r2, L.norm_w, L.gate_up.qweight, L.gate_up.scales, 0.0)
    assert np.array_equal(O.bf16_to_f64(h2), 2.0 * O.bf16_to_f64(h1))
    assert np.array_equal(a1, a2)


def test_layer2_h_equals_add_rmsnorm_h_and_act_close_to_three_kernel_form():
    inp = synth.mlp_inputs(4, 512, 256, n_layers=1, seed=19)
    L = inp.layers[0]
    d3 = O.mlp_decode(inp.x, inp.r, L.norm_w, L.gate_up.qweight, L.gate_up.scales,
                      L.down.qweight, L.down.scales, 0.5, 1e-6)
    d2 = O.mlp_decode2(inp.x, inp.r, L.norm_w, L.gate_up.qweight, L.gate_up.scales,
                       L.down.qweight, L.down.scales, 0.5, 1e-6)
    assert np.array_equal(d2["h"], d3["h"])
    I = 256
    act3 = O.silu_mul(O.bf16_to_f64(d3["gu"][:, :I]), O.bf16_to_f64(d3["gu"][:, I:]))
    a2 = O.bf16_to_f64(d2["act"])
    # the three-kernel form rounds y and gate/up to bf16; the two-kernel form does not
    assert np.max(np.abs(a2 - act3)) <= 0.05 * np.max(np.abs(act3))
    o2, o3 = O.bf16_to_f64(d2["out"]), O.bf16_to_f64(d3["out"])
    assert np.max(np.abs(o2 - o3)) <= 0.05 * np.max(np.abs(o3))


def test_mlp_chain2_defers_residual():
    inp = synth.mlp_inputs(1, 128, 128, n_layers=2, seed=20)
    x2, r2, tr = O.mlp_chain2(inp.x, inp.r, inp.layers, keep=True)
    L0, L1 = inp.layers
    d0 = O.mlp_decode2(inp.x, inp.r, L0.norm_w, L0.gate_up.qweight, L0.gate_up.scales,
                       L0.down.qweight, L0.down.scales, 0.5, 1e-6, residual_in_epilogue=False)
    h1, _ = O.add_rmsnorm(d0["out"], d0["h"], L1.norm_w, 1e-6)
    assert np.array_equal(r2, h1)
    assert np.array_equal(tr[0]["out"], d0["out"])


# ----------------------------------------------------------------------------
# the unfused references
# ----------------------------------------------------------------------------
def test_unfused_act_matches_torch_eager_silu_mul():
    inp = synth.swiglu_gemv_inputs(4, 256, 16, seed=17)
    gt, ut = to_bits_t(inp.g), to_bits_t(inp.u)
    act_t = torch.nn.functional.silu(gt) * ut                       # two bf16 kernels in eager
    act_o = O.f64_to_bf16(O.round_bf16(O.round_bf16(O.silu(O.bf16_to_f64(inp.g)))
                                       * O.bf16_to_f64(inp.u)))
    a, b = O.bf16_to_f64(act_o), O.bf16_to_f64(from_bits_t(act_t))
    assert np.all(np.abs(a - b) <= np.abs(b) * 2.0**-7 + 1e-30)
    assert np.mean(a != b) < 0.01
    # the unfused GEMV is the fused one up to the extra bf16 round trips
    y_un = O.bf16_to_f64(O.unfused_act_gemv(inp.g, inp.u, inp.W.qweight, inp.W.scales, 1.0))
    _, y_f = O.swiglu_w4_gemv(inp.g, inp.u, inp.W.qweight, inp.W.scales, 1.0, return_f64=True)
    assert np.max(np.abs(y_un - y_f)) <= 2e-2 * np.max(np.abs(y_f))


def test_unfused_product_close_to_fused():
    inp = synth.swiglu_gemv_inputs(1, 1024, 512, seed=0, out_scale=0.5)
    y_p = O.bf16_to_f64(O.unfused_product_gemv(inp.g, inp.u, inp.W.qweight, inp.W.scales, 0.5))
    _, y_f = O.swiglu_w4_gemv(inp.g, inp.u, inp.W.qweight, inp.W.scales, 0.5, return_f64=True)
    assert np.all(np.abs(y_p - y_f) <= 2.0**-7 * np.abs(y_f) + 1e-30)
