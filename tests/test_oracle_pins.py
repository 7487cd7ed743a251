"""More pins of the fp64 oracle: the identity-prologue GEMV, the column-chunked GEMVs
across their chunk boundaries, and the reason chains are compared layer by layer.

Each reference here is built from the definitions by a route the oracle does not take:
packed words are split into nibbles through a little-endian byte view (the oracle shifts
each nibble position out of the word), bf16 and E4M3 scales are decoded by PyTorch's
dtypes, E2M1 codes from their bit fields, and sums are pure-Python loops on sampled
columns.  CPU only.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import synth
from oracle import decode_mlp as OD   # the chunked helpers are module-private


# ----------------------------------------------------------------------------
# independent decoders
# ----------------------------------------------------------------------------
def nibbles_by_bytes(qw):
    """uint32 [N, K/8] -> codes int64 [N, K] in k order: byte b of a little-endian word
    holds the codes of k = 2b (low nibble) and k = 2b + 1 (high nibble)."""
    qw = np.ascontiguousarray(qw, dtype="<u4")
    N, KB = qw.shape
    by = qw.view(np.uint8).reshape(N, KB * 4).astype(np.int64)
    return np.stack([by & 0xF, by >> 4], axis=-1).reshape(N, KB * 8)


def bf16_by_torch(bits):
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)
    return t.double().numpy()


def int4_dense(qw, sc):
    """Dequantised int4 weights [K, N] float64 from the byte view and torch's bf16."""
    c = nibbles_by_bytes(qw)
    q = np.where(c >= 8, c - 16, c).astype(np.float64)       # [N, K]
    s = bf16_by_torch(sc)                                     # [K/128, N]
    return (q * np.repeat(s.T, 128, axis=1)).T


def e2m1_fields(c):
    s, e, m = (c >> 3) & 1, (c >> 1) & 3, c & 1
    mag = m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1 + m / 2)
    return -mag if s else mag


def fp4_dense(qw, sc8):
    """Dequantised FP4 weights [K, N] float64: E2M1 from its fields, E4M3 by torch."""
    lut = np.array([e2m1_fields(c) for c in range(16)])
    v = lut[nibbles_by_bytes(qw)]                             # [N, K]
    s = torch.from_numpy(np.ascontiguousarray(sc8, dtype=np.uint8)).view(torch.float8_e4m3fn).double().numpy()
    return (v * np.repeat(s, 16, axis=1)).T                   # s: [N, K/16]


def brute_column(a, qw, sc, n):
    """sum_k a[m, k] * q[k, n] * s[k // 128, n] for one column, pure-Python loops."""
    M, K = a.shape
    s = [float(v) for v in bf16_by_torch(sc[:, n])]
    out = []
    for m in range(M):
        tot = 0.0
        for k in range(K):
            code = (int(qw[n, k // 8]) >> (4 * (k % 8))) & 0xF
            tot += float(a[m, k]) * (code - 16 if code >= 8 else code) * s[k // 128]
        out.append(tot)
    return np.array(out)


# ----------------------------------------------------------------------------
# the identity-prologue GEMV (the gate_up projection's reference)
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("M,K,N", [(1, 128, 3), (2, 256, 8), (3, 384, 5)])
@pytest.mark.parametrize("out_scale", [None, 0.75])
def test_w4_gemv_identity_matches_brute_force(M, K, N, out_scale):
    inp = synth.swiglu_gemv_inputs(M, K, N, seed=M * 100 + N)
    x = inp.g                                    # any bf16 [M, K]
    got, f = O.w4_gemv(x, inp.W.qweight, inp.W.scales, out_scale, return_f64=True)
    xf = bf16_by_torch(x)
    s = 1.0 if out_scale is None else out_scale
    want = np.stack([brute_column(xf, inp.W.qweight, inp.W.scales, n) for n in range(N)], axis=1) * s
    assert np.max(np.abs(f - want)) <= 1e-12 * np.max(np.abs(want))
    # one rounding: the bf16 result is the RNE of the exact value (ties are measure zero)
    ref = torch.from_numpy(want).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    close = np.abs(O.bf16_to_f64(got) - O.bf16_to_f64(ref)) <= 2.0 ** -8 * np.abs(want)
    assert np.all(close) and np.mean(got == ref) > 0.95
    # the identity prologue applies no SiLU: y(-x) = -y(x) exactly
    _, fn = O.w4_gemv(x ^ np.uint16(0x8000), inp.W.qweight, inp.W.scales, out_scale, return_f64=True)
    assert np.array_equal(fn, -f)


def test_w4_gemv_scale_none_is_one_and_scale_is_linear():
    inp = synth.swiglu_gemv_inputs(2, 256, 16, seed=3)
    _, a = O.w4_gemv(inp.g, inp.W.qweight, inp.W.scales, None, return_f64=True)
    _, b = O.w4_gemv(inp.g, inp.W.qweight, inp.W.scales, 1.0, return_f64=True)
    _, c = O.w4_gemv(inp.g, inp.W.qweight, inp.W.scales, 0.5, return_f64=True)
    assert np.array_equal(a, b) and np.array_equal(c, 0.5 * a)


# ----------------------------------------------------------------------------
# column chunks: every C4/C5 reference dequantises its weights 4096 (int4) or 2048
# (FP4) columns at a time
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("N", [4104, 8200])
def test_int4_gemvs_across_column_chunks(N):
    M, K = 2, 128
    inp = synth.swiglu_gemv_inputs(M, K, N, seed=N, out_scale=0.5, with_residual=True)
    Wd = int4_dense(inp.W.qweight, inp.W.scales)
    act = O.silu_mul(bf16_by_torch(inp.g), bf16_by_torch(inp.u))
    x = bf16_by_torch(inp.g)
    want_act, want_x = act @ Wd, x @ Wd
    _, y = O.swiglu_w4_gemv(inp.g, inp.u, inp.W.qweight, inp.W.scales, 0.5, inp.residual, return_f64=True)
    assert np.max(np.abs(y - (0.5 * want_act + bf16_by_torch(inp.residual)))) <= 1e-12 * np.max(np.abs(y))
    _, z = O.w4_gemv(inp.g, inp.W.qweight, inp.W.scales, None, return_f64=True)
    assert np.max(np.abs(z - want_x)) <= 1e-12 * np.max(np.abs(want_x))
    # a chunk width that divides nothing, against the default
    assert np.max(np.abs(OD._chunked_gemv(x, inp.W.qweight, inp.W.scales, 1000) - want_x)) <= \
        1e-12 * np.max(np.abs(want_x))
    # the columns on either side of each boundary, by brute force
    for n in (0, 4095, 4096, 4097, N - 1) + ((8191, 8192) if N > 8192 else ()):
        assert np.max(np.abs(z[:, n] - brute_column(x, inp.W.qweight, inp.W.scales, n))) <= \
            1e-12 * np.max(np.abs(want_x))


@pytest.mark.parametrize("N", [2056, 4104])
def test_fp4_gemvs_across_column_chunks(N):
    M, K = 2, 64
    inp = synth.swiglu_fp4_gemv_inputs(M, K, N, seed=N, out_scale=0.5, with_residual=True)
    Wd = fp4_dense(inp.W.qweight, inp.W.scales)
    act = O.silu_mul(bf16_by_torch(inp.g), bf16_by_torch(inp.u))
    x = bf16_by_torch(inp.g)
    _, y = O.swiglu_fp4_gemv(inp.g, inp.u, inp.W.qweight, inp.W.scales, 0.5, inp.residual, return_f64=True)
    want = 0.5 * (act @ Wd) + bf16_by_torch(inp.residual)
    assert np.max(np.abs(y - want)) <= 1e-12 * np.max(np.abs(want))
    _, z = O.fp4_gemv(inp.g, inp.W.qweight, inp.W.scales, None, return_f64=True)
    assert np.max(np.abs(z - x @ Wd)) <= 1e-12 * np.max(np.abs(x @ Wd))
    assert np.max(np.abs(OD._chunked_fp4_gemv(x, inp.W.qweight, inp.W.scales, 999) - x @ Wd)) <= \
        1e-12 * np.max(np.abs(x @ Wd))


def test_layer_references_do_not_depend_on_the_chunk_width():
    inp = synth.mlp_inputs(2, 256, 384, n_layers=1, seed=21, out_scale=0.5)
    L = inp.layers[0]
    args = (inp.x, inp.r, L.norm_w, L.gate_up.qweight, L.gate_up.scales, L.down.qweight, L.down.scales, 0.5, 1e-6)
    a, b = O.mlp_decode(*args, n_chunk=4096), O.mlp_decode(*args, n_chunk=40)
    for k in ("h", "y", "gu", "out"):
        assert np.array_equal(a[k], b[k]), k
    a2, b2 = O.mlp_decode2(*args, n_chunk=4096), O.mlp_decode2(*args, n_chunk=56)
    for k in ("h", "act", "out"):
        assert np.array_equal(a2[k], b2[k]), k


# ----------------------------------------------------------------------------
# why chains are compared layer by layer
# ----------------------------------------------------------------------------
def test_two_valid_chains_diverge_while_every_layer_is_within_the_bound():
    """Two correct implementations of the deferred-residual chain, the fp64 oracle and one
    that accumulates in fp32 (in k order) with the same bf16 rounding points, stay within the stated
    bound layer by layer when fed the same inputs, yet drift apart by several times the
    bound after a dozen layers: a bf16 step here and there is amplified by later layers.
    So a chain is checked layer by layer, on the inputs each layer read."""
    H, I, NL = 1536, 2048, 12
    inp = synth.mlp_inputs(1, H, I, NL, seed=0, out_scale=0.5)

    def gemv32(a, qw, sc):
        # fp32 products accumulated in k order (numpy's elementwise fp32 arithmetic, so
        # the result does not depend on a BLAS library's blocking)
        W = np.ascontiguousarray(int4_dense(qw, sc), dtype=np.float32)
        a32 = a.astype(np.float32)[0]
        acc = np.zeros(W.shape[1], np.float32)
        for k in range(W.shape[0]):
            acc += a32[k] * W[k]
        return acc[None].astype(np.float64)

    def layer32(x, r, L):
        h, y = O.add_rmsnorm(x, r, L.norm_w, L.eps)
        gu = O.f64_to_bf16(gemv32(O.bf16_to_f64(y), L.gate_up.qweight, L.gate_up.scales))
        act = O.silu_mul(O.bf16_to_f64(gu[:, :I]), O.bf16_to_f64(gu[:, I:]))
        return O.f64_to_bf16(L.out_scale * gemv32(act, L.down.qweight, L.down.scales)), h

    def ratio(got, ref):
        g, r = O.bf16_to_f64(got), O.bf16_to_f64(ref)
        return float(np.max(np.abs(g - r) / (2e-2 * np.abs(r) + 1e-3 * np.max(np.abs(r)))))

    xa, ra, xb, rb = inp.x, inp.r, inp.x, inp.r
    per_layer, free = [], []
    for L in inp.layers:
        d = O.mlp_decode(xa, ra, L.norm_w, L.gate_up.qweight, L.gate_up.scales, L.down.qweight, L.down.scales,
                         L.out_scale, L.eps, residual_in_epilogue=False)
        o32, _ = layer32(xa, ra, L)                 # the fp32 layer on the oracle's inputs
        per_layer.append(ratio(o32, d["out"]))
        xb, rb = layer32(xb, rb, L)                 # the fp32 chain on its own outputs
        xa, ra = d["out"], d["h"]
        free.append(ratio(xb, xa))
    assert max(per_layer) <= 1.0, per_layer
    assert max(free) > 2.0, free


# ----------------------------------------------------------------------------
# the gate_up projection with the SwiGLU epilogue
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("M,K,I", [(1, 128, 8), (3, 256, 16)])
def test_w4_gemv_swiglu_matches_brute_force(M, K, I):
    inp = synth.swiglu_gemv_inputs(M, K, 2 * I, seed=K + I)
    x = bf16_by_torch(inp.g)
    act = O.w4_gemv_swiglu(inp.g, inp.W.qweight, inp.W.scales)
    g = np.stack([brute_column(x, inp.W.qweight, inp.W.scales, n) for n in range(I)], axis=1)
    u = np.stack([brute_column(x, inp.W.qweight, inp.W.scales, I + n) for n in range(I)], axis=1)
    want = np.array([[g[m, i] / (1.0 + math.exp(-g[m, i])) * u[m, i] for i in range(I)] for m in range(M)])
    ref = torch.from_numpy(want).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    # one rounding of the exact value: equal except within 1e-12 of a tie
    assert np.mean(act == ref) > 0.95
    assert np.all(np.abs(O.bf16_to_f64(act) - want) <= 2.0 ** -8 * np.abs(want) + 1e-300)
    # gate and up are not rounded on the way: the three-kernel layer's act, which reads the
    # rounded gate_up, differs from it
    gu_r = O.w4_gemv(inp.g, inp.W.qweight, inp.W.scales)
    act_r = O.f64_to_bf16(O.silu_mul(O.bf16_to_f64(gu_r[:, :I]), O.bf16_to_f64(gu_r[:, I:])))
    assert not np.array_equal(act, act_r)


# ----------------------------------------------------------------------------
# the prefill path: the SwiGLU pass (one rounding) and the GEMM
# ----------------------------------------------------------------------------
def test_swiglu_act_is_one_rounding_of_the_exact_value():
    from test_oracle import f64_to_bf16_bits_bitwise
    inp = synth.swiglu_gemv_inputs(3, 256, 8, seed=41)
    act = O.swiglu_act(inp.g, inp.u)
    g, u = bf16_by_torch(inp.g), bf16_by_torch(inp.u)
    for m in range(3):
        for k in range(256):
            v = g[m, k] / (1.0 + math.exp(-g[m, k])) * u[m, k]
            if v != 0.0 and abs(v) >= 2.0 ** -126:
                assert int(act[m, k]) == f64_to_bf16_bits_bitwise(v), (m, k)


@pytest.mark.parametrize("M,K,N", [(3, 128, 8), (5, 256, 24)])
def test_w4_gemm_matches_brute_force(M, K, N):
    inp = synth.swiglu_gemv_inputs(M, K, N, seed=M + K + N, with_residual=True)
    _, f = O.w4_gemm(inp.g, inp.W.qweight, inp.W.scales, 0.75, inp.residual, return_f64=True)
    x = bf16_by_torch(inp.g)
    want = np.stack([brute_column(x, inp.W.qweight, inp.W.scales, n) for n in range(N)], axis=1) * 0.75 \
        + bf16_by_torch(inp.residual)
    assert np.max(np.abs(f - want)) <= 1e-12 * np.max(np.abs(want))
    # the prefill path rounds the activation where the SwiGLU pass writes it
    _, p = O.swiglu_w4_gemm(inp.g, inp.u, inp.W.qweight, inp.W.scales, 0.75, inp.residual, return_f64=True)
    act = bf16_by_torch(O.swiglu_act(inp.g, inp.u))
    want2 = np.stack([brute_column(act, inp.W.qweight, inp.W.scales, n) for n in range(N)], axis=1) * 0.75 \
        + bf16_by_torch(inp.residual)
    assert np.max(np.abs(p - want2)) <= 1e-12 * np.max(np.abs(want2))
