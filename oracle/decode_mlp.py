"""fp64 CPU oracle for the fused decode-MLP path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module.  It shares no code with the
HIP library (``memory_bound_decode_add_amd``): no kernels, no helpers, no constants,
no pre- or post-processing.  Inputs come from the seeded generators in ``synth``.

Everything is computed in float64 from the same bf16 bit patterns (``uint16``) and
packed int4 words (``uint32``) the GPU reads.  A bf16 result is produced by rounding
the float64 value *directly* to bf16 (round to nearest, ties to even), never through
float32, and only at the points where the GPU path writes a bf16 tensor to memory.

Sources (the pages this follows, cited by title and section):

* [P1] "PyTorch Community Proposes Fusion Fix as Large Intermediate Buffers May Slow
  Single-Token Decoding in Quantized LLMs" (ainews.surl.tw): the single-row matmul
  that Inductor turns into a broadcast multiply plus a sum, the (1, K, N) fp32
  product it can materialise, and the int4 weight-quantised case with a SwiGLU
  pre-operation.
* [P3] "PyTorch folds NVFP4 output scaling into NVGEMM candidates for decode
  workloads" (ainewsletter.today): a zero-dimensional fp32 output-scale multiplier
  applied to a matmul result, and the fallback that multiplies separately.
* [P4] "09 - Operator fusion" (infra.pidoku.co.in), section 5 "Technical
  explanation": the fusion taxonomy (reduction + elementwise, prologue dequant,
  horizontal gate_up fusion), the residual's two consumers, and the three-kernel
  layer (add_rmsnorm -> gate_up GEMM -> down GEMM with residual add).
* [P5] "Kernel Fusion, torch.compile and CUDA Graphs, Measured" (vidyal.ai):
  "Step 1" (SwiGLU = g / (1 + exp(-g)) * u; RMSNorm as Qwen2 spells it),
  "Step 2: fusing them by hand in Triton" (add + RMSNorm with two outputs, h kept in
  bf16), "Step 3: what torch.compile generates" (the down projection computing
  silu(g) * u while reading the weights), "Step 4" (graph replay of the layer chain).

Readings where the pages are silent (each is also listed in the design notes):

* int4 words: eight weights per uint32 along K, weight k = 8*kb + j in bits
  [4j, 4j+4), two's-complement nibbles (values -8..7), qweight [N, K/8] row-major
  (a linear layer's [out_features, in_features] orientation).
* scales: bf16 [K/128, N], group g covering k in [128 g, 128 g + 128).
* act = silu(g) * u is never rounded on the fused path (it is never written).
* epilogue: y = bf16(out_scale * acc [+ residual]) with a single rounding.
* RMSNorm: h = bf16(x + r); mean of h^2 over H; eps inside the square root; one final
  rounding of h * w / sqrt(ms + eps).
* Multi-layer chain: each layer's add_rmsnorm adds the previous layer's down output
  into the residual (the residual add deferred to the next layer's norm).
* FP4 weights ([P3]'s packed FP4 with E4M3 1x16 block scales and an fp32 output
  multiplier) are read as weight-only quantisation: the activation stays the unrounded
  SwiGLU prologue value.  E2M1 codes are packed like the int4 nibbles (code of k = 8*kb
  + j in bits [4j, 4j+4) of word (n, kb)); block scales are E4M3 ('fn': no infinities)
  bytes [N, K/16], scale (n, b) applying to k in [16 b, 16 b + 16) of column n.
* FP4 activations (both operands FP4, as [P3]'s scaled matmul takes them): quantised at
  run time with a given per-tensor scale G, one E4M3 scale per 16 values, every step in
  fp32 with round-to-nearest-even and saturation (see nvfp4_quantize); the per-tensor
  scale travels in the output multiplier.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "GROUP", "bf16_to_f64", "f64_to_bf16", "round_bf16", "w4_unpack", "w4_dequant",
    "silu", "silu_mul", "swiglu_w4_gemv", "w4_gemv", "add_rmsnorm", "mlp_decode",
    "mlp_chain", "product_form_gemv", "factored_form_gemv",
    "product_buffer_bytes", "unfused_act_gemv", "unfused_product_gemv",
    "add_rmsnorm_eager",
    "add_rmsnorm_gemv_swiglu", "w4_gemv_swiglu", "mlp_decode2", "mlp_chain2",
    "swiglu_act", "w4_gemm", "swiglu_w4_gemm",
    "FP4_BLOCK", "e2m1_decode", "e4m3_decode", "fp4_unpack", "fp4_dequant", "swiglu_fp4_gemv", "fp4_gemv",
    "e4m3_encode", "e2m1_encode", "nvfp4_quantize", "nvfp4_dequant", "fp4a4_gemv", "swiglu_fp4a4_gemv",
]

GROUP = 128   # weights per scale group along K (one scale per group per column)
NIB = 8       # int4 weights per packed uint32


# ----------------------------------------------------------------------------
# bf16 <-> float64
# ----------------------------------------------------------------------------
def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact): the bf16 pattern is the top half of an fp32."""
    b = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):                 # NaN patterns stay NaN
        return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def round_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (ties to even), in float64.

    bf16 has an 8-bit significand (7 stored bits) and fp32's exponent range.  For a
    normal result the spacing of bf16 values around x is 2**(e-8) where x = m * 2**e,
    0.5 <= |m| < 1; below 2**-126 the spacing is fixed at 2**-133 (subnormals).
    Dividing by the spacing is exact in float64 (a power of two), and ``np.rint``
    rounds half to even, so this is one correct rounding of the float64 value.
    Values beyond the largest finite bf16 round to +-inf (as fp32 casting does).
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    q = np.maximum(e - 8, -133).astype(np.float64)
    step = np.exp2(q)
    with np.errstate(over="ignore", invalid="ignore"):
        y = np.rint(x / step) * step
    y = np.where(np.isfinite(x), y, x)
    return y


def f64_to_bf16(x) -> np.ndarray:
    """float64 -> bf16 bit patterns (uint16), one round-to-nearest-even step."""
    y = round_bf16(x)
    with np.errstate(over="ignore"):
        f = y.astype(np.float32)                      # exact: y is a bf16 value (or +-inf)
    bits = (np.ascontiguousarray(f).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(y)
    if np.any(nan):
        bits = np.where(nan, np.uint16(0x7FC0), bits)
    return bits


# ----------------------------------------------------------------------------
# int4 weights  ([P4] section 5, prologue fusion: dequantise weights as they are read)
# ----------------------------------------------------------------------------
def w4_unpack(qweight) -> np.ndarray:
    """Packed words uint32 [N, K/8] -> int8 weights [K, N].

    Weight k = 8*kb + j of column n is nibble j of word (n, kb), a two's-complement
    4-bit integer: codes 0..7 are 0..7, codes 8..15 are -8..-1.
    """
    w = np.asarray(qweight, dtype=np.uint32)
    n, kb = w.shape
    out = np.empty((kb, NIB, n), dtype=np.int8)
    for j in range(NIB):
        code = ((w >> np.uint32(4 * j)) & np.uint32(0xF)).astype(np.int16)   # [n, kb]
        out[:, j, :] = np.where(code >= 8, code - 16, code).astype(np.int8).T
    return out.reshape(kb * NIB, n)


def w4_dequant(qweight, scales) -> np.ndarray:
    """Dequantised weights, float64 [K, N]: w[k, n] = q[k, n] * s[k // 128, n].

    The product of a 4-bit integer and a bf16 scale has at most 12 significant bits,
    so the same number is obtained exactly in fp32 on the GPU.
    """
    q = w4_unpack(qweight).astype(np.float64)
    s = bf16_to_f64(scales)
    K = q.shape[0]
    if s.shape[0] * GROUP != K or s.shape[1] != q.shape[1]:
        raise ValueError("scales must be [K/128, N]")
    return q * np.repeat(s, GROUP, axis=0)


# ----------------------------------------------------------------------------
# SwiGLU ([P5] Step 1: silu(g) * u = g / (1 + exp(-g)) * u)
# ----------------------------------------------------------------------------
def silu(g) -> np.ndarray:
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def silu_mul(g, u) -> np.ndarray:
    return silu(g) * np.asarray(u, dtype=np.float64)


def _epilogue(acc, out_scale, residual):
    """[P3]: the fp32 output scale multiplies the matmul result; [P4] section 5: the
    residual add may ride in the same epilogue.  One rounding to bf16."""
    y = acc * (1.0 if out_scale is None else float(out_scale))
    if residual is not None:
        y = y + bf16_to_f64(residual)
    return y


def swiglu_w4_gemv(g, u, qweight, scales, out_scale=1.0, residual=None, *, return_f64=False):
    """y[m, n] = bf16(out_scale * sum_k silu(g[m,k]) u[m,k] w[k,n] (+ residual[m, n])).

    [P1]: the int4 weight-quantised single-row matmul with a SwiGLU pre-operation,
    computed without materialising the (M, K, N) product; [P5] Step 3: the down
    projection computes silu(g) * u while reading its weights; [P3]: the output scale
    is folded into the same result.  The activation is not rounded (it is never
    written on the fused path).
    """
    act = silu_mul(bf16_to_f64(g), bf16_to_f64(u))
    acc = _chunked_gemv(act, qweight, scales)
    y = _epilogue(acc, out_scale, residual)
    return (f64_to_bf16(y), y) if return_f64 else f64_to_bf16(y)


def w4_gemv(x, qweight, scales, out_scale=None, *, return_f64=False):
    """The same GEMV with the identity prologue: y = bf16([out_scale *] x @ dequant(W)).

    Used for the horizontally fused gate_up projection ([P4] section 5, horizontal
    fusion: gate_proj and up_proj as one matmul, gate columns first).
    """
    acc = _chunked_gemv(bf16_to_f64(x), qweight, scales)
    y = _epilogue(acc, out_scale, None)
    return (f64_to_bf16(y), y) if return_f64 else f64_to_bf16(y)


# ----------------------------------------------------------------------------
# residual add + RMSNorm ([P5] Step 2; [P4] section 5, reduction + elementwise and
# the two-output rule for the residual's two consumers)
# ----------------------------------------------------------------------------
def add_rmsnorm(x, r, w, eps=1e-6, *, return_f64=False):
    """(h, y): h = bf16(x + r); y = bf16(h * w / sqrt(mean_H(h^2) + eps)).

    h is the new residual, kept in bf16; the mean is over the H columns of each row;
    eps sits inside the square root; y is rounded once.
    """
    hs = round_bf16(bf16_to_f64(x) + bf16_to_f64(r))        # exact sum, then RNE
    H = hs.shape[-1]
    ms = np.sum(hs * hs, axis=-1, keepdims=True) / H
    y = hs * bf16_to_f64(w) / np.sqrt(ms + float(eps))
    out = (f64_to_bf16(hs), f64_to_bf16(y))
    return out + (y,) if return_f64 else out


# ----------------------------------------------------------------------------
# the layer and the chain ([P4] section 5, the fusion boundary problem)
# ----------------------------------------------------------------------------
def mlp_decode(x, r, norm_w, gu_q, gu_s, d_q, d_s, out_scale=0.5, eps=1e-6,
               residual_in_epilogue=True, *, n_chunk=4096):
    """One decode-MLP layer, three kernels' worth of work.

    1. (h, y) = add_rmsnorm(x, r, norm_w)
    2. gu = bf16(y @ dequant(W_gate_up)); gate = gu[:, :I], up = gu[:, I:]
    3. out = bf16(out_scale * silu(gate) * up @ dequant(W_down) [+ h])

    With ``residual_in_epilogue`` the layer's residual add rides in step 3's epilogue
    (the new residual is h + MLP output); otherwise step 3 writes only the scaled MLP
    output and the caller adds it into the residual at the next layer's step 1.
    Dequantisation is done in column chunks of ``n_chunk`` to bound memory.
    """
    h, y = add_rmsnorm(x, r, norm_w, eps)
    gu = _chunked_gemv(bf16_to_f64(y), gu_q, gu_s, n_chunk)
    gu_b = f64_to_bf16(gu)
    I = gu_b.shape[1] // 2
    act = silu_mul(bf16_to_f64(gu_b[:, :I]), bf16_to_f64(gu_b[:, I:]))
    acc = _chunked_gemv(act, d_q, d_s, n_chunk)
    out = f64_to_bf16(_epilogue(acc, out_scale, h if residual_in_epilogue else None))
    return {"h": h, "y": y, "gu": gu_b, "out": out}


def _chunked_gemv(a, qweight, scales, n_chunk=4096):
    """a @ dequant(W), dequantising ``n_chunk`` columns at a time to bound memory."""
    N = qweight.shape[0]
    out = np.empty((a.shape[0], N), dtype=np.float64)
    for c0 in range(0, N, n_chunk):
        c1 = min(N, c0 + n_chunk)
        out[:, c0:c1] = a @ w4_dequant(qweight[c0:c1], scales[:, c0:c1])
    return out


def mlp_chain(x0, r0, layers, *, keep=False):
    """The multi-layer MLP path with the residual add deferred to the next norm.

    For each layer l: (r_{l+1}, y_l) = add_rmsnorm(x_l, r_l); gu_l = bf16(y_l @ W_gu);
    x_{l+1} = bf16(s_l * silu(g_l) u_l @ W_d).  ``layers`` holds objects with fields
    ``norm_w, gate_up.qweight, gate_up.scales, down.qweight, down.scales, out_scale,
    eps``.  Returns (x_L, r_L[, per-layer dicts]).
    """
    x, r = x0, r0
    trace = []
    for L in layers:
        d = mlp_decode(x, r, L.norm_w, L.gate_up.qweight, L.gate_up.scales,
                       L.down.qweight, L.down.scales, L.out_scale, L.eps,
                       residual_in_epilogue=False)
        if keep:
            trace.append(d)
        x, r = d["out"], d["h"]
    return (x, r, trace) if keep else (x, r)


# ----------------------------------------------------------------------------
# the two-kernel layer ([P4] section 5, "the fusion boundary problem": the gate_up GEMM
# with a silu * up epilogue writing act; here the add + RMSNorm also runs as that GEMM's
# prologue, so y_norm and the gate/up pair are never written)
# ----------------------------------------------------------------------------
def add_rmsnorm_gemv_swiglu(x, r, norm_w, gu_q, gu_s, eps=1e-6, *, n_chunk=4096):
    """(h, act): h = bf16(x + r); y = h * w / sqrt(mean_H(h^2) + eps) (not rounded);
    [g, u] = y @ dequant(W_gate_up) (not rounded); act = bf16(silu(g) * u).

    h and act are the only tensors this step writes, so they are the only roundings.
    """
    hs = round_bf16(bf16_to_f64(x) + bf16_to_f64(r))
    H = hs.shape[-1]
    ms = np.sum(hs * hs, axis=-1, keepdims=True) / H
    y = hs * bf16_to_f64(norm_w) / np.sqrt(ms + float(eps))
    gu = _chunked_gemv(y, gu_q, gu_s, n_chunk)
    I = gu.shape[1] // 2
    act = silu_mul(gu[:, :I], gu[:, I:])
    return f64_to_bf16(hs), f64_to_bf16(act)


def w4_gemv_swiglu(x, gu_q, gu_s, *, n_chunk=4096):
    """The gate_up projection with SwiGLU as its epilogue ([P4] section 5, the gate_up GEMM
    with a silu * up epilogue writing act): [g, u] = x @ dequant(W_gate_up), not rounded
    (never written); act = bf16(silu(g) * u).  Columns [0, I) are gate, [I, 2I) up."""
    gu = _chunked_gemv(bf16_to_f64(x), gu_q, gu_s, n_chunk)
    I = gu.shape[1] // 2
    return f64_to_bf16(silu_mul(gu[:, :I], gu[:, I:]))


def mlp_decode2(x, r, norm_w, gu_q, gu_s, d_q, d_s, out_scale=0.5, eps=1e-6,
                residual_in_epilogue=True, *, y_rounded=False, n_chunk=4096):
    """The layer of ``mlp_decode`` with SwiGLU as the gate_up epilogue (gate/up never
    written, act written):

    1. (h, act) = add_rmsnorm_gemv_swiglu(x, r, norm_w, W_gate_up)       (y never written)
       or, with ``y_rounded`` (the norm as its own kernel, which writes y):
       (h, y) = add_rmsnorm(x, r, norm_w); act = w4_gemv_swiglu(y, W_gate_up)
    2. out = bf16(out_scale * act @ dequant(W_down) [+ h])
    """
    if y_rounded:
        h, y = add_rmsnorm(x, r, norm_w, eps)
        act = w4_gemv_swiglu(y, gu_q, gu_s, n_chunk=n_chunk)
    else:
        h, act = add_rmsnorm_gemv_swiglu(x, r, norm_w, gu_q, gu_s, eps, n_chunk=n_chunk)
        y = None
    acc = _chunked_gemv(bf16_to_f64(act), d_q, d_s, n_chunk)
    out = f64_to_bf16(_epilogue(acc, out_scale, h if residual_in_epilogue else None))
    d = {"h": h, "act": act, "out": out}
    if y is not None:
        d["y"] = y
    return d


def mlp_chain2(x0, r0, layers, *, keep=False, y_rounded=False):
    """``mlp_chain`` built from ``mlp_decode2`` (residual add deferred)."""
    x, r = x0, r0
    trace = []
    for L in layers:
        d = mlp_decode2(x, r, L.norm_w, L.gate_up.qweight, L.gate_up.scales,
                        L.down.qweight, L.down.scales, L.out_scale, L.eps,
                        residual_in_epilogue=False, y_rounded=y_rounded)
        if keep:
            trace.append(d)
        x, r = d["out"], d["h"]
    return (x, r, trace) if keep else (x, r)


# ----------------------------------------------------------------------------
# prefill sizes ([P5]: at 2,048 tokens the MLP half is compute-bound and the fusion win
# shrinks): the activation is formed once, rounded to bf16, then multiplied
# ----------------------------------------------------------------------------
def swiglu_act(g, u):
    """act = bf16(silu(g) * u): the fused SwiGLU elementwise pass ([P5] Step 1), one rounding."""
    return f64_to_bf16(silu_mul(bf16_to_f64(g), bf16_to_f64(u)))


def w4_gemm(x, qweight, scales, out_scale=None, residual=None, *, return_f64=False):
    """y = bf16([out_scale *] x @ dequant(W) (+ residual)) for any number of rows."""
    acc = _chunked_gemv(bf16_to_f64(x), qweight, scales)
    y = _epilogue(acc, out_scale, residual)
    return (f64_to_bf16(y), y) if return_f64 else f64_to_bf16(y)


def swiglu_w4_gemm(g, u, qweight, scales, out_scale=1.0, residual=None, *, return_f64=False):
    """The prefill path: y = bf16(out_scale * bf16(silu(g) * u) @ dequant(W) (+ residual)),
    the activation rounded once where the elementwise pass writes it."""
    return w4_gemm(swiglu_act(g, u), qweight, scales, out_scale, residual, return_f64=return_f64)


# ----------------------------------------------------------------------------
# the unfused definitions (self-checks, and references for the unfused GPU sequence)
# ----------------------------------------------------------------------------
def product_buffer_bytes(M, K, N) -> int:
    """Size of the fp32 (M, K, N) broadcast product the unfused form writes ([P1])."""
    return int(np.empty((0,), dtype=np.float32).itemsize) * int(M) * int(K) * int(N)


def product_form_gemv(g, u, qweight, scales, out_scale=1.0, residual=None):
    """[P1]'s decomposition: P[m, k, n] = act[m, k] * w[k, n] materialised, then summed
    over k.  Returns the float64 pre-rounding output (for small shapes only)."""
    act = silu_mul(bf16_to_f64(g), bf16_to_f64(u))
    W = w4_dequant(qweight, scales)
    P = act[:, :, None] * W[None, :, :]
    return _epilogue(P.sum(axis=1), out_scale, residual)


def factored_form_gemv(g, u, qweight, scales, out_scale=1.0, residual=None):
    """Scale factored out of each 128-wide group: sum_g s[g,n] * sum_{k in g} act * q."""
    act = silu_mul(bf16_to_f64(g), bf16_to_f64(u))
    q = w4_unpack(qweight).astype(np.float64)
    s = bf16_to_f64(scales)
    M, K = act.shape
    acc = np.zeros((M, q.shape[1]))
    for gi in range(K // GROUP):
        ks = slice(gi * GROUP, (gi + 1) * GROUP)
        acc += s[gi][None, :] * (act[:, ks] @ q[ks, :])
    return _epilogue(acc, out_scale, residual)


def unfused_act_gemv(g, u, qweight, scales, out_scale=1.0, residual=None):
    """The eager op-by-op sequence with its bf16 round trips ([P5] Step 1, eager SwiGLU
    as two kernels; [P3] the separate scaling launch; [P4] the separate residual add).

    s1 = bf16(silu(g)); act = bf16(s1 * u); z = bf16(act @ W); y = bf16(out_scale * z);
    y = bf16(y + residual) if a residual is given.
    """
    s1 = round_bf16(silu(bf16_to_f64(g)))
    act = round_bf16(s1 * bf16_to_f64(u))
    z = round_bf16(act @ w4_dequant(qweight, scales))
    y = round_bf16(z * (1.0 if out_scale is None else float(out_scale)))
    if residual is not None:
        y = round_bf16(y + bf16_to_f64(residual))
    return f64_to_bf16(y)


def unfused_product_gemv(g, u, qweight, scales, out_scale=1.0):
    """[P1]'s materialised-product sequence, M = 1: the fp32 product is summed over k
    and written as bf16, then a separate launch applies the output scale.  The sum is
    exact here (float64), which the fp32 GPU reduction approximates."""
    z = round_bf16(silu_mul(bf16_to_f64(g), bf16_to_f64(u)) @ w4_dequant(qweight, scales))
    return f64_to_bf16(z * (1.0 if out_scale is None else float(out_scale)))


def add_rmsnorm_eager(x, r, w, eps=1e-6):
    """RMSNorm as the Qwen2 model code spells it after the residual add ([P5] Step 1):
    h = bf16(x + r); rstd = 1/sqrt(mean(h^2) + eps); y = bf16(bf16(h * rstd) * w)."""
    hs = round_bf16(bf16_to_f64(x) + bf16_to_f64(r))
    ms = np.mean(hs * hs, axis=-1, keepdims=True)
    t = round_bf16(hs / np.sqrt(ms + float(eps)))
    y = round_bf16(t * bf16_to_f64(w))
    return f64_to_bf16(hs), f64_to_bf16(y)


# ----------------------------------------------------------------------------
# FP4 weights with E4M3 block scales ([P3]: packed FP4 inputs with E4M3 1x16 block
# scales and a zero-dimensional fp32 output multiplier folded into the GEMM)
# ----------------------------------------------------------------------------
FP4_BLOCK = 16    # weights per E4M3 block scale along K

# E2M1: one sign bit, two exponent bits, one mantissa bit.  The magnitudes of codes
# 0..7 (sign bit clear), in code order: exponent field 0 holds zero and the single
# subnormal 0.5; fields 1..3 hold 1, 1.5, 2, 3, 4, 6.
_E2M1_MAGNITUDE = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def e2m1_decode(codes) -> np.ndarray:
    """E2M1 codes 0..15 -> float64; bit 3 is the sign (code 8 is -0)."""
    c = np.asarray(codes).astype(np.int64)
    mag = _E2M1_MAGNITUDE[c & 7]
    return np.where((c & 8) != 0, -mag, mag)


def e4m3_decode(codes) -> np.ndarray:
    """E4M3 byte codes -> float64.  Sign bit 7, exponent bits 6..3 (bias 7), mantissa
    bits 2..0.  Exponent field 0: subnormal m/8 * 2**-6.  No infinities: exponent 15
    with mantissa 7 is NaN, every other code is finite (largest 448)."""
    c = np.asarray(codes).astype(np.int64)
    sign = np.where((c & 0x80) != 0, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    val = np.where((e == 15) & (c & 7 == 7), np.nan, val)
    return sign * val


def fp4_unpack(qweight) -> np.ndarray:
    """Packed words uint32 [N, K/8] -> E2M1 codes uint8 [K, N] (code of k = 8*kb + j in
    bits [4j, 4j+4) of word (n, kb))."""
    w = np.asarray(qweight, dtype=np.uint32)
    n, kb = w.shape
    out = np.empty((kb, NIB, n), dtype=np.uint8)
    for j in range(NIB):
        out[:, j, :] = ((w >> np.uint32(4 * j)) & np.uint32(0xF)).astype(np.uint8).T
    return out.reshape(kb * NIB, n)


def fp4_dequant(qweight, scales) -> np.ndarray:
    """Dequantised weights, float64 [K, N]: w[k, n] = e2m1(code[k, n]) * e4m3(s[n, k // 16]).

    An E2M1 value has 2 significant bits and an E4M3 value 4, so the product is exact in
    fp32 (and in fp16 up to the range) on the GPU."""
    v = e2m1_decode(fp4_unpack(qweight))
    s = e4m3_decode(scales)
    K = v.shape[0]
    if s.shape[1] * FP4_BLOCK != K or s.shape[0] != v.shape[1]:
        raise ValueError("scales must be [N, K/16]")
    return v * np.repeat(s.T, FP4_BLOCK, axis=0)


def _chunked_fp4_gemv(a, qweight, scales, n_chunk=2048):
    """a [M, K] float64 times fp4_dequant(W) [K, N], N in chunks (bounded memory)."""
    N = qweight.shape[0]
    sc = np.asarray(scales)
    out = np.empty((a.shape[0], N), dtype=np.float64)
    for n0 in range(0, N, n_chunk):
        n1 = min(N, n0 + n_chunk)
        out[:, n0:n1] = a @ fp4_dequant(qweight[n0:n1], sc[n0:n1])
    return out


def swiglu_fp4_gemv(g, u, qweight, scales, out_scale=1.0, residual=None, *, return_f64=False):
    """y[m, n] = bf16(out_scale * sum_k silu(g[m,k]) u[m,k] w[k,n] (+ residual[m, n]))
    with FP4 weights w = e2m1 * e4m3 block scale ([P3]); the activation is unrounded."""
    act = silu_mul(bf16_to_f64(g), bf16_to_f64(u))
    acc = _chunked_fp4_gemv(act, qweight, scales)
    y = _epilogue(acc, out_scale, residual)
    return (f64_to_bf16(y), y) if return_f64 else f64_to_bf16(y)


def fp4_gemv(x, qweight, scales, out_scale=None, residual=None, *, return_f64=False):
    """The same GEMV with the identity prologue: y = bf16([out_scale *] x @ W (+ residual))."""
    acc = _chunked_fp4_gemv(bf16_to_f64(x), qweight, scales)
    y = _epilogue(acc, out_scale, residual)
    return (f64_to_bf16(y), y) if return_f64 else f64_to_bf16(y)


# ----------------------------------------------------------------------------
# FP4 activations ([P3]: the scaled matmul takes packed FP4 for both of its inputs, each
# with E4M3 1x16 block scales; the zero-dimensional fp32 multiplier carries what the
# block scales do not, here the activation's per-tensor scale G times the weights').
# The activation is quantised at run time with a given per-tensor scale G (a calibrated
# constant), one E4M3 scale per 16 values along K:
#     s_b = e4m3(amax_b / (6 G))                 amax_b: the block's largest magnitude
#     q_k = e2m1(x_k / (s_b G)), 0 where s_b = 0
# each step an fp32 operation (the precision the kernels decide in), both roundings to
# nearest with ties to the even code, saturating (E4M3 at 448, E2M1 at 6).  The GEMM
# then multiplies the exact values q_k s_b by the FP4 weights.
# ----------------------------------------------------------------------------
_E4M3_FINITE = e4m3_decode(np.arange(127))      # codes 0..126: 0 .. 448, increasing


def e4m3_encode(t) -> np.ndarray:
    """Non-negative values -> E4M3 codes 0..126: the nearest finite E4M3 value, ties to
    the even code, 448 for everything above it."""
    t = np.asarray(t, dtype=np.float64)
    i = np.clip(np.searchsorted(_E4M3_FINITE, t), 1, 126)         # _E4M3_FINITE[i - 1] < t <= [i]
    lo, hi = _E4M3_FINITE[i - 1], _E4M3_FINITE[i]
    up = (hi - t < t - lo) | ((hi - t == t - lo) & (i % 2 == 0))
    code = np.where(up, i, i - 1)
    code = np.where(t >= 448.0, 126, np.where(t <= 0.0, 0, code))
    return code.astype(np.uint8)


def e2m1_encode(y) -> np.ndarray:
    """Values -> E2M1 codes 0..15: the magnitude to the nearest E2M1 magnitude, ties to the
    even code, 6 for everything above it; bit 3 is the value's sign bit."""
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    i = np.clip(np.searchsorted(_E2M1_MAGNITUDE, a), 1, 7)
    lo, hi = _E2M1_MAGNITUDE[i - 1], _E2M1_MAGNITUDE[i]
    up = (hi - a < a - lo) | ((hi - a == a - lo) & (i % 2 == 0))
    code = np.where(a >= 6.0, 7, np.where(up, i, i - 1))
    return (code | np.where(np.signbit(y), 8, 0)).astype(np.uint8)


def nvfp4_quantize(x, global_scale):
    """x float32 [M, K] (K % 16 == 0), per-tensor scale G > 0 -> (E2M1 codes uint8 [M, K],
    E4M3 block-scale codes uint8 [M, K/16]), every step in fp32 as described above."""
    x = np.asarray(x, dtype=np.float32)
    G = np.float32(global_scale)
    M, K = x.shape
    if K % FP4_BLOCK:
        raise ValueError("K must be a multiple of 16")
    xb = x.reshape(M, K // FP4_BLOCK, FP4_BLOCK)
    amax = np.max(np.abs(xb), axis=-1)                      # float32
    sc = e4m3_encode(amax / (np.float32(6.0) * G))           # float32 quotient, then E4M3
    s = e4m3_decode(sc).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        y = xb / (s * G)[..., None]                          # float32 product, float32 quotient
    codes = np.where(s[..., None] > 0, e2m1_encode(y), 0)
    return codes.reshape(M, K).astype(np.uint8), sc


def nvfp4_dequant(codes, scale_codes) -> np.ndarray:
    """float64 [M, K]: e2m1(code[m, k]) * e4m3(scale[m, k // 16]) (exact)."""
    s = e4m3_decode(scale_codes)
    return e2m1_decode(codes) * np.repeat(s, FP4_BLOCK, axis=-1)


def fp4a4_gemv(x, qweight, scales, act_global_scale, out_scale=None, residual=None, *, return_f64=False):
    """Both operands FP4 ([P3]'s scaled matmul): x (bf16 [M, K]) quantised with
    nvfp4_quantize, then y = bf16([out_scale *] sum_k xq[m, k] w[k, n] (+ residual)) with
    xq = e2m1 * e4m3 (without G: the output multiplier carries it) and the FP4 weights."""
    codes, sc = nvfp4_quantize(bf16_to_f64(x).astype(np.float32), act_global_scale)
    acc = _chunked_fp4_gemv(nvfp4_dequant(codes, sc), qweight, scales)
    y = _epilogue(acc, out_scale, residual)
    return (f64_to_bf16(y), y) if return_f64 else f64_to_bf16(y)


def swiglu_fp4a4_gemv(g, u, qweight, scales, act_global_scale, out_scale=1.0, residual=None, *,
                      return_f64=False):
    """The same with the SwiGLU prologue: act = silu(g) * u, rounded to fp32 (the
    precision the quantisation decides in), then quantised and multiplied as above."""
    act = silu_mul(bf16_to_f64(g), bf16_to_f64(u)).astype(np.float32)
    codes, sc = nvfp4_quantize(act, act_global_scale)
    acc = _chunked_fp4_gemv(nvfp4_dequant(codes, sc), qweight, scales)
    y = _epilogue(acc, out_scale, residual)
    return (f64_to_bf16(y), y) if return_f64 else f64_to_bf16(y)
