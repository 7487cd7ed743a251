"""Algorithmic HBM bytes per call of each entry point.

"Algorithmic" bytes are what the operation must move at minimum: packed int4 weights,
bf16 group scales, activations read, outputs written and the 4-byte fp32 output
scale.  They exclude anything a fused kernel avoids (dense weights, the (M, K, N)
product, the SwiGLU activation) and its own small split-K partials.  Dividing them by
the measured time gives the effective bandwidth the kernel-fusion measurement article
("Kernel Fusion, torch.compile and CUDA Graphs, Measured", Measured section) reports:
the job's bytes over time, not the traffic the hardware actually served.

The unfused sequences are counted kernel by kernel, the way that article's Step 1
counts the nine eager kernels of the Qwen2 residual add + RMSNorm (42 bytes per
element against 8 for one fused kernel) and the two eager SwiGLU kernels (10 bytes per
element against 6).
"""
from __future__ import annotations

BF16 = 2
F32 = 4
GROUP = 128


def w4_weight_bytes(K: int, N: int) -> int:
    """Packed int4 weights (K*N/2) plus bf16 group scales ((K/128)*N*2)."""
    return K * N // 2 + (K // GROUP) * N * BF16


def swiglu_w4_gemv_bytes(M: int, K: int, N: int, residual: bool = False,
                         out_scale: bool = True) -> int:
    """g and u in, y out (+ residual in), weights, and the fp32 scalar."""
    b = w4_weight_bytes(K, N) + 2 * M * K * BF16 + M * N * BF16
    if residual:
        b += M * N * BF16
    if out_scale:
        b += F32
    return b


def w4_gemv_bytes(M: int, K: int, N: int, out_scale: bool = False) -> int:
    """Identity-prologue GEMV (the gate_up projection): x in, y out, weights."""
    return w4_weight_bytes(K, N) + M * K * BF16 + M * N * BF16 + (F32 if out_scale else 0)


def fp4_weight_bytes(K: int, N: int) -> int:
    """Packed E2M1 weights (K*N/2) plus E4M3 block scales, one byte per 16 along K."""
    return K * N // 2 + (K // 16) * N


def swiglu_fp4_gemv_bytes(M: int, K: int, N: int, residual: bool = False, out_scale: bool = True) -> int:
    """The SwiGLU-prologue GEMV with FP4 weights: g and u in, y out (+ residual), weights,
    and the fp32 scalar."""
    b = fp4_weight_bytes(K, N) + 2 * M * K * BF16 + M * N * BF16
    if residual:
        b += M * N * BF16
    if out_scale:
        b += F32
    return b


def add_rmsnorm_bytes(M: int, H: int) -> int:
    """x and residual in, h and y out (8 bytes per element), plus the weight vector."""
    return 4 * M * H * BF16 + H * BF16


def add_rmsnorm_eager_bytes(M: int, H: int) -> int:
    """The nine-kernel eager sequence, per element: add (2+2 in, 2 out), cast to fp32
    (2 in, 4 out), square (4+4), mean (4 in), multiply by rstd (4+4), cast to bf16
    (4 in, 2 out), multiply by the weight (2 in, 2 out) = 42 bytes; the per-row kernels
    (mean's output, + eps, rsqrt) move 4 bytes per row each way, and the weight vector
    is read once."""
    per_elem = 6 + 6 + 8 + 4 + 8 + 6 + 4
    per_row = F32 + 2 * F32 + 2 * F32 + F32      # mean out; +eps in/out; rsqrt in/out; mul reads rstd
    return per_elem * M * H + per_row * M + H * BF16


def mlp_layer_bytes(M: int, H: int, I: int, residual_in_epilogue: bool) -> int:
    """add_rmsnorm + gate_up GEMV (K=H, N=2I) + SwiGLU-down GEMV (K=I, N=H)."""
    return (add_rmsnorm_bytes(M, H) + w4_gemv_bytes(M, H, 2 * I)
            + swiglu_w4_gemv_bytes(M, I, H, residual=residual_in_epilogue))


def w4_gemv_swiglu_bytes(M: int, K: int, I: int) -> int:
    """The gate_up projection with the SwiGLU epilogue: x in, gate_up weights [K, 2I],
    act [M, I] out (the gate/up pair is never written)."""
    return w4_weight_bytes(K, 2 * I) + M * K * BF16 + M * I * BF16


def mlp2_layer_bytes(M: int, H: int, I: int, residual_in_epilogue: bool) -> int:
    """The layer with SwiGLU as the gate_up epilogue.

    Up to 4 rows, two kernels.  Kernel 1: x, residual and the norm weight in, gate_up
    weights, h and act out.  Kernel 2: act in, down weights, out out (+ h in for the
    residual add), the fp32 scalar, and the residual update (h in, residual out).
    From 5 rows, three kernels: add_rmsnorm; the gate_up GEMV with the SwiGLU epilogue;
    the down GEMV on act (+ the residual, which the norm updated in place)."""
    if M > 4:
        down = w4_gemv_bytes(M, I, H, out_scale=True) + (M * H * BF16 if residual_in_epilogue else 0)
        return add_rmsnorm_bytes(M, H) + w4_gemv_swiglu_bytes(M, H, I) + down
    k1 = 2 * M * H * BF16 + H * BF16 + w4_weight_bytes(H, 2 * I) + M * H * BF16 + M * I * BF16
    k2 = M * I * BF16 + w4_weight_bytes(I, H) + M * H * BF16 + F32 + 2 * M * H * BF16
    if residual_in_epilogue:
        k2 += M * H * BF16
    return k1 + k2


def product_bytes(M: int, K: int, N: int) -> int:
    """The fp32 (M, K, N) broadcast product the unfused single-row path materialises."""
    return M * K * N * F32


def unfused_product_gemv_bytes(K: int, N: int) -> int:
    """M = 1.  Product kernel (g, u, weights in; product out), reduction (product in,
    bf16 out), separate scale launch (bf16 in, scalar in, bf16 out)."""
    return (2 * K * BF16 + w4_weight_bytes(K, N) + product_bytes(1, K, N)
            + product_bytes(1, K, N) + N * BF16
            + N * BF16 + F32 + N * BF16)


def unfused_act_gemv_bytes(M: int, K: int, N: int, residual: bool = False) -> int:
    """silu (g in, s out), mul (s, u in, act out), GEMV (act, weights in, z out),
    scale (z, scalar in, y out), and a residual add (y, r in, y out) if present."""
    b = (2 * M * K * BF16) + (3 * M * K * BF16) + (M * K * BF16 + w4_weight_bytes(K, N)
                                                   + M * N * BF16) + (2 * M * N * BF16 + F32)
    if residual:
        b += 3 * M * N * BF16
    return b
