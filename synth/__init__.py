"""Seeded synthetic inputs for the fused decode-MLP path.

This module only draws random numbers and packs them into the storage formats the
library takes. It holds none of the method's arithmetic (no SiLU, no dequantisation,
no normalisation, no matrix products), so both the fp64 oracle and the GPU path can be
fed from it without sharing any computation.

Storage formats produced here:

* bf16 tensors are ``numpy.uint16`` arrays of bf16 bit patterns.  Values are drawn in
  fp32 and rounded to bf16 (round to nearest, ties to even) by PyTorch's own
  ``float32 -> bfloat16`` conversion.
* int4 weights are ``numpy.uint32`` arrays of shape ``[N, K/8]`` (row-major, the
  orientation of a linear layer's ``[out_features, in_features]`` weight, so the K
  values of one output column are contiguous).  Word ``(n, kb)`` holds the eight
  weights ``k = 8*kb + j`` (j = 0..7) of column ``n``; weight ``j`` sits in bits
  ``[4j, 4j+4)`` as a two's-complement nibble, so values span ``[-8, 7]``.  Drawing
  every word uniformly over all 2**32 patterns draws every nibble independently and
  uniformly over its 16 codes, i.e. every weight uniformly over ``[-8, 7]``.
* group scales are bf16 ``[K/128, N]`` (row-major), scale ``(g, n)`` applying to
  ``k`` in ``[128 g, 128 g + 128)``, drawn uniformly from ``[0.005, 0.02)``.

Seeding: ``numpy.random.SeedSequence(seed)`` is spawned into one child per tensor, in
the fixed order documented by each generator, so every tensor of a workload is
reproducible on its own and independent of the others.  Multi-layer workloads spawn
one child per layer and then one grandchild per tensor of that layer.

Workload shapes follow the pages: the int4 SwiGLU GEMV at K=9216, N=2560 (the
PyTorch issue about the materialised (1,K,N) product), the 8,192 x 4,096 bf16
add+RMSNorm tensor (the kernel-fusion measurement article), a Llama-3-8B-sized MLP
(hidden 4096, width 14336, the torch.compile chapter) and a Qwen2.5-1.5B-sized MLP
(hidden 1536, width 8960, 28 layers, the kernel-fusion article's decode step).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

GROUP = 128          # int4 group size along K
PACK = 8             # int4 values per uint32 word

SCALE_LO = 0.005
SCALE_HI = 0.02


# ----------------------------------------------------------------------------
# storage helpers (format conversion only)
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns via PyTorch's RNE conversion."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def pack_int4(q: np.ndarray) -> np.ndarray:
    """Pack int values in [-8, 7], shape [K, N] with K % 8 == 0, into uint32 [N, K/8].

    Used to build hand-made weight matrices for tests; random workloads draw the
    packed words directly.
    """
    q = np.asarray(q)
    if q.ndim != 2 or q.shape[0] % PACK:
        raise ValueError("pack_int4 wants [K, N] with K % 8 == 0")
    if q.min(initial=0) < -8 or q.max(initial=0) > 7:
        raise ValueError("int4 values must lie in [-8, 7]")
    codes = (q.astype(np.int64) & 0xF).astype(np.uint32)          # two's complement nibble
    codes = codes.reshape(q.shape[0] // PACK, PACK, q.shape[1])    # [kb, j, n]
    words = np.zeros((q.shape[1], q.shape[0] // PACK), dtype=np.uint32)
    for j in range(PACK):
        words |= codes[:, j, :].T << np.uint32(4 * j)
    return words


def _children(seed: int, n: int):
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(n)]


def _normal_bf16(rng, shape, mean=0.0, std=1.0):
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0 or mean != 0.0:
        a = a * np.float32(std) + np.float32(mean)
    return f32_to_bf16_bits(a)


def _scales_bf16(rng, shape):
    a = rng.uniform(SCALE_LO, SCALE_HI, size=shape).astype(np.float32)
    return f32_to_bf16_bits(a)


def _qweight(rng, K, N):
    return rng.integers(0, 2**32, size=(N, K // PACK), dtype=np.uint32)


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------
@dataclass
class W4:
    qweight: np.ndarray   # uint32 [N, K/8]
    scales: np.ndarray    # uint16 (bf16 bits) [K/128, N]

    @property
    def K(self):
        return self.qweight.shape[1] * PACK

    @property
    def N(self):
        return self.qweight.shape[0]


def w4_weight(rng, K, N) -> W4:
    """One int4 matrix: qweight drawn first, then scales, from the same generator."""
    if K % GROUP or N <= 0:
        raise ValueError("K must be a multiple of 128")
    return W4(_qweight(rng, K, N), _scales_bf16(rng, (K // GROUP, N)))


@dataclass
class GemvInputs:
    g: np.ndarray          # bf16 bits [M, K]
    u: np.ndarray          # bf16 bits [M, K]
    W: W4
    out_scale: float
    residual: np.ndarray | None = None   # bf16 bits [M, N]


def swiglu_gemv_inputs(M: int, K: int, N: int, seed: int = 0, out_scale: float = 1.0,
                       with_residual: bool = False) -> GemvInputs:
    """Children in order: g, u, weights (qweight then scales), residual."""
    rg, ru, rw, rr = _children(seed, 4)
    g = _normal_bf16(rg, (M, K))
    u = _normal_bf16(ru, (M, K))
    W = w4_weight(rw, K, N)
    res = _normal_bf16(rr, (M, N)) if with_residual else None
    return GemvInputs(g, u, W, float(out_scale), res)


# ----------------------------------------------------------------------------
# FP4 weights with E4M3 block scales
# ----------------------------------------------------------------------------
FP4_BLOCK = 16       # FP4 weights per E4M3 block scale along K


def f32_to_e4m3_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> E4M3 ('fn': no infinities) byte codes via PyTorch's RNE conversion."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


@dataclass
class FP4:
    qweight: np.ndarray   # uint32 [N, K/8]: eight E2M1 codes per word, code j in bits [4j, 4j+4)
    scales: np.ndarray    # uint8 (E4M3 codes) [N, K/16]: the scales of a column are contiguous

    @property
    def K(self):
        return self.qweight.shape[1] * PACK

    @property
    def N(self):
        return self.qweight.shape[0]


def fp4_weight(rng, K, N) -> FP4:
    """One FP4 matrix: words uniform over all 2**32 patterns (every E2M1 code, -0
    included, equally likely), then block scales drawn from U[0.005, 0.02) and rounded
    to E4M3, from the same generator."""
    if K % 32 or N <= 0:
        raise ValueError("K must be a multiple of 32")
    q = _qweight(rng, K, N)
    sc = f32_to_e4m3_bits(rng.uniform(SCALE_LO, SCALE_HI, size=(N, K // FP4_BLOCK)).astype(np.float32))
    return FP4(q, sc)


@dataclass
class Fp4GemvInputs:
    g: np.ndarray          # bf16 bits [M, K]
    u: np.ndarray          # bf16 bits [M, K]
    W: FP4
    out_scale: float
    residual: np.ndarray | None = None   # bf16 bits [M, N]


def swiglu_fp4_gemv_inputs(M: int, K: int, N: int, seed: int = 0, out_scale: float = 1.0,
                           with_residual: bool = False) -> Fp4GemvInputs:
    """Children in order: g, u, weights (words then block scales), residual."""
    rg, ru, rw, rr = _children(seed, 4)
    g = _normal_bf16(rg, (M, K))
    u = _normal_bf16(ru, (M, K))
    W = fp4_weight(rw, K, N)
    res = _normal_bf16(rr, (M, N)) if with_residual else None
    return Fp4GemvInputs(g, u, W, float(out_scale), res)


@dataclass
class NormInputs:
    x: np.ndarray          # bf16 bits [M, H]
    r: np.ndarray          # bf16 bits [M, H]
    w: np.ndarray          # bf16 bits [H]
    eps: float


def add_rmsnorm_inputs(M: int, H: int, seed: int = 0, eps: float = 1e-6) -> NormInputs:
    """Children in order: x, residual, weight.  x, r ~ N(0,1); weight ~ N(1, 0.1)."""
    rx, rr, rw = _children(seed, 3)
    return NormInputs(_normal_bf16(rx, (M, H)), _normal_bf16(rr, (M, H)),
                      _normal_bf16(rw, (H,), mean=1.0, std=0.1), float(eps))


@dataclass
class MlpLayer:
    norm_w: np.ndarray     # bf16 bits [H]
    gate_up: W4            # K = H, N = 2I (gate columns [0, I), up columns [I, 2I))
    down: W4               # K = I, N = H
    out_scale: float
    eps: float


@dataclass
class MlpInputs:
    x: np.ndarray          # bf16 bits [M, H]
    r: np.ndarray          # bf16 bits [M, H]
    layers: list = field(default_factory=list)


def mlp_inputs(M: int, H: int, I: int, n_layers: int = 1, seed: int = 0,
               out_scale: float = 0.5, eps: float = 1e-6) -> MlpInputs:
    """Children in order: x, residual, then one child per layer.

    Each layer child is spawned into: norm weight, gate_up weights, down weights.
    """
    ss = np.random.SeedSequence(seed)
    kids = ss.spawn(2 + n_layers)
    rx, rr = (np.random.default_rng(k) for k in kids[:2])
    x = _normal_bf16(rx, (M, H))
    r = _normal_bf16(rr, (M, H))
    layers = []
    for lk in kids[2:]:
        rn, rgu, rd = (np.random.default_rng(k) for k in lk.spawn(3))
        layers.append(MlpLayer(_normal_bf16(rn, (H,), mean=1.0, std=0.1),
                               w4_weight(rgu, H, 2 * I), w4_weight(rd, I, H),
                               float(out_scale), float(eps)))
    return MlpInputs(x, r, layers)


# ----------------------------------------------------------------------------
# the five named workloads
# ----------------------------------------------------------------------------
CONFIGS = {
    "swiglu_w4_gemv_1x1024x512": dict(kind="gemv", M=1, K=1024, N=512, out_scale=0.5),
    "swiglu_w4_gemv_1x9216x2560": dict(kind="gemv", M=1, K=9216, N=2560, out_scale=1.0),
    "add_rmsnorm_8192x4096": dict(kind="norm", M=8192, H=4096, eps=1e-6),
    "mlp_llama3_8b_m16": dict(kind="mlp", M=16, H=4096, I=14336, n_layers=1,
                              out_scale=0.5, eps=1e-6, residual_in_epilogue=True),
    "mlp_qwen2_5_1_5b_28l": dict(kind="mlp", M=1, H=1536, I=8960, n_layers=28,
                                 out_scale=0.5, eps=1e-6, residual_in_epilogue=False),
}


def make(name: str, seed: int = 0):
    c = CONFIGS[name]
    if c["kind"] == "gemv":
        return swiglu_gemv_inputs(c["M"], c["K"], c["N"], seed, c["out_scale"])
    if c["kind"] == "norm":
        return add_rmsnorm_inputs(c["M"], c["H"], seed, c["eps"])
    return mlp_inputs(c["M"], c["H"], c["I"], c["n_layers"], seed, c["out_scale"], c["eps"])
