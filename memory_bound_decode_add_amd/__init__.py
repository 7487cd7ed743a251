"""fdec: fused decode-MLP kernels for AMD MI355X (gfx950) -- the Python binding.

A thin ctypes layer over ``libfdec.so`` (built by ``python -m
memory_bound_decode_add_amd.build``).  It only marshals arguments: it checks tensor
dtypes, devices and sizes, passes raw device pointers and the current HIP stream, and
turns a non-zero status into :class:`FdecError`.  Every step of the computation runs in
the library's HIP kernels; there is no fallback.  PyTorch provides device memory and
streams.

bf16 tensors are ``torch.bfloat16``; packed int4 weights are ``torch.int32`` tensors
of shape ``[N, K/8]`` holding the uint32 words bit for bit (see ``fdec.h``); group
scales are ``torch.bfloat16`` ``[K/128, N]``.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np
import torch

from . import traffic  # noqa: F401  (byte models)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfdec.so")

FDEC_OK = 0
UNFUSED_PRODUCT = 0
UNFUSED_ACT = 1

_c_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t


class FdecError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


class FdecNotBuilt(RuntimeError):
    pass


class CW4(ctypes.Structure):
    _fields_ = [("qweight", _c_p), ("scales", _c_p), ("K", _i32), ("N", _i32)]


class CFP4(ctypes.Structure):
    _fields_ = [("qweight", _c_p), ("scales", _c_p), ("K", _i32), ("N", _i32)]


class CLayer(ctypes.Structure):
    _fields_ = [("norm_weight", _c_p), ("eps", ctypes.c_float), ("gate_up", CW4), ("down", CW4),
                ("out_scale", _c_p), ("residual_in_epilogue", _i32)]


# name: (restype, argtypes)
_SIGS = {
    "fdec_abi_version": (ctypes.c_int, []),
    "fdec_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "fdec_last_error": (ctypes.c_char_p, []),
    "fdec_workspace_init": (ctypes.c_int, [_c_p, _sz, _c_p]),
    "fdec_add_rmsnorm": (ctypes.c_int, [_c_p, _c_p, _c_p, ctypes.c_float, _i32, _i32, _c_p, _c_p, _c_p]),
    "fdec_w4_gemv_workspace_bytes": (_sz, [_i32, _i32, _i32]),
    "fdec_swiglu_w4_gemv": (ctypes.c_int, [_c_p, _c_p, _i64, ctypes.POINTER(CW4), _c_p, _c_p, _i32, _c_p,
                                           _c_p, _sz, _c_p]),
    "fdec_w4_gemv": (ctypes.c_int, [_c_p, ctypes.POINTER(CW4), _c_p, _i32, _c_p, _c_p, _sz, _c_p]),
    "fdec_swiglu_w4_gemv_noalloc": (ctypes.c_int, [_c_p, _c_p, _i64, ctypes.POINTER(CW4), _c_p, _c_p, _i32, _c_p,
                                                   _c_p]),
    "fdec_mlp_workspace_bytes": (_sz, [_i32, _i32, _i32]),
    "fdec_mlp_decode": (ctypes.c_int, [ctypes.POINTER(CLayer), _i32, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _sz,
                                       _c_p]),
    "fdec_mlp_chain": (ctypes.c_int, [ctypes.POINTER(CLayer), _i32, _i32, _c_p, _c_p, _c_p, _c_p, _c_p, _sz,
                                      _c_p]),
    "fdec_mlp_graph_create": (ctypes.c_int, [ctypes.POINTER(CLayer), _i32, _i32, _c_p, _c_p, _c_p, _c_p, _c_p,
                                             _sz, _c_p, ctypes.POINTER(_c_p)]),
    "fdec_add_rmsnorm_w4_gemv_swiglu": (ctypes.c_int, [_c_p, _c_p, _c_p, ctypes.c_float, ctypes.POINTER(CW4), _i32,
                                                       _c_p, _c_p, _c_p]),
    "fdec_mlp2_workspace_bytes": (_sz, [_i32, _i32, _i32]),
    "fdec_w4_gemv_swiglu_workspace_bytes": (_sz, [_i32, _i32, _i32]),
    "fdec_swiglu": (ctypes.c_int, [_c_p, _c_p, _i64, _i32, _i32, _c_p, _c_p]),
    "fdec_w4_gemm": (ctypes.c_int, [_c_p, ctypes.POINTER(CW4), _c_p, _c_p, _i32, _c_p, _c_p]),
    "fdec_swiglu_w4_gemm_workspace_bytes": (_sz, [_i32, _i32]),
    "fdec_swiglu_w4_gemm": (ctypes.c_int, [_c_p, _c_p, _i64, ctypes.POINTER(CW4), _c_p, _c_p, _i32, _c_p, _c_p,
                                           _sz, _c_p]),
    "fdec_w4_gemv_swiglu": (ctypes.c_int, [_c_p, ctypes.POINTER(CW4), _i32, _c_p, _c_p, _sz, _c_p]),
    "fdec_mlp_decode2": (ctypes.c_int, [ctypes.POINTER(CLayer), _i32, _c_p, _c_p, _c_p, _c_p, _c_p, _sz, _c_p]),
    "fdec_mlp_chain2": (ctypes.c_int, [ctypes.POINTER(CLayer), _i32, _i32, _c_p, _c_p, _c_p, _c_p, _sz, _c_p]),
    "fdec_mlp_graph_create2": (ctypes.c_int, [ctypes.POINTER(CLayer), _i32, _i32, _c_p, _c_p, _c_p, _c_p, _sz,
                                              _c_p, ctypes.POINTER(_c_p)]),
    "fdec_mlp_graph_update": (ctypes.c_int, [_c_p, ctypes.POINTER(CLayer), _i32, _i32, _c_p, _c_p, _c_p, _c_p,
                                             _c_p, _sz, _c_p]),
    "fdec_mlp_graph_update2": (ctypes.c_int, [_c_p, ctypes.POINTER(CLayer), _i32, _i32, _c_p, _c_p, _c_p, _c_p,
                                              _sz, _c_p]),
    "fdec_graph_launch": (ctypes.c_int, [_c_p, _c_p]),
    "fdec_graph_kernel_count": (ctypes.c_int, [_c_p]),
    "fdec_graph_destroy": (ctypes.c_int, [_c_p]),
    "fdec_unfused_gemv_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32]),
    "fdec_unfused_swiglu_w4_gemv": (ctypes.c_int, [_i32, _c_p, _c_p, _i64, ctypes.POINTER(CW4), _c_p, _c_p, _i32,
                                                   _c_p, _c_p, _sz, _c_p]),
    "fdec_unfused_add_rmsnorm_workspace_bytes": (_sz, [_i32, _i32]),
    "fdec_unfused_add_rmsnorm": (ctypes.c_int, [_c_p, _c_p, _c_p, ctypes.c_float, _i32, _i32, _c_p, _c_p, _c_p,
                                                _sz, _c_p]),
    "fdec_unfused_mlp_workspace_bytes": (_sz, [_i32, _i32, _i32]),
    "fdec_unfused_mlp_decode": (ctypes.c_int, [ctypes.POINTER(CLayer), _i32, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p,
                                               _sz, _c_p]),
    "fdec_w4_unpack": (ctypes.c_int, [ctypes.POINTER(CW4), _c_p, _c_p]),
    "fdec_w4_dequant": (ctypes.c_int, [ctypes.POINTER(CW4), _c_p, _c_p]),
    "fdec_fp4_gemv_workspace_bytes": (_sz, [_i32, _i32, _i32]),
    "fdec_swiglu_fp4_gemv": (ctypes.c_int, [_c_p, _c_p, _i64, ctypes.POINTER(CFP4), _c_p, _c_p, _i32, _c_p,
                                            _c_p, _sz, _c_p]),
    "fdec_fp4_gemv": (ctypes.c_int, [_c_p, ctypes.POINTER(CFP4), _c_p, _c_p, _i32, _c_p, _c_p, _sz, _c_p]),
    "fdec_fp4_dequant": (ctypes.c_int, [ctypes.POINTER(CFP4), _c_p, _c_p]),
    "fdec_swiglu_fp4a4_gemv": (ctypes.c_int, [_c_p, _c_p, _i64, ctypes.POINTER(CFP4), _c_p, _c_p, _c_p, _i32, _c_p,
                                              _c_p, _sz, _c_p]),
    "fdec_fp4a4_gemv": (ctypes.c_int, [_c_p, ctypes.POINTER(CFP4), _c_p, _c_p, _c_p, _i32, _c_p, _c_p, _sz, _c_p]),
    "fdec_nvfp4_quantize": (ctypes.c_int, [_c_p, _i64, _i32, _i32, _c_p, _c_p, _c_p, _c_p]),
    # include/fdec_test.h
    "fdec_set_gemv_split": (None, [_i32]),
    "fdec_set_gemv_tiling": (None, [_i32, _i32]),
    "fdec_test_fail_launches": (None, [_i32]),
    "fdec_set_mfma_plan": (None, [_i32, _i32, _i32]),
    "fdec_set_kmfma_waves": (None, [_i32]),
    "fdec_test_gemv_workspace_bytes": (_sz, [_i32, _i32, _i32]),
    "fdec_test_gemv_kernel": (_i32, [_i32, _i32, _i32, _i32]),
    "fdec_test_mlp_workspace_bytes": (_sz, [_i32, _i32, _i32]),
    "fdec_test_empty_kernel": (ctypes.c_int, [_i32, _i32, _c_p]),
    "fdec_test_read_ceiling": (ctypes.c_int, [_c_p, _sz, _i32, _c_p, _c_p, _sz, _c_p, _sz, _i32, _i32, _i32, _i32,
                                              _c_p, _c_p]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises FdecNotBuilt if libfdec.so is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise FdecNotBuilt(f"{LIB_PATH} is missing: run `python -m memory_bound_decode_add_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def exported_symbols():
    return list(_SIGS)


def _check(status: int):
    if status != FDEC_OK:
        msg = lib().fdec_last_error().decode(errors="replace")
        raise FdecError(status, msg or lib().fdec_status_str(status).decode())


def _stream(device=None) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _need(t, name, dtype, shape=None, numel=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} is too small")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _rows(t, name, M, K):
    """A [M, K] bf16 view whose rows may be strided (e.g. a column slice); returns ld."""
    if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or t.device.type != "cuda":
        raise TypeError(f"{name} must be a bf16 GPU tensor")
    if t.dim() != 2 or tuple(t.shape) != (M, K) or t.stride(1) != 1:
        raise ValueError(f"{name} must be a [M, K] = [{M}, {K}] view with unit column stride")
    return t.stride(0) if M > 1 else max(K, t.stride(0))


# ----------------------------------------------------------------------------
# bf16 bit-pattern helpers (host <-> device)
# ----------------------------------------------------------------------------
def from_bits(a: np.ndarray, device="cuda") -> torch.Tensor:
    """numpy uint16 bf16 bit patterns -> torch.bfloat16 tensor on `device`."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def to_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def words_to_tensor(a: np.ndarray, device="cuda") -> torch.Tensor:
    """numpy uint32 packed words -> torch.int32 tensor (same bits) on `device`."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint32).view(np.int32)).to(device)


# ----------------------------------------------------------------------------
# weights and layers
# ----------------------------------------------------------------------------
@dataclass
class W4Weight:
    qweight: torch.Tensor   # int32 [N, K/8] (uint32 words)
    scales: torch.Tensor    # bf16 [K/128, N]

    def __post_init__(self):
        _need(self.qweight, "qweight", torch.int32)
        _need(self.scales, "scales", torch.bfloat16)
        n, kb = self.qweight.shape
        if tuple(self.scales.shape) != (kb * 8 // 128, n):
            raise ValueError("scales must be [K/128, N]")

    @property
    def K(self):
        return self.qweight.shape[1] * 8

    @property
    def N(self):
        return self.qweight.shape[0]

    def c(self) -> CW4:
        return CW4(self.qweight.data_ptr(), self.scales.data_ptr(), self.K, self.N)

    @classmethod
    def from_numpy(cls, qweight: np.ndarray, scales: np.ndarray, device="cuda"):
        return cls(words_to_tensor(qweight, device), from_bits(scales, device))


@dataclass
class MlpLayer:
    norm_weight: torch.Tensor        # bf16 [H]
    gate_up: W4Weight                # K = H, N = 2I
    down: W4Weight                   # K = I, N = H
    out_scale: torch.Tensor | None   # fp32 0-dim (or 1-element) device tensor, or None
    eps: float = 1e-6
    residual_in_epilogue: bool = True

    @property
    def H(self):
        return self.gate_up.K

    @property
    def I(self):  # noqa: E743
        return self.down.K

    def c(self) -> CLayer:
        _need(self.norm_weight, "norm_weight", torch.bfloat16, shape=(self.H,))
        if self.out_scale is not None:
            _need(self.out_scale, "out_scale", torch.float32, numel=1)
        return CLayer(self.norm_weight.data_ptr(), float(self.eps), self.gate_up.c(), self.down.c(),
                      _ptr(self.out_scale), int(bool(self.residual_in_epilogue)))


def scalar(v: float, device="cuda") -> torch.Tensor:
    """A 0-dim fp32 device tensor (the output-scale multiplier)."""
    return torch.tensor(float(v), dtype=torch.float32, device=device)


# ----------------------------------------------------------------------------
# workspaces
# ----------------------------------------------------------------------------
GEMV_KERNELS = {0: "column", 1: "split-K", 2: "matrix-core, row blocks", 3: "matrix-core, waves split K",
                4: "matrix-core, direct-to-LDS ring"}


def gemv_kernel(M, K, N, swiglu=True) -> str:
    """The kernel the GEMV entry point launches for this shape (host-side plan)."""
    k = int(lib().fdec_test_gemv_kernel(int(M), int(K), int(N), 1 if swiglu else 0))
    if k < 0:
        raise FdecError(f"gemv shape M={M} K={K} N={N} rejected")
    return GEMV_KERNELS[k]


def gemv_workspace_bytes(M, K, N) -> int:
    """Workspace of fdec_swiglu_w4_gemv / fdec_w4_gemv.  While a test override set through
    this module (set_gemv_split, set_gemv_tiling) is active, the size under it."""
    if _overrides_active:
        return int(lib().fdec_test_gemv_workspace_bytes(M, K, N))
    return int(lib().fdec_w4_gemv_workspace_bytes(M, K, N))


def mlp_workspace_bytes(M, H, I) -> int:
    """Workspace of the three-kernel layer, chain and graph calls (override-aware as above)."""
    if _overrides_active:
        return int(lib().fdec_test_mlp_workspace_bytes(M, H, I))
    return int(lib().fdec_mlp_workspace_bytes(M, H, I))


def unfused_gemv_workspace_bytes(mode, M, K, N) -> int:
    return int(lib().fdec_unfused_gemv_workspace_bytes(mode, M, K, N))


def unfused_add_rmsnorm_workspace_bytes(M, H) -> int:
    return int(lib().fdec_unfused_add_rmsnorm_workspace_bytes(M, H))


def unfused_mlp_workspace_bytes(M, H, I) -> int:
    return int(lib().fdec_unfused_mlp_workspace_bytes(M, H, I))


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A workspace of at least 16 bytes (zero-filled; the kernels need no initial content)."""
    return torch.zeros(max(16, int(nbytes)), dtype=torch.uint8, device=device)


def workspace_init(ws: torch.Tensor):
    _check(lib().fdec_workspace_init(ws.data_ptr(), ws.numel(), _stream(ws.device)))


class _NoWorkspace:
    """Stands for 'no workspace' (a NULL pointer and 0 bytes) where a call needs none, so
    that no tensor is allocated per call (inside a graph capture an allocation records a
    fill kernel)."""

    def data_ptr(self):
        return 0

    def numel(self):
        return 0


_NO_WS = _NoWorkspace()


def _ws(ws, need, device):
    if ws is None:
        return _NO_WS if need == 0 else workspace(need, device)
    _need(ws, "ws", torch.uint8)
    if ws.numel() < need:
        raise ValueError(f"workspace has {ws.numel()} bytes, {need} required")
    return ws


# ----------------------------------------------------------------------------
# entry points
# ----------------------------------------------------------------------------
def add_rmsnorm(x, residual, weight, eps=1e-6, h_out=None, y_out=None, inplace=False):
    """(h, y) = (bf16(x + residual), bf16(h * weight / rms(h))).  inplace: h_out = residual."""
    _need(x, "x", torch.bfloat16)
    if x.dim() != 2:
        raise ValueError("x must be [M, H]")
    M, H = x.shape
    _need(residual, "residual", torch.bfloat16, shape=(M, H))
    _need(weight, "weight", torch.bfloat16, shape=(H,))
    h = residual if inplace else (torch.empty_like(x) if h_out is None else h_out)
    y = torch.empty_like(x) if y_out is None else y_out
    _need(h, "h_out", torch.bfloat16, shape=(M, H))
    _need(y, "y_out", torch.bfloat16, shape=(M, H))
    _check(lib().fdec_add_rmsnorm(x.data_ptr(), residual.data_ptr(), weight.data_ptr(), float(eps), M, H,
                                  h.data_ptr(), y.data_ptr(), _stream(x.device)))
    return h, y


def swiglu_w4_gemv(g, u, W: W4Weight, out_scale=None, residual=None, out=None, ws=None):
    """y = bf16(s * (silu(g) * u) @ dequant(W) (+ residual)); g, u are [M, K] views."""
    M = g.shape[0]
    ld = _rows(g, "g", M, W.K)
    ldu = _rows(u, "u", M, W.K)
    if M > 1 and ldu != ld:
        raise ValueError("g and u must share a row stride")
    if out_scale is not None:
        _need(out_scale, "out_scale", torch.float32, numel=1)
    if residual is not None:
        _need(residual, "residual", torch.bfloat16, shape=(M, W.N))
    y = torch.empty((M, W.N), dtype=torch.bfloat16, device=g.device) if out is None else out
    _need(y, "out", torch.bfloat16, shape=(M, W.N))
    ws = _ws(ws, gemv_workspace_bytes(M, W.K, W.N), g.device)
    cw = W.c()
    _check(lib().fdec_swiglu_w4_gemv(g.data_ptr(), u.data_ptr(), ld, ctypes.byref(cw), _ptr(out_scale),
                                     _ptr(residual), M, y.data_ptr(), ws.data_ptr(), ws.numel(),
                                     _stream(g.device)))
    return y


def swiglu_w4_gemv_noalloc(g, u, W: W4Weight, out_scale=None, residual=None, out=None):
    """swiglu_w4_gemv without a workspace: the library keeps the partial sums in its static
    per-GPU scratch (fdec_swiglu_w4_gemv_noalloc).  Allocates nothing when `out` is given;
    calls that may overlap in time on one GPU must not be issued."""
    M = g.shape[0]
    ld = _rows(g, "g", M, W.K)
    ldu = _rows(u, "u", M, W.K)
    if M > 1 and ldu != ld:
        raise ValueError("g and u must share a row stride")
    if out_scale is not None:
        _need(out_scale, "out_scale", torch.float32, numel=1)
    if residual is not None:
        _need(residual, "residual", torch.bfloat16, shape=(M, W.N))
    y = torch.empty((M, W.N), dtype=torch.bfloat16, device=g.device) if out is None else out
    _need(y, "out", torch.bfloat16, shape=(M, W.N))
    cw = W.c()
    _check(lib().fdec_swiglu_w4_gemv_noalloc(g.data_ptr(), u.data_ptr(), ld, ctypes.byref(cw), _ptr(out_scale),
                                             _ptr(residual), M, y.data_ptr(), _stream(g.device)))
    return y


def w4_gemv(x, W: W4Weight, out_scale=None, out=None, ws=None):
    """y = bf16(s * x @ dequant(W)) (the identity-prologue GEMV, e.g. gate_up)."""
    _need(x, "x", torch.bfloat16)
    M = x.shape[0]
    _need(x, "x", torch.bfloat16, shape=(M, W.K))
    if out_scale is not None:
        _need(out_scale, "out_scale", torch.float32, numel=1)
    y = torch.empty((M, W.N), dtype=torch.bfloat16, device=x.device) if out is None else out
    _need(y, "out", torch.bfloat16, shape=(M, W.N))
    ws = _ws(ws, gemv_workspace_bytes(M, W.K, W.N), x.device)
    cw = W.c()
    _check(lib().fdec_w4_gemv(x.data_ptr(), ctypes.byref(cw), _ptr(out_scale), M, y.data_ptr(), ws.data_ptr(),
                              ws.numel(), _stream(x.device)))
    return y


@dataclass
class MlpBuffers:
    """Caller-owned activation buffers of one layer (or a chain) at batch M."""
    x: torch.Tensor          # [M, H]  layer input; with out=x, the layer output
    residual: torch.Tensor   # [M, H]
    y_norm: torch.Tensor     # [M, H]
    gate_up: torch.Tensor    # [M, 2I]
    out: torch.Tensor        # [M, H]

    @classmethod
    def empty(cls, M, H, I, device="cuda", out_is_x=False):
        x = torch.empty((M, H), dtype=torch.bfloat16, device=device)
        return cls(x, torch.empty_like(x), torch.empty_like(x),
                   torch.empty((M, 2 * I), dtype=torch.bfloat16, device=device),
                   x if out_is_x else torch.empty_like(x))


def _check_bufs(layer: MlpLayer, b: MlpBuffers):
    M = b.x.shape[0]
    for name, t, shp in (("x", b.x, (M, layer.H)), ("residual", b.residual, (M, layer.H)),
                         ("y_norm", b.y_norm, (M, layer.H)), ("gate_up", b.gate_up, (M, 2 * layer.I)),
                         ("out", b.out, (M, layer.H))):
        _need(t, name, torch.bfloat16, shape=shp)
    return M


def mlp_decode(layer: MlpLayer, bufs: MlpBuffers, ws=None):
    """One layer: residual <- h; y_norm; gate_up; out (see fdec.h)."""
    M = _check_bufs(layer, bufs)
    ws = _ws(ws, mlp_workspace_bytes(M, layer.H, layer.I), bufs.x.device)
    cl = layer.c()
    _check(lib().fdec_mlp_decode(ctypes.byref(cl), M, bufs.x.data_ptr(), bufs.residual.data_ptr(),
                                 bufs.y_norm.data_ptr(), bufs.gate_up.data_ptr(), bufs.out.data_ptr(),
                                 ws.data_ptr(), ws.numel(), _stream(bufs.x.device)))
    return bufs


def _layer_array(layers):
    arr = (CLayer * len(layers))()
    for i, L in enumerate(layers):
        arr[i] = L.c()
    return arr


def mlp_chain(layers, bufs: MlpBuffers, ws=None):
    """All layers eagerly, x updated in place (out = x), residual <- the last h."""
    M = _check_bufs(layers[0], bufs)
    ws = _ws(ws, mlp_workspace_bytes(M, layers[0].H, layers[0].I), bufs.x.device)
    arr = _layer_array(layers)
    _check(lib().fdec_mlp_chain(arr, len(layers), M, bufs.x.data_ptr(), bufs.residual.data_ptr(),
                                bufs.y_norm.data_ptr(), bufs.gate_up.data_ptr(), ws.data_ptr(), ws.numel(),
                                _stream(bufs.x.device)))
    return bufs


class MlpGraph:
    """The layer chain captured once into a hipGraph; launch() replays it."""

    def __init__(self, layers, bufs: MlpBuffers, ws=None, stream: torch.cuda.Stream | None = None):
        M = _check_bufs(layers[0], bufs)
        self.layers = list(layers)          # keep the tensors alive
        self.bufs = bufs
        self.ws = _ws(ws, mlp_workspace_bytes(M, layers[0].H, layers[0].I), bufs.x.device)
        self._handle = _c_p()
        cap = stream if stream is not None else torch.cuda.Stream(device=bufs.x.device)
        cap.wait_stream(torch.cuda.current_stream(bufs.x.device))
        arr = _layer_array(self.layers)
        _check(lib().fdec_mlp_graph_create(arr, len(self.layers), M, bufs.x.data_ptr(), bufs.residual.data_ptr(),
                                           bufs.y_norm.data_ptr(), bufs.gate_up.data_ptr(), self.ws.data_ptr(),
                                           self.ws.numel(), cap.cuda_stream, ctypes.byref(self._handle)))

    def update(self, layers, bufs: MlpBuffers, ws=None, stream: torch.cuda.Stream | None = None):
        """Point the graph at other layers and buffers of the same shapes, without a new
        instantiation (fdec_mlp_graph_update).  Waits for pending work on the device first."""
        M = _check_bufs(layers[0], bufs)
        ws = _ws(ws, mlp_workspace_bytes(M, layers[0].H, layers[0].I), bufs.x.device)
        torch.cuda.synchronize(bufs.x.device)
        cap = stream if stream is not None else torch.cuda.Stream(device=bufs.x.device)
        layers = list(layers)
        arr = _layer_array(layers)
        _check(lib().fdec_mlp_graph_update(self._handle, arr, len(layers), M, bufs.x.data_ptr(),
                                           bufs.residual.data_ptr(), bufs.y_norm.data_ptr(), bufs.gate_up.data_ptr(),
                                           ws.data_ptr(), ws.numel(), cap.cuda_stream))
        self.layers, self.bufs, self.ws = layers, bufs, ws

    @property
    def kernel_count(self) -> int:
        return int(lib().fdec_graph_kernel_count(self._handle))

    def launch(self, stream: torch.cuda.Stream | None = None):
        s = stream.cuda_stream if stream is not None else _stream(self.bufs.x.device)
        _check(lib().fdec_graph_launch(self._handle, s))

    def close(self):
        if self._handle:
            _check(lib().fdec_graph_destroy(self._handle))
            self._handle = _c_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ---------------------------------------------------------------------------
# the two-kernel layer: add + RMSNorm as the gate_up prologue, SwiGLU as its epilogue
# ---------------------------------------------------------------------------
def add_rmsnorm_w4_gemv_swiglu(x, residual, weight, W_gu: W4Weight, eps=1e-6, h_out=None, act_out=None):
    """(h, act): h = bf16(x + residual); act = bf16(silu(g) * u) with [g, u] = rmsnorm(h) @ W_gu."""
    M, H = x.shape
    I = W_gu.N // 2
    _need(x, "x", torch.bfloat16, shape=(M, H))
    _need(residual, "residual", torch.bfloat16, shape=(M, H))
    _need(weight, "weight", torch.bfloat16, shape=(H,))
    h = h_out if h_out is not None else torch.empty_like(x)
    act = act_out if act_out is not None else torch.empty((M, I), dtype=torch.bfloat16, device=x.device)
    _need(h, "h_out", torch.bfloat16, shape=(M, H))
    _need(act, "act_out", torch.bfloat16, shape=(M, I))
    cw = W_gu.c()
    _check(lib().fdec_add_rmsnorm_w4_gemv_swiglu(x.data_ptr(), residual.data_ptr(), weight.data_ptr(), float(eps),
                                                 ctypes.byref(cw), M, h.data_ptr(), act.data_ptr(),
                                                 _stream(x.device)))
    return h, act


def w4_gemv_swiglu_workspace_bytes(M, K, I) -> int:
    return int(lib().fdec_w4_gemv_swiglu_workspace_bytes(M, K, I))


def w4_gemv_swiglu(x, gate_up: W4Weight, out=None, ws=None):
    """act = bf16(silu(x @ W[:, :I]) * (x @ W[:, I:])): the gate_up projection with SwiGLU as
    its epilogue (the matrix-core kernel, 1..64 rows); x [M, K], W [K, 2I]."""
    _need(x, "x", torch.bfloat16)
    if x.dim() != 2 or x.shape[1] != gate_up.K:
        raise ValueError("x must be [M, K]")
    M, I = x.shape[0], gate_up.N // 2
    act = torch.empty((M, I), dtype=torch.bfloat16, device=x.device) if out is None else out
    _need(act, "out", torch.bfloat16, shape=(M, I))
    ws = _ws(ws, w4_gemv_swiglu_workspace_bytes(M, gate_up.K, I), x.device)
    cw = gate_up.c()
    _check(lib().fdec_w4_gemv_swiglu(x.data_ptr(), ctypes.byref(cw), M, act.data_ptr(), ws.data_ptr(), ws.numel(),
                                     _stream(x.device)))
    return act


# ----------------------------------------------------------------------------
# prefill sizes
# ----------------------------------------------------------------------------
def swiglu(g, u, out=None):
    """act = bf16(silu(g) * u), one rounding; g, u are [M, K] views with one row stride."""
    M, K = g.shape
    ld = _rows(g, "g", M, K)
    if M > 1 and _rows(u, "u", M, K) != ld:
        raise ValueError("g and u must share a row stride")
    act = torch.empty((M, K), dtype=torch.bfloat16, device=g.device) if out is None else out
    _need(act, "out", torch.bfloat16, shape=(M, K))
    _check(lib().fdec_swiglu(g.data_ptr(), u.data_ptr(), ld, M, K, act.data_ptr(), _stream(g.device)))
    return act


def w4_gemm(x, W: W4Weight, out_scale=None, residual=None, out=None):
    """y = bf16(s * x @ dequant(W) (+ residual)) for any number of rows (matrix-core GEMM)."""
    _need(x, "x", torch.bfloat16)
    if x.dim() != 2 or x.shape[1] != W.K:
        raise ValueError("x must be [M, K]")
    M = x.shape[0]
    if out_scale is not None:
        _need(out_scale, "out_scale", torch.float32, numel=1)
    if residual is not None:
        _need(residual, "residual", torch.bfloat16, shape=(M, W.N))
    y = torch.empty((M, W.N), dtype=torch.bfloat16, device=x.device) if out is None else out
    _need(y, "out", torch.bfloat16, shape=(M, W.N))
    cw = W.c()
    _check(lib().fdec_w4_gemm(x.data_ptr(), ctypes.byref(cw), _ptr(out_scale), _ptr(residual), M, y.data_ptr(),
                              _stream(x.device)))
    return y


def swiglu_w4_gemm_workspace_bytes(M, K) -> int:
    return int(lib().fdec_swiglu_w4_gemm_workspace_bytes(M, K))


def swiglu_w4_gemm(g, u, W: W4Weight, out_scale=None, residual=None, out=None, ws=None):
    """y = bf16(s * bf16(silu(g) * u) @ dequant(W) (+ residual)): the prefill-size path
    (the SwiGLU pass into the workspace, then the GEMM)."""
    M = g.shape[0]
    ld = _rows(g, "g", M, W.K)
    if M > 1 and _rows(u, "u", M, W.K) != ld:
        raise ValueError("g and u must share a row stride")
    if out_scale is not None:
        _need(out_scale, "out_scale", torch.float32, numel=1)
    if residual is not None:
        _need(residual, "residual", torch.bfloat16, shape=(M, W.N))
    y = torch.empty((M, W.N), dtype=torch.bfloat16, device=g.device) if out is None else out
    _need(y, "out", torch.bfloat16, shape=(M, W.N))
    ws = _ws(ws, swiglu_w4_gemm_workspace_bytes(M, W.K), g.device)
    cw = W.c()
    _check(lib().fdec_swiglu_w4_gemm(g.data_ptr(), u.data_ptr(), ld, ctypes.byref(cw), _ptr(out_scale),
                                     _ptr(residual), M, y.data_ptr(), ws.data_ptr(), ws.numel(), _stream(g.device)))
    return y


def mlp2_workspace_bytes(M, H, I) -> int:
    return int(lib().fdec_mlp2_workspace_bytes(M, H, I))


@dataclass
class Mlp2Buffers:
    """Caller-owned activation buffers of the two-kernel layer (or chain) at batch M."""
    x: torch.Tensor          # [M, H]  layer input; with out=x, the layer output
    residual: torch.Tensor   # [M, H]
    act: torch.Tensor        # [M, I]  silu(gate) * up, written by the first kernel
    out: torch.Tensor        # [M, H]

    @classmethod
    def empty(cls, M, H, I, device="cuda", out_is_x=False):
        x = torch.empty((M, H), dtype=torch.bfloat16, device=device)
        return cls(x, torch.empty_like(x), torch.empty((M, I), dtype=torch.bfloat16, device=device),
                   x if out_is_x else torch.empty_like(x))


def _check_bufs2(layer: MlpLayer, b: Mlp2Buffers):
    M = b.x.shape[0]
    for name, t, shp in (("x", b.x, (M, layer.H)), ("residual", b.residual, (M, layer.H)),
                         ("act", b.act, (M, layer.I)), ("out", b.out, (M, layer.H))):
        _need(t, name, torch.bfloat16, shape=shp)
    return M


def mlp_decode2(layer: MlpLayer, bufs: Mlp2Buffers, ws=None):
    """One two-kernel layer: residual <- h; act; out (see fdec.h)."""
    M = _check_bufs2(layer, bufs)
    ws = _ws(ws, mlp2_workspace_bytes(M, layer.H, layer.I), bufs.x.device)
    cl = layer.c()
    _check(lib().fdec_mlp_decode2(ctypes.byref(cl), M, bufs.x.data_ptr(), bufs.residual.data_ptr(),
                                  bufs.act.data_ptr(), bufs.out.data_ptr(), ws.data_ptr(), ws.numel(),
                                  _stream(bufs.x.device)))
    return bufs


def mlp_chain2(layers, bufs: Mlp2Buffers, ws=None):
    """All layers eagerly, two kernels each, x updated in place, residual <- the last h."""
    M = _check_bufs2(layers[0], bufs)
    ws = _ws(ws, mlp2_workspace_bytes(M, layers[0].H, layers[0].I), bufs.x.device)
    arr = _layer_array(layers)
    _check(lib().fdec_mlp_chain2(arr, len(layers), M, bufs.x.data_ptr(), bufs.residual.data_ptr(),
                                 bufs.act.data_ptr(), ws.data_ptr(), ws.numel(), _stream(bufs.x.device)))
    return bufs


class Mlp2Graph(MlpGraph):
    """The two-kernel layer chain captured once into a hipGraph; launch() replays it."""

    def __init__(self, layers, bufs: Mlp2Buffers, ws=None, stream: torch.cuda.Stream | None = None):
        M = _check_bufs2(layers[0], bufs)
        self.layers = list(layers)
        self.bufs = bufs
        self.ws = _ws(ws, mlp2_workspace_bytes(M, layers[0].H, layers[0].I), bufs.x.device)
        self._handle = _c_p()
        cap = stream if stream is not None else torch.cuda.Stream(device=bufs.x.device)
        cap.wait_stream(torch.cuda.current_stream(bufs.x.device))
        arr = _layer_array(self.layers)
        _check(lib().fdec_mlp_graph_create2(arr, len(self.layers), M, bufs.x.data_ptr(), bufs.residual.data_ptr(),
                                            bufs.act.data_ptr(), self.ws.data_ptr(), self.ws.numel(),
                                            cap.cuda_stream, ctypes.byref(self._handle)))

    def update(self, layers, bufs: Mlp2Buffers, ws=None, stream: torch.cuda.Stream | None = None):
        """Point the graph at other layers and buffers of the same shapes, without a new
        instantiation (fdec_mlp_graph_update2).  Waits for pending work on the device first."""
        M = _check_bufs2(layers[0], bufs)
        ws = _ws(ws, mlp2_workspace_bytes(M, layers[0].H, layers[0].I), bufs.x.device)
        torch.cuda.synchronize(bufs.x.device)
        cap = stream if stream is not None else torch.cuda.Stream(device=bufs.x.device)
        layers = list(layers)
        arr = _layer_array(layers)
        _check(lib().fdec_mlp_graph_update2(self._handle, arr, len(layers), M, bufs.x.data_ptr(),
                                            bufs.residual.data_ptr(), bufs.act.data_ptr(), ws.data_ptr(), ws.numel(),
                                            cap.cuda_stream))
        self.layers, self.bufs, self.ws = layers, bufs, ws


def unfused_swiglu_w4_gemv(mode, g, u, W: W4Weight, out_scale=None, residual=None, out=None, ws=None):
    M = g.shape[0]
    ld = _rows(g, "g", M, W.K)
    _rows(u, "u", M, W.K)
    if out_scale is not None:
        _need(out_scale, "out_scale", torch.float32, numel=1)
    if residual is not None:
        _need(residual, "residual", torch.bfloat16, shape=(M, W.N))
    y = torch.empty((M, W.N), dtype=torch.bfloat16, device=g.device) if out is None else out
    _need(y, "out", torch.bfloat16, shape=(M, W.N))
    need = unfused_gemv_workspace_bytes(mode, M, W.K, W.N)
    ws = _ws(ws, need, g.device)
    cw = W.c()
    _check(lib().fdec_unfused_swiglu_w4_gemv(mode, g.data_ptr(), u.data_ptr(), ld, ctypes.byref(cw),
                                             _ptr(out_scale), _ptr(residual), M, y.data_ptr(), ws.data_ptr(),
                                             ws.numel(), _stream(g.device)))
    return y


def unfused_add_rmsnorm(x, residual, weight, eps=1e-6, h_out=None, y_out=None, ws=None):
    _need(x, "x", torch.bfloat16)
    M, H = x.shape
    _need(residual, "residual", torch.bfloat16, shape=(M, H))
    _need(weight, "weight", torch.bfloat16, shape=(H,))
    h = torch.empty_like(x) if h_out is None else h_out
    y = torch.empty_like(x) if y_out is None else y_out
    ws = _ws(ws, unfused_add_rmsnorm_workspace_bytes(M, H), x.device)
    _check(lib().fdec_unfused_add_rmsnorm(x.data_ptr(), residual.data_ptr(), weight.data_ptr(), float(eps), M, H,
                                          h.data_ptr(), y.data_ptr(), ws.data_ptr(), ws.numel(), _stream(x.device)))
    return h, y


def unfused_mlp_decode(layer: MlpLayer, bufs: MlpBuffers, ws=None):
    M = _check_bufs(layer, bufs)
    ws = _ws(ws, unfused_mlp_workspace_bytes(M, layer.H, layer.I), bufs.x.device)
    cl = layer.c()
    _check(lib().fdec_unfused_mlp_decode(ctypes.byref(cl), M, bufs.x.data_ptr(), bufs.residual.data_ptr(),
                                         bufs.y_norm.data_ptr(), bufs.gate_up.data_ptr(), bufs.out.data_ptr(),
                                         ws.data_ptr(), ws.numel(), _stream(bufs.x.device)))
    return bufs


def w4_unpack(W: W4Weight) -> torch.Tensor:
    q = torch.empty((W.K, W.N), dtype=torch.int8, device=W.qweight.device)
    cw = W.c()
    _check(lib().fdec_w4_unpack(ctypes.byref(cw), q.data_ptr(), _stream(q.device)))
    return q


def w4_dequant(W: W4Weight) -> torch.Tensor:
    w = torch.empty((W.K, W.N), dtype=torch.float32, device=W.qweight.device)
    cw = W.c()
    _check(lib().fdec_w4_dequant(ctypes.byref(cw), w.data_ptr(), _stream(w.device)))
    return w


# ---------------------------------------------------------------------------
# FP4 (E2M1) weights with E4M3 1x16 block scales
# ---------------------------------------------------------------------------
@dataclass
class FP4Weight:
    qweight: torch.Tensor   # int32 [N, K/8] (uint32 words of eight E2M1 codes)
    scales: torch.Tensor    # uint8 [N, K/16] (E4M3 codes)

    def __post_init__(self):
        _need(self.qweight, "qweight", torch.int32)
        _need(self.scales, "scales", torch.uint8)
        n, kb = self.qweight.shape
        if tuple(self.scales.shape) != (n, kb * 8 // 16):
            raise ValueError("scales must be [N, K/16]")

    @property
    def K(self):
        return self.qweight.shape[1] * 8

    @property
    def N(self):
        return self.qweight.shape[0]

    def c(self) -> CFP4:
        return CFP4(self.qweight.data_ptr(), self.scales.data_ptr(), self.K, self.N)

    @classmethod
    def from_numpy(cls, qweight: np.ndarray, scales: np.ndarray, device="cuda"):
        return cls(words_to_tensor(qweight, device),
                   torch.from_numpy(np.ascontiguousarray(scales, dtype=np.uint8)).to(device))


def fp4_gemv_workspace_bytes(M, K, N) -> int:
    return int(lib().fdec_fp4_gemv_workspace_bytes(M, K, N))


def swiglu_fp4_gemv(g, u, W: FP4Weight, out_scale=None, residual=None, out=None, ws=None):
    """y = bf16(s * (silu(g) * u) @ W (+ residual)) with FP4 weights; g, u are [M, K] views."""
    M = g.shape[0]
    ld = _rows(g, "g", M, W.K)
    ldu = _rows(u, "u", M, W.K)
    if M > 1 and ldu != ld:
        raise ValueError("g and u must share a row stride")
    if out_scale is not None:
        _need(out_scale, "out_scale", torch.float32, numel=1)
    if residual is not None:
        _need(residual, "residual", torch.bfloat16, shape=(M, W.N))
    y = torch.empty((M, W.N), dtype=torch.bfloat16, device=g.device) if out is None else out
    _need(y, "out", torch.bfloat16, shape=(M, W.N))
    ws = _ws(ws, fp4_gemv_workspace_bytes(M, W.K, W.N), g.device)
    cw = W.c()
    _check(lib().fdec_swiglu_fp4_gemv(g.data_ptr(), u.data_ptr(), ld, ctypes.byref(cw), _ptr(out_scale),
                                      _ptr(residual), M, y.data_ptr(), ws.data_ptr(), ws.numel(),
                                      _stream(g.device)))
    return y


def fp4_gemv(x, W: FP4Weight, out_scale=None, residual=None, out=None, ws=None):
    """y = bf16(s * x @ W (+ residual)) with FP4 weights (identity prologue)."""
    _need(x, "x", torch.bfloat16)
    M = x.shape[0]
    _need(x, "x", torch.bfloat16, shape=(M, W.K))
    if out_scale is not None:
        _need(out_scale, "out_scale", torch.float32, numel=1)
    if residual is not None:
        _need(residual, "residual", torch.bfloat16, shape=(M, W.N))
    y = torch.empty((M, W.N), dtype=torch.bfloat16, device=x.device) if out is None else out
    _need(y, "out", torch.bfloat16, shape=(M, W.N))
    ws = _ws(ws, fp4_gemv_workspace_bytes(M, W.K, W.N), x.device)
    cw = W.c()
    _check(lib().fdec_fp4_gemv(x.data_ptr(), ctypes.byref(cw), _ptr(out_scale), _ptr(residual), M, y.data_ptr(),
                               ws.data_ptr(), ws.numel(), _stream(x.device)))
    return y


def swiglu_fp4a4_gemv(g, u, W: FP4Weight, act_scale, out_scale=None, residual=None, out=None, ws=None):
    """Both operands FP4: act = silu(g) * u quantised with its per-tensor scale act_scale
    (device fp32 scalar; E4M3 block scales of 16), times the FP4 weights:
    y = bf16(s * sum_k q s_b w (+ residual))."""
    M = g.shape[0]
    ld = _rows(g, "g", M, W.K)
    ldu = _rows(u, "u", M, W.K)
    if M > 1 and ldu != ld:
        raise ValueError("g and u must share a row stride")
    _need(act_scale, "act_scale", torch.float32, numel=1)
    if out_scale is not None:
        _need(out_scale, "out_scale", torch.float32, numel=1)
    if residual is not None:
        _need(residual, "residual", torch.bfloat16, shape=(M, W.N))
    y = torch.empty((M, W.N), dtype=torch.bfloat16, device=g.device) if out is None else out
    _need(y, "out", torch.bfloat16, shape=(M, W.N))
    ws = _ws(ws, fp4_gemv_workspace_bytes(M, W.K, W.N), g.device)
    cw = W.c()
    _check(lib().fdec_swiglu_fp4a4_gemv(g.data_ptr(), u.data_ptr(), ld, ctypes.byref(cw), act_scale.data_ptr(),
                                        _ptr(out_scale), _ptr(residual), M, y.data_ptr(), ws.data_ptr(), ws.numel(),
                                        _stream(g.device)))
    return y


def fp4a4_gemv(x, W: FP4Weight, act_scale, out_scale=None, residual=None, out=None, ws=None):
    """Both operands FP4 with the identity prologue: x [M, K] bf16 quantised, then times W."""
    _need(x, "x", torch.bfloat16)
    M = x.shape[0]
    _need(x, "x", torch.bfloat16, shape=(M, W.K))
    _need(act_scale, "act_scale", torch.float32, numel=1)
    if out_scale is not None:
        _need(out_scale, "out_scale", torch.float32, numel=1)
    if residual is not None:
        _need(residual, "residual", torch.bfloat16, shape=(M, W.N))
    y = torch.empty((M, W.N), dtype=torch.bfloat16, device=x.device) if out is None else out
    _need(y, "out", torch.bfloat16, shape=(M, W.N))
    ws = _ws(ws, fp4_gemv_workspace_bytes(M, W.K, W.N), x.device)
    cw = W.c()
    _check(lib().fdec_fp4a4_gemv(x.data_ptr(), ctypes.byref(cw), act_scale.data_ptr(), _ptr(out_scale),
                                 _ptr(residual), M, y.data_ptr(), ws.data_ptr(), ws.numel(), _stream(x.device)))
    return y


def nvfp4_quantize(x, act_scale):
    """The activation quantiser alone (test hook): x [M, K] bf16 -> (codes int32 [M, K/8]
    packed words, E4M3 scale codes uint8 [M, K/16]); x may be a row-strided view."""
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise TypeError("x must be a 2-D bf16 GPU tensor")
    M, K = x.shape
    ld = _rows(x, "x", M, K)
    _need(act_scale, "act_scale", torch.float32, numel=1)
    codes = torch.empty((M, K // 8), dtype=torch.int32, device=x.device)
    scales = torch.empty((M, K // 16), dtype=torch.uint8, device=x.device)
    _check(lib().fdec_nvfp4_quantize(x.data_ptr(), ld, M, K, act_scale.data_ptr(), codes.data_ptr(),
                                     scales.data_ptr(), _stream(x.device)))
    return codes, scales


def fp4_dequant(W: FP4Weight) -> torch.Tensor:
    w = torch.empty((W.K, W.N), dtype=torch.float32, device=W.qweight.device)
    cw = W.c()
    _check(lib().fdec_fp4_dequant(ctypes.byref(cw), w.data_ptr(), _stream(w.device)))
    return w


# ----------------------------------------------------------------------------
# test, tuning and measurement controls (include/fdec_test.h; not for production use)
# ----------------------------------------------------------------------------
_overrides_active = False
_override_state = {"split": 0, "tiling": (0, 0), "mfma": (0, 0, 0), "kmfma_waves": 0}


def _note_overrides():
    global _overrides_active
    _overrides_active = (_override_state["split"] != 0 or _override_state["tiling"] != (0, 0)
                         or _override_state["mfma"] != (0, 0, 0) or _override_state["kmfma_waves"] != 0)


def set_mfma_plan(kernel: int, tiles: int = 0, groups_per_wave: int = 0):
    lib().fdec_set_mfma_plan(int(kernel), int(tiles), int(groups_per_wave))
    _override_state["mfma"] = (int(kernel), int(tiles), int(groups_per_wave))
    _note_overrides()


def set_kmfma_waves(waves: int):
    """Waves per workgroup (6..8) of the matrix-core kernel whose waves split K; 0: built in."""
    lib().fdec_set_kmfma_waves(int(waves))
    _override_state["kmfma_waves"] = int(waves) if 6 <= int(waves) <= 8 else 0
    _note_overrides()


def set_gemv_split(k: int):
    lib().fdec_set_gemv_split(int(k))
    _override_state["split"] = max(0, int(k))
    _note_overrides()


def set_gemv_tiling(waves: int, cols_per_workgroup: int):
    lib().fdec_set_gemv_tiling(int(waves), int(cols_per_workgroup))
    _override_state["tiling"] = (max(0, int(waves)), max(0, int(cols_per_workgroup)))
    _note_overrides()


def test_fail_launches(on: bool):
    lib().fdec_test_fail_launches(int(bool(on)))


def empty_kernel(wgs=256, threads=256):
    """One launch of a kernel that does nothing (the per-launch floor)."""
    _check(lib().fdec_test_empty_kernel(int(wgs), int(threads), _stream()))


def read_ceiling(stream_buf, per_wg, g, u, pieces, rows, row_bytes, piece_bytes, wgs, sink):
    """One launch of the read-only probe (fdec_test.h): workgroup b reads chunks
    [b * per_wg, (b + 1) * per_wg) of stream_buf, all of g and u, and its pieces of each of
    `rows` rows of `pieces`; writes one word per workgroup to sink (int32 [wgs])."""
    for t, name in ((stream_buf, "stream_buf"), (g, "g"), (u, "u"), (pieces, "pieces"), (sink, "sink")):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    if g.numel() * g.element_size() != u.numel() * u.element_size():
        raise ValueError("g and u must have the same size")
    if sink.numel() * sink.element_size() < 4 * wgs:
        raise ValueError("sink is too small")
    nb = lambda t: t.numel() * t.element_size()  # noqa: E731
    _check(lib().fdec_test_read_ceiling(stream_buf.data_ptr(), nb(stream_buf), int(per_wg), g.data_ptr(),
                                        u.data_ptr(), nb(g), pieces.data_ptr(), nb(pieces), int(rows),
                                        int(row_bytes), int(piece_bytes), int(wgs), sink.data_ptr(),
                                        _stream(stream_buf.device)))
