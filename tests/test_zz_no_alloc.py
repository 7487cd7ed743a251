"""GPU test of the allocation-free SwiGLU GEMV (fdec_swiglu_w4_gemv_noalloc): through the C
ABI it gives the workspace entry point's result bit for bit (the same kernels and plan),
on consecutive calls whose second input is smaller, so the static scratch keeps the
previous call's partial sums and must not leak into the result."""
import ctypes

import numpy as np
import pytest
import torch

import memory_bound_decode_add_amd as F
import oracle as O
import synth
from helpers import assert_bits_equal, assert_close, say

pytestmark = pytest.mark.gpu
WS_ERR = -5


def noalloc_call(g, u, W, scale, res, y):
    L = F.lib()
    cw = W.c()
    st = L.fdec_swiglu_w4_gemv_noalloc(g.data_ptr(), u.data_ptr(), g.stride(0), ctypes.byref(cw),
                                       scale.data_ptr() if scale is not None else None,
                                       res.data_ptr() if res is not None else None, g.shape[0], y.data_ptr(),
                                       torch.cuda.current_stream().cuda_stream)
    return st


def case(M, K, N, seed):
    inp = synth.swiglu_gemv_inputs(M, K, N, seed=seed, out_scale=0.5, with_residual=True)
    g, u, res = F.from_bits(inp.g), F.from_bits(inp.u), F.from_bits(inp.residual)
    W = F.W4Weight.from_numpy(inp.W.qweight, inp.W.scales)
    return inp, g, u, res, W


@pytest.mark.parametrize("shapes", [((64, 9216, 2560), (16, 4096, 1000)),
                                    ((16, 14336, 4096), (8, 9216, 2560)),
                                    ((5, 4096, 520), (1, 1024, 512))])
def test_noalloc_matches_the_workspace_entry_point(shapes):
    sc = F.scalar(0.5)
    for i, (M, K, N) in enumerate(shapes):
        say(f"[noalloc] call {i}: M={M} K={K} N={N}")
        inp, g, u, res, W = case(M, K, N, seed=M * 7 + i)
        want = F.to_bits(F.swiglu_w4_gemv(g, u, W, sc, res, ws=F.workspace(F.gemv_workspace_bytes(M, K, N))))
        y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        assert noalloc_call(g, u, W, sc, res, y) == 0, F.lib().fdec_last_error()
        torch.cuda.synchronize()
        got = F.to_bits(y)
        assert_bits_equal(got, want, f"noalloc vs workspace entry, call {i}")
        ref = O.swiglu_w4_gemv(inp.g, inp.u, inp.W.qweight, inp.W.scales, 0.5, inp.residual)
        assert_close(got, ref, f"noalloc vs oracle, call {i}")
        # the binding's wrapper, into a preallocated output
        y2 = torch.empty_like(y)
        F.swiglu_w4_gemv_noalloc(g, u, W, sc, res, out=y2)
        torch.cuda.synchronize()
        assert_bits_equal(F.to_bits(y2), want, f"binding, call {i}")


def test_noalloc_refuses_a_plan_beyond_the_scratch():
    # 64 rows at K = N = 16384 need about 60 MB of partial sums: refused before any launch
    M, K, N = 64, 16384, 16384
    g = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    W = F.W4Weight(torch.zeros((N, K // 8), dtype=torch.int32, device="cuda"),
                   torch.zeros((K // 128, N), dtype=torch.bfloat16, device="cuda"))
    assert F.gemv_workspace_bytes(M, K, N) > 32 << 20
    y = torch.full((M, N), 7.0, dtype=torch.bfloat16, device="cuda")
    assert noalloc_call(g, g, W, None, None, y) == WS_ERR
    torch.cuda.synchronize()
    assert bool(torch.all(y == 7.0))
