"""GPU parity of the fused residual add + RMSNorm against the fp64 oracle."""
import numpy as np
import pytest
import torch

import memory_bound_decode_add_amd as F
import oracle as O
import synth
from helpers import assert_bits_equal, assert_close, say

pytestmark = pytest.mark.gpu


def run(inp, inplace=False):
    x, r, w = F.from_bits(inp.x), F.from_bits(inp.r), F.from_bits(inp.w)
    h, y = F.add_rmsnorm(x, r, w, inp.eps, inplace=inplace)
    torch.cuda.synchronize()
    return F.to_bits(h), F.to_bits(y)


def test_add_rmsnorm_full_8192x4096():
    say("[norm] M=8192 H=4096 seed 0")
    inp = synth.make("add_rmsnorm_8192x4096")
    h, y = run(inp)
    rh, ry = O.add_rmsnorm(inp.x, inp.r, inp.w, inp.eps)
    assert_bits_equal(h, rh, "h")
    say("  worst y err/bound", assert_close(y, ry, "y"))
    # the pages observed y within one bf16 step of the reference
    d = np.abs(O.bf16_to_f64(y) - O.bf16_to_f64(ry))
    assert np.all(d <= np.abs(O.bf16_to_f64(ry)) * 2.0**-7 + 1e-30)
    h2, y2 = run(inp)
    assert_bits_equal(y, y2, "repeat")


@pytest.mark.parametrize("M,H", [(1, 1536), (16, 4096), (5, 1000), (3, 8), (2, 16384), (7, 520), (1, 4104)])
def test_add_rmsnorm_shapes(M, H):
    say(f"[norm] M={M} H={H}")
    inp = synth.add_rmsnorm_inputs(M, H, seed=M + H)
    h, y = run(inp)
    rh, ry = O.add_rmsnorm(inp.x, inp.r, inp.w, inp.eps)
    assert_bits_equal(h, rh, "h")
    assert_close(y, ry, "y")


@pytest.mark.parametrize("M", [1, 3, 64, 65])
@pytest.mark.parametrize("H", [8, 512, 1032, 1536, 2048, 3072, 3592, 4096])
def test_add_rmsnorm_decode_batches(M, H):
    """Up to 64 rows use one chunk per lane with the row over 1..8 waves; 65 rows the
    general shapes: every row width class on both sides of the switch."""
    inp = synth.add_rmsnorm_inputs(M, H, seed=7 * M + H)
    h, y = run(inp)
    rh, ry = O.add_rmsnorm(inp.x, inp.r, inp.w, inp.eps)
    assert_bits_equal(h, rh, f"h M={M} H={H}")
    assert_close(y, ry, f"y M={M} H={H}")


def test_add_rmsnorm_in_place_residual():
    say("[norm] in place")
    inp = synth.add_rmsnorm_inputs(33, 2048, seed=4)
    x, r, w = F.from_bits(inp.x), F.from_bits(inp.r), F.from_bits(inp.w)
    h, y = F.add_rmsnorm(x, r, w, inp.eps, inplace=True)
    assert h.data_ptr() == r.data_ptr()
    rh, ry = O.add_rmsnorm(inp.x, inp.r, inp.w, inp.eps)
    assert_bits_equal(F.to_bits(r), rh, "h in place")
    assert_close(F.to_bits(y), ry, "y")


def test_add_rmsnorm_empty_batch():
    say("[norm] M=0")
    x = torch.empty((0, 512), dtype=torch.bfloat16, device="cuda")
    h, y = F.add_rmsnorm(x, x.clone(), torch.ones(512, dtype=torch.bfloat16, device="cuda"))
    torch.cuda.synchronize()
    assert h.shape == (0, 512) and y.shape == (0, 512)


def test_add_rmsnorm_unit_weight_unit_rms():
    say("[norm] unit RMS")
    inp = synth.add_rmsnorm_inputs(64, 4096, seed=9)
    inp.w = synth.f32_to_bf16_bits(np.ones(4096, dtype=np.float32))
    _, y = run(inp)
    yf = O.bf16_to_f64(y)
    assert np.max(np.abs(np.sqrt(np.mean(yf * yf, axis=1)) - 1.0)) < 2.0**-8
