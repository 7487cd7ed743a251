"""Shared test helpers: tolerance checks and host <-> device marshalling."""
import sys

import numpy as np

import oracle as O

# |gpu - ref| <= REL * |ref| + ABS * max|ref|, elementwise, ref = the oracle's bf16 output
REL = 2e-2
ABS = 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def tol_report(gpu_bits, ref_bits):
    g = O.bf16_to_f64(gpu_bits)
    r = O.bf16_to_f64(ref_bits)
    bound = REL * np.abs(r) + ABS * np.max(np.abs(r))
    err = np.abs(g - r)
    worst = float(np.max(err / np.maximum(bound, 1e-300))) if err.size else 0.0
    return bool(np.all(err <= bound)), worst


def assert_close(gpu_bits, ref_bits, what=""):
    assert gpu_bits.shape == ref_bits.shape, (what, gpu_bits.shape, ref_bits.shape)
    ok, worst = tol_report(gpu_bits, ref_bits)
    assert np.all(np.isfinite(O.bf16_to_f64(gpu_bits))), f"{what}: non-finite output"
    assert ok, f"{what}: worst error / bound = {worst:.3f}"
    return worst


def assert_bits_equal(a, b, what=""):
    assert a.shape == b.shape, (what, a.shape, b.shape)
    bad = np.flatnonzero(a.ravel() != b.ravel())
    assert bad.size == 0, f"{what}: {bad.size} elements differ, first at {bad[:5]}"
