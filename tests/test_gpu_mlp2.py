"""GPU parity of the decode-MLP layer with SwiGLU as the gate_up GEMV's epilogue: up to 4
rows two kernels (add + RMSNorm as the gate_up GEMV's prologue, then the down GEMV), from
5 rows three (the norm, the matrix-core gate_up with the SwiGLU epilogue, the down GEMV);
its chain and its hipGraph, against the fp64 oracle."""
import numpy as np
import pytest
import torch

import memory_bound_decode_add_amd as F
import oracle as O
import synth
from helpers import assert_bits_equal, assert_close, say
from test_gpu_mlp import dev_layers

pytestmark = pytest.mark.gpu


def check_layer2(L, x, r, got, resid):
    """Each of the two kernels against the oracle fed the bf16 inputs that kernel read."""
    h, act = O.add_rmsnorm_gemv_swiglu(x, r, L.norm_w, L.gate_up.qweight, L.gate_up.scales, L.eps)
    assert_bits_equal(got["h"], h, "h")
    w = [assert_close(got["act"], act, "act")]
    out = O.w4_gemv(got["act"], L.down.qweight, L.down.scales, L.out_scale, return_f64=True)[1]
    if resid:
        out = out + O.bf16_to_f64(got["h"])
    w.append(assert_close(got["out"], O.f64_to_bf16(out), "out"))
    return w


@pytest.mark.parametrize("M,H,I", [(1, 1536, 8960), (1, 128, 8), (2, 1024, 2048), (3, 640, 392),
                                   (4, 1024, 1000), (1, 4096, 14336), (2, 256, 20480)])
def test_add_rmsnorm_gemv_swiglu(M, H, I):
    say(f"[norm+gate_up+swiglu] M={M} H={H} I={I}")
    nin = synth.add_rmsnorm_inputs(M, H, seed=3 * M + H + I)
    Wn = synth.w4_weight(np.random.default_rng(M + H + 7 * I), H, 2 * I)
    Wg = F.W4Weight.from_numpy(Wn.qweight, Wn.scales)
    x, r, nw = F.from_bits(nin.x), F.from_bits(nin.r), F.from_bits(nin.w)
    h, act = F.add_rmsnorm_w4_gemv_swiglu(x, r, nw, Wg, nin.eps)
    torch.cuda.synchronize()
    h_ref, act_ref = O.add_rmsnorm_gemv_swiglu(nin.x, nin.r, nin.w, Wn.qweight, Wn.scales, nin.eps)
    assert_bits_equal(F.to_bits(h), h_ref, "h")
    say("  worst err/bound", assert_close(F.to_bits(act), act_ref, "act"))
    # same inputs, same bits
    h2, act2 = F.add_rmsnorm_w4_gemv_swiglu(x, r, nw, Wg, nin.eps)
    torch.cuda.synchronize()
    assert_bits_equal(F.to_bits(act2), F.to_bits(act), "repeat")


def test_add_rmsnorm_gemv_swiglu_exact_gate_up():
    # eps = 0 and rows of constant magnitude with unit norm weight make y = +-1 exactly;
    # with power-of-two scales every gate/up sum is then exact in fp32, so the only
    # rounding on either side is act's single bf16 rounding of silu(g) * u, which the
    # fp32 silu and the fp64 one agree on except within a few ulps of a rounding tie.
    M, H, I = 2, 1024, 512
    rng = np.random.default_rng(5)
    sign = rng.choice([-1.0, 1.0], size=(M, H))
    x = synth.f32_to_bf16_bits(0.75 * sign)
    r = synth.f32_to_bf16_bits(0.25 * sign)
    nw = synth.f32_to_bf16_bits(np.ones(H))
    q = rng.integers(-8, 8, size=(H, 2 * I))
    s = synth.f32_to_bf16_bits(np.full((H // 128, 2 * I), 2.0**-6))
    qw = synth.pack_int4(q)
    W = F.W4Weight.from_numpy(qw, s)
    h, act = F.add_rmsnorm_w4_gemv_swiglu(F.from_bits(x), F.from_bits(r), F.from_bits(nw), W, 0.0)
    torch.cuda.synchronize()
    h_ref, act_ref = O.add_rmsnorm_gemv_swiglu(x, r, nw, qw, s, 0.0)
    assert_bits_equal(F.to_bits(h), h_ref, "h")
    got, ref = O.bf16_to_f64(F.to_bits(act)), O.bf16_to_f64(act_ref)
    mism = got != ref
    assert mism.mean() < 0.01
    assert np.all(np.abs(got - ref)[mism] <= np.abs(ref[mism]) * 2.0**-7)


def test_add_rmsnorm_gemv_swiglu_rejects_what_it_cannot_do():
    inp = synth.mlp_inputs(1, 256, 128, n_layers=1, seed=9)
    L = inp.layers[0]
    Wg = F.W4Weight.from_numpy(L.gate_up.qweight, L.gate_up.scales)
    x, r, nw = F.from_bits(inp.x), F.from_bits(inp.r), F.from_bits(L.norm_w)
    with pytest.raises(F.FdecError) as e:
        F.add_rmsnorm_w4_gemv_swiglu(x, r, nw, Wg, L.eps, h_out=x)
    assert e.value.status == -4
    x16 = torch.zeros((16, 256), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(F.FdecError) as e:
        F.add_rmsnorm_w4_gemv_swiglu(x16, x16.clone(), nw, Wg, L.eps)
    assert e.value.status == -6


@pytest.mark.parametrize("M,H,I", [(1, 1536, 8960), (2, 1024, 2048), (3, 384, 640)])
def test_mlp_decode2_both_residual_modes(M, H, I):
    say(f"[mlp2] M={M} H={H} I={I}")
    inp = synth.mlp_inputs(M, H, I, n_layers=1, seed=M + H + I + 1)
    for resid in (True, False):
        layer = dev_layers(inp, resid)[0]
        b = F.Mlp2Buffers.empty(M, H, I)
        b.x.copy_(F.from_bits(inp.x))
        b.residual.copy_(F.from_bits(inp.r))
        F.mlp_decode2(layer, b)
        torch.cuda.synchronize()
        got = {"h": F.to_bits(b.residual), "act": F.to_bits(b.act), "out": F.to_bits(b.out)}
        say(f"  resid={resid} worst err/bound (act, out)", check_layer2(inp.layers[0], inp.x, inp.r, got, resid))


def test_chain2_qwen2_5_1_5b_28_layers_graph():
    say("[chain2] M=1 H=1536 I=8960, 28 two-kernel layers: parity of every layer, graph == eager")
    inp = synth.make("mlp_qwen2_5_1_5b_28l")
    M, H, I = 1, 1536, 8960
    layers = dev_layers(inp, False)
    b = F.Mlp2Buffers.empty(M, H, I, out_is_x=True)
    ws = F.workspace(F.mlp2_workspace_bytes(M, H, I))
    b.x.copy_(F.from_bits(inp.x))
    b.residual.copy_(F.from_bits(inp.r))
    trace = []
    for L in layers:
        xin, rin = F.to_bits(b.x), F.to_bits(b.residual)
        F.mlp_decode2(L, b, ws)
        torch.cuda.synchronize()
        trace.append({"x": xin, "r": rin, "h": F.to_bits(b.residual), "act": F.to_bits(b.act),
                      "out": F.to_bits(b.x)})
    for l in range(28):
        say(f"  layer {l}")
        t = trace[l]
        check_layer2(inp.layers[l], t["x"], t["r"], t, False)

    b.x.copy_(F.from_bits(inp.x))
    b.residual.copy_(F.from_bits(inp.r))
    F.mlp_chain2(layers, b, ws)
    torch.cuda.synchronize()
    assert_bits_equal(F.to_bits(b.x), trace[-1]["out"], "chain x")
    assert_bits_equal(F.to_bits(b.residual), trace[-1]["h"], "chain r")

    graph = F.Mlp2Graph(layers, b, ws)
    assert graph.kernel_count == 2 * 28
    for rep in range(3):
        b.x.copy_(F.from_bits(inp.x))
        b.residual.copy_(F.from_bits(inp.r))
        graph.launch()
        torch.cuda.synchronize()
        assert_bits_equal(F.to_bits(b.x), trace[-1]["out"], f"graph replay {rep} x")
        assert_bits_equal(F.to_bits(b.residual), trace[-1]["h"], f"graph replay {rep} r")
        torch.randn(1 << 20, device="cuda").sum().item()
    graph.close()
    # (Per-layer parity is checked on the inputs each layer actually read.  An oracle
    # chaining its own 28 layers would also measure how single-ulp differences in the
    # materialised bf16 tensors grow through the chain, which the per-call bound does
    # not cover.)


# ----------------------------------------------------------------------------
# the gate_up projection with the SwiGLU epilogue on the matrix cores, and the layer
# built on it from 5 rows
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("M,K,I", [(16, 4096, 14336), (5, 1024, 520), (1, 1536, 8960), (8, 9216, 1032),
                                   (16, 14336, 2048), (32, 2048, 776), (64, 4096, 1024), (3, 128, 8)])
def test_w4_gemv_swiglu(M, K, I):
    need = F.w4_gemv_swiglu_workspace_bytes(M, K, I)
    say(f"[gate_up+swiglu] M={M} K={K} I={I} workspace {need} B")
    inp = synth.swiglu_gemv_inputs(M, K, 2 * I, seed=M * 31 + K + I)
    W = F.W4Weight.from_numpy(inp.W.qweight, inp.W.scales)
    x = F.from_bits(inp.g)
    ws = torch.full((max(16, need),), 0xFF, dtype=torch.uint8, device="cuda")   # NaN patterns
    act = F.to_bits(F.w4_gemv_swiglu(x, W, ws=ws))
    ref = O.w4_gemv_swiglu(inp.g, inp.W.qweight, inp.W.scales)
    say("  worst err/bound", assert_close(act, ref, "act"))
    assert_bits_equal(F.to_bits(F.w4_gemv_swiglu(x, W, ws=ws)), act, "repeat")


def check_layer2_mc(L, x, r, got, resid):
    """The three kernels of the matrix-core form, each against the oracle fed the bf16
    inputs that kernel read (y is read back from the workspace)."""
    h, y = O.add_rmsnorm(x, r, L.norm_w, L.eps)
    assert_bits_equal(got["h"], h, "h")
    w = [assert_close(got["y"], y, "y")]
    act = O.w4_gemv_swiglu(got["y"], L.gate_up.qweight, L.gate_up.scales)
    w.append(assert_close(got["act"], act, "act"))
    out = O.w4_gemv(got["act"], L.down.qweight, L.down.scales, L.out_scale, return_f64=True)[1]
    if resid:
        out = out + O.bf16_to_f64(got["h"])
    w.append(assert_close(got["out"], O.f64_to_bf16(out), "out"))
    return w


@pytest.mark.parametrize("M,H,I", [(16, 4096, 14336), (5, 512, 640), (8, 1024, 2048), (16, 384, 256),
                                   (12, 1536, 8960)])
def test_mlp_decode2_matrix_core_both_residual_modes(M, H, I):
    say(f"[mlp2, matrix cores] M={M} H={H} I={I}")
    inp = synth.mlp_inputs(M, H, I, n_layers=1, seed=M + H + I + 2)
    for resid in (True, False):
        layer = dev_layers(inp, resid)[0]
        b = F.Mlp2Buffers.empty(M, H, I)
        b.x.copy_(F.from_bits(inp.x))
        b.residual.copy_(F.from_bits(inp.r))
        ws = F.workspace(F.mlp2_workspace_bytes(M, H, I))
        F.mlp_decode2(layer, b, ws)
        torch.cuda.synchronize()
        y = ws[: M * H * 2].view(torch.int16).view(torch.bfloat16).reshape(M, H)
        got = {"h": F.to_bits(b.residual), "y": F.to_bits(y), "act": F.to_bits(b.act), "out": F.to_bits(b.out)}
        say(f"  resid={resid} worst err/bound (y, act, out)", check_layer2_mc(inp.layers[0], inp.x, inp.r, got, resid))


@pytest.mark.parametrize("M,H,I", [(16, 4096, 14336), (5, 4096, 1152), (12, 3584, 2048), (8, 1024, 2048)])
def test_mlp_decode2_gate_up_reads_the_norms_staged_copy(M, H, I):
    # From 5 rows the norm kernel also writes y as the matrix-core GEMVs stage it, and the
    # row-block gate_up copies that instead of staging y itself; its act must be bit-identical
    # to the standalone gate_up's on the same y (which stages y itself).  At H = 1024 the
    # gate_up runs on the ring kernel, which stages from y either way.
    say(f"[mlp2, staged y] M={M} H={H} I={I}")
    inp = synth.mlp_inputs(M, H, I, n_layers=1, seed=M * 5 + H + I)
    layer = dev_layers(inp, True)[0]
    b = F.Mlp2Buffers.empty(M, H, I)
    b.x.copy_(F.from_bits(inp.x))
    b.residual.copy_(F.from_bits(inp.r))
    ws = torch.full((F.mlp2_workspace_bytes(M, H, I),), 0xFF, dtype=torch.uint8, device="cuda")
    F.mlp_decode2(layer, b, ws)
    torch.cuda.synchronize()
    y = ws[: M * H * 2].view(torch.int16).view(torch.bfloat16).reshape(M, H).clone()
    act = F.to_bits(F.w4_gemv_swiglu(y, layer.gate_up))
    assert_bits_equal(F.to_bits(b.act), act, "act: staged copy vs staged by the gate_up itself")


def test_chain2_matrix_core_graph():
    M, H, I, n = 16, 512, 1024, 4
    say(f"[chain2, matrix cores] M={M} H={H} I={I}, {n} layers: every layer, graph == eager")
    inp = synth.mlp_inputs(M, H, I, n_layers=n, seed=77)
    layers = dev_layers(inp, False)
    b = F.Mlp2Buffers.empty(M, H, I, out_is_x=True)
    ws = F.workspace(F.mlp2_workspace_bytes(M, H, I))
    b.x.copy_(F.from_bits(inp.x))
    b.residual.copy_(F.from_bits(inp.r))
    trace = []
    for L in layers:
        xin, rin = F.to_bits(b.x), F.to_bits(b.residual)
        F.mlp_decode2(L, b, ws)
        torch.cuda.synchronize()
        y = ws[: M * H * 2].view(torch.int16).view(torch.bfloat16).reshape(M, H)
        trace.append({"x": xin, "r": rin, "h": F.to_bits(b.residual), "y": F.to_bits(y), "act": F.to_bits(b.act),
                      "out": F.to_bits(b.x)})
    for l, t in enumerate(trace):
        check_layer2_mc(inp.layers[l], t["x"], t["r"], t, False)
    b.x.copy_(F.from_bits(inp.x))
    b.residual.copy_(F.from_bits(inp.r))
    F.mlp_chain2(layers, b, ws)
    torch.cuda.synchronize()
    assert_bits_equal(F.to_bits(b.x), trace[-1]["out"], "chain x")
    assert_bits_equal(F.to_bits(b.residual), trace[-1]["h"], "chain r")
    graph = F.Mlp2Graph(layers, b, ws)
    # three kernels per layer, plus a slice-summing kernel after each K-split GEMV
    assert 3 * n <= graph.kernel_count <= 5 * n
    for rep in range(3):
        b.x.copy_(F.from_bits(inp.x))
        b.residual.copy_(F.from_bits(inp.r))
        graph.launch()
        torch.cuda.synchronize()
        assert_bits_equal(F.to_bits(b.x), trace[-1]["out"], f"graph replay {rep} x")
        assert_bits_equal(F.to_bits(b.residual), trace[-1]["h"], f"graph replay {rep} r")
        torch.randn(1 << 20, device="cuda").sum().item()
    graph.close()
