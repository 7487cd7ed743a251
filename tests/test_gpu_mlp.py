"""GPU parity of the three-kernel decode-MLP layer, the multi-layer chain and its
hipGraph capture, against the fp64 oracle."""
import numpy as np
import pytest
import torch

import memory_bound_decode_add_amd as F
import oracle as O
import synth
from helpers import assert_bits_equal, assert_close, say

pytestmark = pytest.mark.gpu


def dev_layers(inp: synth.MlpInputs, residual_in_epilogue):
    out = []
    for L in inp.layers:
        out.append(F.MlpLayer(F.from_bits(L.norm_w), F.W4Weight.from_numpy(L.gate_up.qweight, L.gate_up.scales),
                              F.W4Weight.from_numpy(L.down.qweight, L.down.scales), F.scalar(L.out_scale),
                              L.eps, residual_in_epilogue))
    return out


def check_layer(L, x, r, got, resid):
    """Each of the layer's three kernels against the oracle fed the bf16 inputs that
    kernel read (the per-call tolerance applies per call; an oracle chaining its own
    intermediates would also measure how rounding differences propagate)."""
    h, y = O.add_rmsnorm(x, r, L.norm_w, L.eps)
    assert_bits_equal(got["h"], h, "h")
    w = [assert_close(got["y"], y, "y")]
    gu = O.w4_gemv(got["y"], L.gate_up.qweight, L.gate_up.scales)
    w.append(assert_close(got["gu"], gu, "gate_up"))
    I = L.down.qweight.shape[1] * 8
    out = O.swiglu_w4_gemv(got["gu"][:, :I], got["gu"][:, I:], L.down.qweight, L.down.scales, L.out_scale,
                           got["h"] if resid else None)
    w.append(assert_close(got["out"], out, "out"))
    return w


def test_mlp_layer_llama3_8b_m16():
    say("[mlp] M=16 H=4096 I=14336, residual in the epilogue")
    inp = synth.make("mlp_llama3_8b_m16")
    layer = dev_layers(inp, True)[0]
    b = F.MlpBuffers.empty(16, 4096, 14336)
    b.x.copy_(F.from_bits(inp.x))
    b.residual.copy_(F.from_bits(inp.r))
    F.mlp_decode(layer, b)
    torch.cuda.synchronize()
    got = {"h": F.to_bits(b.residual), "y": F.to_bits(b.y_norm), "gu": F.to_bits(b.gate_up),
           "out": F.to_bits(b.out)}
    say("  worst err/bound (y, gu, out)", check_layer(inp.layers[0], inp.x, inp.r, got, True))


@pytest.mark.parametrize("M,H,I", [(16, 4096, 14336), (5, 4096, 1152), (12, 3584, 2048), (8, 1024, 2048)])
def test_mlp_layer_gate_up_reads_the_norms_staged_copy(M, H, I):
    # From 5 rows the norm kernel also writes y staged for the matrix cores, and a row-block
    # gate_up copies that instead of staging y itself: gate_up must be bit-identical to the
    # standalone GEMV's on the same y_norm (which stages it itself).  At H = 1024 the
    # gate_up runs on the ring kernel, which stages from y_norm either way.
    say(f"[mlp, staged y] M={M} H={H} I={I}")
    inp = synth.mlp_inputs(M, H, I, n_layers=1, seed=M * 7 + H + I)
    layer = dev_layers(inp, True)[0]
    b = F.MlpBuffers.empty(M, H, I)
    b.x.copy_(F.from_bits(inp.x))
    b.residual.copy_(F.from_bits(inp.r))
    ws = torch.full((max(16, F.mlp_workspace_bytes(M, H, I)),), 0xFF, dtype=torch.uint8, device="cuda")
    F.mlp_decode(layer, b, ws)
    torch.cuda.synchronize()
    gu = F.to_bits(F.w4_gemv(b.y_norm.clone(), layer.gate_up))
    assert_bits_equal(F.to_bits(b.gate_up), gu, "gate_up: staged copy vs staged by the GEMV itself")


@pytest.mark.parametrize("M,H,I", [(1, 256, 384), (3, 512, 640), (16, 384, 256)])
def test_mlp_layer_small_shapes_both_residual_modes(M, H, I):
    say(f"[mlp] M={M} H={H} I={I}")
    inp = synth.mlp_inputs(M, H, I, n_layers=1, seed=M + H + I)
    for resid in (True, False):
        layer = dev_layers(inp, resid)[0]
        b = F.MlpBuffers.empty(M, H, I)
        b.x.copy_(F.from_bits(inp.x))
        b.residual.copy_(F.from_bits(inp.r))
        F.mlp_decode(layer, b)
        got = {"h": F.to_bits(b.residual), "y": F.to_bits(b.y_norm), "gu": F.to_bits(b.gate_up),
               "out": F.to_bits(b.out)}
        check_layer(inp.layers[0], inp.x, inp.r, got, resid)


def test_chain_small_per_layer_and_chain_calls():
    """Chains are checked layer by layer: each layer's outputs against the oracle fed the
    bf16 inputs that layer read.  Comparing the last layer against the oracle's own chain
    is not a parity test: two correct roundings of a layer differ by a bf16 step here and
    there, and later layers amplify the difference past the per-call tolerance."""
    say("[chain] M=1 H=256 I=512, 4 layers: per layer, eager chain, graph")
    inp = synth.mlp_inputs(1, 256, 512, n_layers=4, seed=21)
    layers = dev_layers(inp, False)
    trace = run_layers_eagerly(inp, layers, 1, 256, 512)
    for l, t in enumerate(trace):
        check_layer(inp.layers[l], t["x"], t["r"], t, False)
    b = F.MlpBuffers.empty(1, 256, 512, out_is_x=True)
    b.x.copy_(F.from_bits(inp.x))
    b.residual.copy_(F.from_bits(inp.r))
    F.mlp_chain(layers, b)
    assert_bits_equal(F.to_bits(b.x), trace[-1]["out"], "chain x")
    assert_bits_equal(F.to_bits(b.residual), trace[-1]["h"], "chain r")
    g = F.MlpGraph(layers, b)
    b.x.copy_(F.from_bits(inp.x))
    b.residual.copy_(F.from_bits(inp.r))
    g.launch()
    torch.cuda.synchronize()
    assert_bits_equal(F.to_bits(b.x), trace[-1]["out"], "graph x")
    g.close()


def run_layers_eagerly(inp, layers, M, H, I):
    """Run the chain layer by layer, keeping every layer's inputs and outputs."""
    b = F.MlpBuffers.empty(M, H, I, out_is_x=True)
    b.x.copy_(F.from_bits(inp.x))
    b.residual.copy_(F.from_bits(inp.r))
    ws = F.workspace(F.mlp_workspace_bytes(M, H, I))
    trace = []
    for L in layers:
        xin, rin = F.to_bits(b.x), F.to_bits(b.residual)
        F.mlp_decode(L, b, ws)
        torch.cuda.synchronize()
        trace.append({"x": xin, "r": rin, "h": F.to_bits(b.residual), "y": F.to_bits(b.y_norm),
                      "gu": F.to_bits(b.gate_up), "out": F.to_bits(b.x)})
    return trace


def test_chain_qwen2_5_1_5b_28_layers_graph():
    say("[chain] M=1 H=1536 I=8960, 28 layers: parity of every layer, graph == eager")
    inp = synth.make("mlp_qwen2_5_1_5b_28l")
    M, H, I = 1, 1536, 8960
    layers = dev_layers(inp, False)
    trace = run_layers_eagerly(inp, layers, M, H, I)
    for l in range(28):
        say(f"  layer {l}")
        t = trace[l]
        check_layer(inp.layers[l], t["x"], t["r"], t, False)

    # the same chain through one eager call and through a captured graph
    b = F.MlpBuffers.empty(M, H, I, out_is_x=True)
    ws = F.workspace(F.mlp_workspace_bytes(M, H, I))
    b.x.copy_(F.from_bits(inp.x))
    b.residual.copy_(F.from_bits(inp.r))
    F.mlp_chain(layers, b, ws)
    torch.cuda.synchronize()
    assert_bits_equal(F.to_bits(b.x), trace[-1]["out"], "chain x")
    assert_bits_equal(F.to_bits(b.residual), trace[-1]["h"], "chain r")

    graph = F.MlpGraph(layers, b, ws)
    assert graph.kernel_count == 3 * 28
    for rep in range(3):
        b.x.copy_(F.from_bits(inp.x))
        b.residual.copy_(F.from_bits(inp.r))
        graph.launch()
        torch.cuda.synchronize()
        assert_bits_equal(F.to_bits(b.x), trace[-1]["out"], f"graph replay {rep} x")
        assert_bits_equal(F.to_bits(b.residual), trace[-1]["h"], f"graph replay {rep} r")
        # unrelated eager work between replays
        torch.randn(1 << 20, device="cuda").sum().item()
    graph.close()


def test_graph_reads_scale_at_replay():
    say("[graph] out_scale changed in device memory between replays")
    inp = synth.mlp_inputs(1, 256, 384, n_layers=2, seed=31)
    layers = dev_layers(inp, False)
    b = F.MlpBuffers.empty(1, 256, 384, out_is_x=True)
    graph = F.MlpGraph(layers, b)
    outs = {}
    for v in (0.5, 2.0):
        for L in layers:
            L.out_scale.fill_(v)
        b.x.copy_(F.from_bits(inp.x))
        b.residual.copy_(F.from_bits(inp.r))
        graph.launch()
        torch.cuda.synchronize()
        outs[v] = F.to_bits(b.x)
        for L in inp.layers:
            L.out_scale = v
        trace = run_layers_eagerly(inp, layers, 1, 256, 384)
        assert_bits_equal(outs[v], trace[-1]["out"], f"graph vs eager, scale {v}")
        for l, t in enumerate(trace):
            check_layer(inp.layers[l], t["x"], t["r"], t, False)
    assert not np.array_equal(outs[0.5], outs[2.0])
    graph.close()
