"""GPU tests of the graph parameter update (fdec_mlp_graph_update, _update2): a graph
captured on one set of layers and buffers is re-pointed at another set of the same
shapes and must then replay exactly what an eager chain computes on that set.  The eager
chains' parity with the oracle is tested layer by layer in test_gpu_mlp.py and
test_gpu_mlp2.py; here the first layer of each new set is checked against the oracle too."""
import numpy as np
import pytest
import torch

import memory_bound_decode_add_amd as F
import synth
from helpers import assert_bits_equal, say
from test_gpu_mlp import check_layer, dev_layers
from test_gpu_mlp2 import check_layer2, check_layer2_mc

pytestmark = pytest.mark.gpu

UNSUP = -6


def eager_chain(inp, layers, M, H, I, two_kernel):
    """The chain launched eagerly on fresh buffers: final (x, residual) bits."""
    if two_kernel:
        b = F.Mlp2Buffers.empty(M, H, I, out_is_x=True)
    else:
        b = F.MlpBuffers.empty(M, H, I, out_is_x=True)
    b.x.copy_(F.from_bits(inp.x))
    b.residual.copy_(F.from_bits(inp.r))
    (F.mlp_chain2 if two_kernel else F.mlp_chain)(layers, b)
    torch.cuda.synchronize()
    return F.to_bits(b.x), F.to_bits(b.residual)


def first_layer_parity(inp, layer, M, H, I, two_kernel):
    """The first layer of a set, eagerly, against the oracle."""
    if two_kernel:
        b = F.Mlp2Buffers.empty(M, H, I)
        b.x.copy_(F.from_bits(inp.x))
        b.residual.copy_(F.from_bits(inp.r))
        ws = F.workspace(F.mlp2_workspace_bytes(M, H, I))
        F.mlp_decode2(layer, b, ws)
        torch.cuda.synchronize()
        got = {"h": F.to_bits(b.residual), "act": F.to_bits(b.act), "out": F.to_bits(b.out)}
        if M <= 4:
            check_layer2(inp.layers[0], inp.x, inp.r, got, False)
        else:   # the matrix-core form: y is in the workspace
            got["y"] = F.to_bits(ws[: M * H * 2].view(torch.int16).view(torch.bfloat16).reshape(M, H))
            check_layer2_mc(inp.layers[0], inp.x, inp.r, got, False)
    else:
        b = F.MlpBuffers.empty(M, H, I)
        b.x.copy_(F.from_bits(inp.x))
        b.residual.copy_(F.from_bits(inp.r))
        F.mlp_decode(layer, b)
        torch.cuda.synchronize()
        got = {"h": F.to_bits(b.residual), "y": F.to_bits(b.y_norm), "gu": F.to_bits(b.gate_up),
               "out": F.to_bits(b.out)}
        check_layer(inp.layers[0], inp.x, inp.r, got, False)


def replay_and_check(graph, b, inp, want, tag):
    for rep in range(3):
        b.x.copy_(F.from_bits(inp.x))
        b.residual.copy_(F.from_bits(inp.r))
        graph.launch()
        torch.cuda.synchronize()
        assert_bits_equal(F.to_bits(b.x), want[0], f"{tag} replay {rep} x")
        assert_bits_equal(F.to_bits(b.residual), want[1], f"{tag} replay {rep} r")
        torch.randn(1 << 20, device="cuda").sum().item()     # unrelated eager work between replays


@pytest.mark.parametrize("two_kernel,M,H,I,n", [(False, 1, 256, 512, 4), (False, 16, 384, 256, 3),
                                                (True, 1, 1536, 8960, 4), (True, 3, 512, 640, 3),
                                                (True, 16, 384, 256, 3)])
def test_graph_update_repoints_layers_and_buffers(two_kernel, M, H, I, n):
    say(f"[graph update] {'two' if two_kernel else 'three'}-kernel layers, M={M} H={H} I={I}, {n} layers")
    inp_a = synth.mlp_inputs(M, H, I, n_layers=n, seed=101 + M)
    inp_b = synth.mlp_inputs(M, H, I, n_layers=n, seed=202 + M)
    lay_a, lay_b = dev_layers(inp_a, False), dev_layers(inp_b, False)
    want_a = eager_chain(inp_a, lay_a, M, H, I, two_kernel)
    want_b = eager_chain(inp_b, lay_b, M, H, I, two_kernel)
    first_layer_parity(inp_b, lay_b[0], M, H, I, two_kernel)
    Bufs, Graph = (F.Mlp2Buffers, F.Mlp2Graph) if two_kernel else (F.MlpBuffers, F.MlpGraph)
    ba, bb = Bufs.empty(M, H, I, out_is_x=True), Bufs.empty(M, H, I, out_is_x=True)

    graph = Graph(lay_a, ba)
    kernels = graph.kernel_count
    replay_and_check(graph, ba, inp_a, want_a, "before update")

    graph.update(lay_b, bb)
    assert graph.kernel_count == kernels
    sentinel = torch.full_like(ba.x, 7.0)
    ba.x.copy_(sentinel)
    replay_and_check(graph, bb, inp_b, want_b, "after update")
    assert torch.equal(ba.x, sentinel), "the updated graph still wrote the old buffers"

    # other shapes are refused and leave the graph as it was
    with pytest.raises(F.FdecError) as e:
        graph.update(lay_b[: n - 1], bb)
    assert e.value.status == UNSUP
    replay_and_check(graph, bb, inp_b, want_b, "after a refused update")

    # and back to the first set
    graph.update(lay_a, ba)
    replay_and_check(graph, ba, inp_a, want_a, "updated back")
    assert not np.array_equal(want_a[0], want_b[0])
    graph.close()


def test_graph_update_refuses_the_other_layer_form():
    say("[graph update] a three-kernel graph refuses a two-kernel update")
    M, H, I = 1, 256, 512
    inp = synth.mlp_inputs(M, H, I, n_layers=2, seed=303)
    layers = dev_layers(inp, False)
    b = F.MlpBuffers.empty(M, H, I, out_is_x=True)
    graph = F.MlpGraph(layers, b)
    b2 = F.Mlp2Buffers.empty(M, H, I, out_is_x=True)
    ws = F.workspace(F.mlp2_workspace_bytes(M, H, I))
    arr = F._layer_array(layers)
    st = F.lib().fdec_mlp_graph_update2(graph._handle, arr, 2, M, b2.x.data_ptr(), b2.residual.data_ptr(),
                                        b2.act.data_ptr(), ws.data_ptr(), ws.numel(),
                                        torch.cuda.Stream().cuda_stream)
    assert st == UNSUP
    want = eager_chain(inp, layers, M, H, I, False)
    replay_and_check(graph, b, inp, want, "after a refused form change")
    graph.close()


def test_graph_update_with_other_kernels_keeps_a_consistent_graph():
    """Forcing the split-K GEMV makes the re-captured chain use other kernel functions.
    Either HIP takes the update (the graph then replays the split-K chain on the new
    buffers) or it refuses (FDEC_ERR_UNSUPPORTED, and the graph keeps replaying the old
    chain on the old buffers); both are checked bit for bit against eager chains."""
    say("[graph update] re-captured chain with other kernel functions")
    M, H, I = 1, 256, 512
    inp_a = synth.mlp_inputs(M, H, I, n_layers=2, seed=404)
    inp_b = synth.mlp_inputs(M, H, I, n_layers=2, seed=505)
    lay_a, lay_b = dev_layers(inp_a, False), dev_layers(inp_b, False)
    want_a = eager_chain(inp_a, lay_a, M, H, I, False)
    ba, bb = F.MlpBuffers.empty(M, H, I, out_is_x=True), F.MlpBuffers.empty(M, H, I, out_is_x=True)
    graph = F.MlpGraph(lay_a, ba)
    replay_and_check(graph, ba, inp_a, want_a, "before")
    F.set_gemv_split(2)
    try:
        want_b_split = eager_chain(inp_b, lay_b, M, H, I, False)
        try:
            graph.update(lay_b, bb)
            took = True
        except F.FdecError as e:
            assert e.status == UNSUP
            took = False
    finally:
        F.set_gemv_split(0)
    say(f"  update {'taken' if took else 'refused'}")
    if took:
        # the split-K chain has a finish kernel after each K-sliced GEMV
        F.set_gemv_split(2)
        try:
            fresh = F.MlpGraph(lay_b, F.MlpBuffers.empty(M, H, I, out_is_x=True))
            assert graph.kernel_count == fresh.kernel_count
            fresh.close()
        finally:
            F.set_gemv_split(0)
        replay_and_check(graph, bb, inp_b, want_b_split, "after a taken update")
    else:
        replay_and_check(graph, ba, inp_a, want_a, "after a refused update")
    graph.close()
