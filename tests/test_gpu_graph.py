"""moe_forward captured into a HIP graph (torch.cuda.CUDAGraph) and replayed.

The library enqueues kernels only (no allocation, memset or host sync), so a
whole layer can be captured once and replayed.  Each replay is checked bit
for bit against the eager result, with eager work and synchronisations
between the replays, and the replays see new input values written into the
captured buffers.
"""
from __future__ import annotations

import pytest
import torch

import synth
from tests.gpu_layer import GpuLayer

pytestmark = pytest.mark.gpu

CASES = ["tiny", "20b_decode", "20b_mxfp4_decode", "20b_mxfp4_decode+packed"]


def _eager(g: GpuLayer) -> torch.Tensor:
    g.forward(want_routing=True)
    torch.cuda.synchronize()
    return g.y.clone()


@pytest.mark.parametrize("name", CASES)
def test_graph_replay_matches_eager(name):
    layer = synth.make_layer(name.split("+")[0])
    g = GpuLayer(layer, packed=name.endswith("+packed"))
    ref = _eager(g)  # also warms up the library (kernel attributes, occupancy)
    x0 = g.x.clone()
    x1 = torch.roll(x0, shifts=1, dims=0).contiguous()  # different tokens, same values
    g.x.copy_(x1)
    ref1 = _eager(g)
    g.x.copy_(x0)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            g.forward(want_routing=True)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    for rep in range(4):
        xin, want = (x0, ref) if rep % 2 == 0 else (x1, ref1)
        g.x.copy_(xin)
        g.y.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(g.y, want), f"{name}: replay {rep} differs from the eager result"
        # eager work between replays
        _ = _eager(g)
        g.x.copy_(xin)
        torch.cuda.synchronize()


def test_backward_graph_replay_matches_eager():
    """moe_backward also only enqueues kernels: captured once, replayed with
    eager work between replays, bit-identical to the eager gradients."""
    import numpy as np

    import mixture_experts_ffn_05_amd as moe
    from tests.gpu_layer import to_dev
    layer = synth.make_layer("tiny")
    c = layer.cfg
    g = GpuLayer(layer)
    dy = to_dev(synth.bf16_from_f32(np.random.default_rng(3).standard_normal((c.T, c.H)).astype(np.float32)))
    d = moe.dims(c.T, c.H, c.E, c.k, c.I)
    nbytes = moe.moe_backward_workspace_size(d)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    outs = [torch.empty((c.T, c.H), dtype=torch.int16, device="cuda"),
            torch.empty((c.E, c.H), dtype=torch.float32, device="cuda"),
            torch.empty((c.E, 2 * c.I, c.H), dtype=torch.float32, device="cuda"),
            torch.empty((c.E, c.H, c.I), dtype=torch.float32, device="cuda")]
    W = moe.expert_weights(g.gate_up, g.down)

    def run():
        moe.moe_backward(d, g.x, g.w_router, W, dy, *outs, ws, nbytes)

    run()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            assert torch.equal(o, r), f"backward replay {rep} differs from the eager result"
        run()  # eager work between replays
        torch.cuda.synchronize()
