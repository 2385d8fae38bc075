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

CASES = ["tiny", "20b_decode", "20b_mxfp4_decode"]


def _eager(g: GpuLayer) -> torch.Tensor:
    g.forward(want_routing=True)
    torch.cuda.synchronize()
    return g.y.clone()


@pytest.mark.parametrize("name", CASES)
def test_graph_replay_matches_eager(name):
    layer = synth.make_layer(name)
    g = GpuLayer(layer)
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
