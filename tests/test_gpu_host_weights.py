"""Host-streamed experts: the decode layer with its expert weights in pinned
host memory (read over the host link by the same skinny kernels) gives the
same output, bit for bit, as with the weights resident in HBM; that output
is parity-checked against the oracle in test_gpu_parity.py.  The MXFP4
layer is checked in the row-major and in the packed order."""
from __future__ import annotations

import pytest
import torch

import mixture_experts_ffn_05_amd as moe
import synth
from tests.gpu_layer import GpuLayer
from tests.host_weights import pinned_weights

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["tiny", "20b_decode", "20b_mxfp4_decode", "20b_mxfp4_decode+packed"])
def test_host_resident_weights_match_device_resident(name):
    print(f"host-resident weights {name}", flush=True)
    packed = name.endswith("+packed")
    layer = synth.make_layer(name.split("+")[0])
    g = GpuLayer(layer, packed=packed)
    g.forward()
    torch.cuda.synchronize()
    ref = g.y.clone()
    w = layer.weights
    if packed:  # the device-packed weights, copied to the host
        w = synth.Weights(1, *(t.cpu().numpy() for t in (g.gate_up, g.down, g.gate_up_scale, g.down_scale)))
    parts = pinned_weights(w)
    if parts is None:
        pytest.skip("pinned host memory is not mapped for the device on this runtime")
    ptrs = [p.dev for p in parts] + [None, None]
    g.weights = moe.expert_weights(ptrs[0], ptrs[1], ptrs[2], ptrs[3])
    g.y.zero_()
    g.forward()
    torch.cuda.synchronize()
    assert torch.equal(g.y, ref)
