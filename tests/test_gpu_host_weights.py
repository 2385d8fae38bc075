"""Host-streamed experts: the decode layer with its expert weights in pinned
host memory (read over the host link by the same skinny kernels) gives the
same output, bit for bit, as with the weights resident in HBM; that output
is parity-checked against the oracle in test_gpu_parity.py."""
from __future__ import annotations

import pytest
import torch

import mixture_experts_ffn_05_amd as moe
import synth
from tests.gpu_layer import GpuLayer
from tests.host_weights import pinned_weights

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["tiny", "20b_decode", "20b_mxfp4_decode"])
def test_host_resident_weights_match_device_resident(name):
    print(f"host-resident weights {name}", flush=True)
    layer = synth.make_layer(name)
    g = GpuLayer(layer)
    g.forward()
    torch.cuda.synchronize()
    ref = g.y.clone()
    parts = pinned_weights(layer.weights)
    if parts is None:
        pytest.skip("pinned host memory is not mapped for the device on this runtime")
    ptrs = [p.dev for p in parts] + [None, None]
    g.weights = moe.expert_weights(ptrs[0], ptrs[1], ptrs[2], ptrs[3])
    g.y.zero_()
    g.forward()
    torch.cuda.synchronize()
    assert torch.equal(g.y, ref)
