"""Small-batch routing: for up to 8 tokens moe_forward runs selection and
permutation as one workgroup after the logits kernel (select_permute_small),
above that the parallel selection kernel and the permutation kernel; the
stage entry points run moe_route (logits, then a per-token selection kernel)
and moe_permute as separate launches.  Both must take the same decisions:
routing indices and weights and the layer output identical bits, indices
equal to the oracle's, output within 1e-2 * max|ref|.  Shapes cover one
token, k = E, 64 pairs in one wave (8 tokens x 8 experts), 64 experts, one
expert per token, exactly tied logits (duplicated router rows, resolved to the
lower index) and the 20b MXFP4 decode layer, on both sides of the 8-token
switch, with bf16 and packed MXFP4 experts."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_layer import GpuLayer, bf16_dev_to_f64, rel_err

pytestmark = pytest.mark.gpu

TOL = 1e-2

SHAPES = [(16, 256, 32, 4, 128), (1, 128, 8, 2, 64), (5, 192, 64, 8, 128), (64, 128, 16, 1, 64),
          (16, 64, 64, 4, 64), (3, 64, 3, 3, 64), (13, 128, 24, 4, 192), (8, 64, 64, 8, 64),
          (8, 128, 32, 4, 128), (9, 128, 32, 4, 128)]


def _check(layer, tag):
    c = layer.cfg
    print(f"[small-route] {tag}", flush=True)
    g = GpuLayer(layer, packed=c.wfmt == 1)
    g.y.fill_(0)
    g.forward()
    torch.cuda.synchronize()
    idx_f, w_f, y_f = g.topk_idx.clone(), g.topk_w.clone(), g.y.clone()
    g.y.fill_(0)
    g.stages()
    torch.cuda.synchronize()
    assert torch.equal(idx_f, g.topk_idx)
    assert torch.equal(w_f.view(torch.int32), g.topk_w.view(torch.int32))
    assert torch.equal(y_f, g.y)
    orc = oracle.get()
    _, idx_ref, w_ref = orc.route(layer.x, layer.w_router, c.k)
    assert np.array_equal(idx_f.cpu().numpy(), idx_ref)
    assert np.max(np.abs(w_f.cpu().numpy() - w_ref)) <= 1e-5
    tokens = np.arange(c.T) if c.T <= 64 else synth.sample_tokens(c.T, 64, 3)
    y_ref, _, _ = orc.forward_tokens(layer.x, layer.w_router, layer.weights, c.k, c.I, tokens)
    e = rel_err(bf16_dev_to_f64(y_f)[tokens], y_ref)
    print(f"[small-route] {tag} rel err y {e:.2e}")
    assert e <= TOL, e


@pytest.mark.parametrize("wfmt", [0, 1], ids=["bf16", "mxfp4_packed"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "T{}_H{}_E{}_k{}_I{}".format(*s))
def test_small_routing_matches_staged(shape, wfmt):
    T, H, E, k, I = shape
    cfg = synth.LayerConfig(f"sr_T{T}_H{H}_E{E}_k{k}_I{I}", T=T, H=H, E=E, k=k, I=I, wfmt=wfmt, seed=11)
    _check(synth.make_layer(cfg), cfg.name)


@pytest.mark.parametrize("T", [16, 8])
def test_small_routing_ties(T):
    """Router rows 2, 5 and 7 equal: their logits tie exactly for every token
    and go to the lower index."""
    cfg = synth.LayerConfig(f"sr_ties_T{T}", T=T, H=128, E=16, k=4, I=64, wfmt=1, seed=12)
    layer = synth.make_layer(cfg)
    wr = layer.w_router.copy()
    wr[5] = wr[2]
    wr[7] = wr[2]
    _check(synth.Layer(cfg, layer.x, wr, layer.weights), cfg.name)


@pytest.mark.parametrize("T", [16, 8, 1])
def test_small_routing_20b(T):
    cfg = synth.CONFIGS["20b_mxfp4_decode"].with_T(T)
    w = synth.make_weights(synth.CONFIGS["20b_mxfp4_decode"])
    layer = synth.Layer(cfg, synth.make_x(cfg), synth.make_router(cfg), w)
    _check(layer, f"20b_mxfp4_decode@{T}")
