"""Near ties in the router on every top-k path of the GPU (per-token ranks for
E <= 64 in the small-batch select+permute kernel of up to 8 tokens and in
the per-token selection kernel, arg-max rounds for E > 64, the selection fused into the
fp64 matrix-core logits kernel from 1024 tokens).  The inputs
(synth.near_tie_router) have logits that are exact in fp64 whatever the
summation order, with two experts 2^-20 apart near 512 (relative 2^-29), an
exact tie, and a fifth expert 2^-20 below the tie: every token must take the
designed experts in the designed order, bit-exact against the oracle, with
weights within 1e-5, through both moe_route and moe_forward."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_layer import GpuLayer

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,E", [(8, 32), (8, 128), (16, 32), (16, 128), (300, 64), (2048, 32), (2048, 128)], ids=lambda v: str(v))
def test_near_ties(T, E):
    H, k, I = 256, 4, 64
    print(f"[near-tie] T={T} E={E}", flush=True)
    x, wr = synth.near_tie_router(T, H, E, seed=T + E)
    cfg = synth.LayerConfig(f"nt_T{T}_E{E}", T=T, H=H, E=E, k=k, I=I, seed=3)
    weights = synth.make_weights(cfg)
    layer = synth.Layer(cfg, x, wr, weights)
    nt = synth.NEAR_TIE
    want = np.array([nt["A2"], nt["A1"], nt["B1"], nt["B2"]], np.int32)
    _, idx_ref, w_ref = oracle.get().route(x, wr, k)
    assert (idx_ref == want).all()
    g = GpuLayer(layer)
    g.route()
    torch.cuda.synchronize()
    assert (g.topk_idx.cpu().numpy() == want).all()
    assert np.max(np.abs(g.topk_w.cpu().numpy() - w_ref)) <= 1e-5
    g.topk_idx.fill_(-1)
    g.forward()
    torch.cuda.synchronize()
    assert (g.topk_idx.cpu().numpy() == want).all()
    assert np.max(np.abs(g.topk_w.cpu().numpy() - w_ref)) <= 1e-5
