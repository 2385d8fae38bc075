"""GPU parity of moe_backward against the oracle's backward.

Bar: every gradient tensor within max|gpu - ref| <= 1e-2 * max|ref| (the
layer's tolerance; the GPU keeps w*dy, g, u, [dg; du] and the per-pair dx in
bf16 and accumulates in fp32).  Inputs: x ~ N(0, 1), router and expert
weights ~ N(0, 0.02) in bf16 (the layer generator), dy ~ N(0, 1) bf16.

Cases: the tiny config; ragged H and I (multiples of 32 only, so GEMM and
transpose tiles have tails) with one expert that never receives a token;
k = E; E = 1; the 20b shape at 16 tokens; and the 20b prefill config with
Zipf routing (8192 tokens) in its full launch configuration, with dy
nonzero on 16 seeded tokens only: the gradients are linear in dy, so the
exact reference is the oracle's backward of those 16 tokens alone, and every
other token's dx must be exactly zero.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mixture_experts_ffn_05_amd as moe
import oracle
import synth
from tests.gpu_layer import bf16_dev_to_f64, rel_err, to_dev

pytestmark = pytest.mark.gpu

TOL = 1e-2


def _gpu_backward(x, wr, gate_up, down, dy, k):
    T, H = x.shape
    E, twoI, _ = gate_up.shape
    I = twoI // 2
    d = moe.dims(T, H, E, k, I)
    nbytes = moe.moe_backward_workspace_size(d)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda")
    dx = torch.empty((T, H), dtype=torch.int16, device="cuda")
    dwr = torch.empty((E, H), dtype=torch.float32, device="cuda")
    dgu = torch.empty((E, 2 * I, H), dtype=torch.float32, device="cuda")
    ddn = torch.empty((E, H, I), dtype=torch.float32, device="cuda")
    g_gu, g_dn = to_dev(gate_up), to_dev(down)
    moe.moe_backward(d, to_dev(x), to_dev(wr), moe.expert_weights(g_gu, g_dn), to_dev(dy), dx, dwr, dgu, ddn, ws,
                     nbytes)
    torch.cuda.synchronize()
    return bf16_dev_to_f64(dx), dwr.cpu().numpy(), dgu.cpu().numpy(), ddn.cpu().numpy()


def _compare(got, ref, what):
    for name, g, r in zip(("dx", "dw_router", "dgate_up", "ddown"), got, ref):
        err = rel_err(np.asarray(g, np.float64), r)
        assert err <= TOL, f"{what}: {name} max err {err:.3g} of max|ref| {np.max(np.abs(r)):.3g}"


def _layer(T, H, E, k, I, seed, dead_expert=False):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H))
    wr = rng.standard_normal((E, H)) * 0.02
    if dead_expert:  # a constant input channel keeps expert E-1 out of every top-k
        x[:, H - 1] = 1.0
        wr[E - 1, H - 1] = -8.0
    b = synth.bf16_from_f32
    gu = b((rng.standard_normal((E, 2 * I, H)) * 0.02).astype(np.float32))
    dn = b((rng.standard_normal((E, H, I)) * 0.02).astype(np.float32))
    dy = b(rng.standard_normal((T, H)).astype(np.float32))
    return b(x.astype(np.float32)), b(wr.astype(np.float32)), gu, dn, dy


CASES = {
    "ragged_dead_expert": dict(T=37, H=160, E=6, k=2, I=96, seed=1, dead_expert=True),
    "k_equals_E": dict(T=24, H=64, E=4, k=4, I=96, seed=2),
    "E1": dict(T=19, H=96, E=1, k=1, I=64, seed=3),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_backward_small(name):
    c = CASES[name]
    print(f"backward parity {name} {c}", flush=True)
    x, wr, gu, dn, dy = _layer(**c)
    if name == "ragged_dead_expert":
        idx = oracle.get().route(x, wr, c["k"])[1]
        assert not np.any(idx == c["E"] - 1), "the dead expert received a token"
    ref = oracle.get().backward(x, wr, gu, dn, dy, c["k"])
    got = _gpu_backward(x, wr, gu, dn, dy, c["k"])
    _compare(got, ref, name)
    if name == "ragged_dead_expert":
        assert np.all(got[2][c["E"] - 1] == 0) and np.all(got[3][c["E"] - 1] == 0)


@pytest.mark.parametrize("cfg", ["tiny", "20b_decode"])
def test_backward_configs(cfg):
    print(f"backward parity {cfg}", flush=True)
    layer = synth.make_layer(cfg)
    c = layer.cfg
    dy = synth.bf16_from_f32(np.random.default_rng(c.seed + 7).standard_normal((c.T, c.H)).astype(np.float32))
    w = layer.weights
    ref = oracle.get().backward(layer.x, layer.w_router, w.gate_up, w.down, dy, c.k)
    got = _gpu_backward(layer.x, layer.w_router, w.gate_up, w.down, dy, c.k)
    _compare(got, ref, cfg)


def test_backward_no_tokens_zeroes_weight_gradients():
    d = moe.dims(0, 64, 4, 2, 96)
    dwr = torch.full((4, 64), 7.0, device="cuda")
    dgu = torch.full((4, 192, 64), 7.0, device="cuda")
    ddn = torch.full((4, 64, 96), 7.0, device="cuda")
    w = torch.zeros(4 * 192 * 64, dtype=torch.int16, device="cuda")
    moe.moe_backward(d, None, w, moe.expert_weights(w, w), None, None, dwr, dgu, ddn, None, 0)
    torch.cuda.synchronize()
    assert torch.all(dwr == 0) and torch.all(dgu == 0) and torch.all(ddn == 0)


@pytest.mark.slow
def test_backward_full_prefill_sparse_dy():
    layer = synth.make_layer("20b_prefill_zipf")
    c = layer.cfg
    print(f"backward full-size {c.name} T={c.T}", flush=True)
    rng = np.random.default_rng(c.seed + 8)
    tokens = np.sort(rng.choice(c.T, 16, replace=False))
    dy = np.zeros((c.T, c.H), np.uint16)
    dy[tokens] = synth.bf16_from_f32(rng.standard_normal((16, c.H)).astype(np.float32))
    w = layer.weights
    got = _gpu_backward(layer.x, layer.w_router, w.gate_up, w.down, dy, c.k)
    ref = oracle.get().backward(np.ascontiguousarray(layer.x[tokens]), layer.w_router, w.gate_up, w.down,
                                np.ascontiguousarray(dy[tokens]), c.k)
    others = np.setdiff1d(np.arange(c.T), tokens)
    assert np.all(got[0][others] == 0), "dx of a token with zero dy is not zero"
    _compare((got[0][tokens], *got[1:]), ref, "20b_prefill_zipf sparse dy")
