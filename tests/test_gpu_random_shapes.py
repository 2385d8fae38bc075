"""Seeded sweep of random layer shapes against the oracle (forward on every
schedule, backward, and the quantiser), beyond the hand-picked edge cases.

Each case draws T in [1, 300], H and I as 32 x [1, 12] (so tiles of every
kernel have tails), E in [1, 40], k in [1, min(E, 8)], the weight format, the
schedule (AUTO / SKINNY / TILED) and uniform or Zipf(1.1) routing, from a
fixed seed; the parameters are printed before each case runs.  The MXFP4
cases run again with the weights in the packed order.  Same bar as
the parity tests: routing bit-exact, weights within 1e-5, outputs and
gradients within 1e-2 * max|ref|, quantiser bytes bit-exact.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mixture_experts_ffn_05_amd as moe
import oracle
import synth
from tests.gpu_layer import GpuLayer, bf16_dev_to_f64, rel_err, to_dev

pytestmark = pytest.mark.gpu

TOL = 1e-2
N_CASES = 24


def _cases():
    rng = np.random.default_rng(2026)
    out = []
    for i in range(N_CASES):
        E = int(rng.integers(1, 41))
        out.append(dict(T=int(rng.integers(1, 301)), H=32 * int(rng.integers(1, 13)), I=32 * int(rng.integers(1, 13)),
                        E=E, k=int(rng.integers(1, min(E, 8) + 1)), wfmt=int(rng.integers(0, 2)),
                        path=int(rng.integers(0, 3)), zipf=float(rng.choice([0.0, 1.1])), seed=100 + i))
    return out


CASES = _cases()


def _layer(c):
    cfg = synth.LayerConfig(f"rand_T{c['T']}_H{c['H']}_E{c['E']}_k{c['k']}_I{c['I']}", T=c["T"], H=c["H"], E=c["E"],
                            k=c["k"], I=c["I"], wfmt=c["wfmt"], seed=c["seed"], zipf_s=c["zipf"])
    return synth.make_layer(cfg)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_forward(i):
    c = CASES[i]
    print(f"[random forward] {c}", flush=True)
    layer = _layer(c)
    orc = oracle.get()
    y_ref, idx_ref, w_ref = orc.forward_tokens(layer.x, layer.w_router, layer.weights, c["k"], c["I"],
                                               np.arange(c["T"], dtype=np.int32))
    g = GpuLayer(layer, c["path"])
    g.forward()
    torch.cuda.synchronize()
    assert np.array_equal(g.topk_idx.cpu().numpy(), idx_ref)
    assert np.max(np.abs(g.topk_w.cpu().numpy() - w_ref)) <= 1e-5
    e = rel_err(bf16_dev_to_f64(g.y), y_ref)
    assert e <= TOL, e


@pytest.mark.parametrize("i", [i for i in range(N_CASES) if CASES[i]["wfmt"] == 1])
def test_random_forward_packed(i):
    """The MXFP4 cases again with the weights in the packed order."""
    c = CASES[i]
    print(f"[random forward packed] {c}", flush=True)
    layer = _layer(c)
    y_ref, idx_ref, _ = oracle.get().forward_tokens(layer.x, layer.w_router, layer.weights, c["k"], c["I"],
                                                    np.arange(c["T"], dtype=np.int32))
    g = GpuLayer(layer, c["path"], packed=True)
    g.forward()
    torch.cuda.synchronize()
    assert np.array_equal(g.topk_idx.cpu().numpy(), idx_ref)
    e = rel_err(bf16_dev_to_f64(g.y), y_ref)
    assert e <= TOL, e


@pytest.mark.parametrize("i", [i for i in range(N_CASES) if CASES[i]["wfmt"] == 0])
def test_random_backward(i):
    c = CASES[i]
    print(f"[random backward] {c}", flush=True)
    layer = _layer(c)
    T, H, E, k, I = c["T"], c["H"], c["E"], c["k"], c["I"]
    dy = synth.bf16_from_f32(np.random.default_rng(c["seed"] + 1).standard_normal((T, H)).astype(np.float32))
    w = layer.weights
    ref = oracle.get().backward(layer.x, layer.w_router, w.gate_up, w.down, dy, k)
    d = moe.dims(T, H, E, k, I)
    nbytes = moe.moe_backward_workspace_size(d)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda")
    dx = torch.empty((T, H), dtype=torch.int16, device="cuda")
    outs = [torch.empty(s, dtype=torch.float32, device="cuda") for s in ((E, H), (E, 2 * I, H), (E, H, I))]
    gu, dn = to_dev(w.gate_up), to_dev(w.down)
    moe.moe_backward(d, to_dev(layer.x), to_dev(layer.w_router), moe.expert_weights(gu, dn), to_dev(dy), dx, *outs,
                     ws, nbytes)
    torch.cuda.synchronize()
    got = [bf16_dev_to_f64(dx)] + [o.cpu().numpy() for o in outs]
    for name, a, r in zip(("dx", "dw_router", "dgate_up", "ddown"), got, ref):
        e = rel_err(np.asarray(a, np.float64), r)
        assert e <= TOL, f"{name}: {e:.3g}"


@pytest.mark.parametrize("i", range(8))
def test_random_quantize(i):
    rng = np.random.default_rng(300 + i)
    rows, cols = int(rng.integers(1, 200)), 32 * int(rng.integers(1, 100))
    print(f"[random quantize] rows={rows} cols={cols}", flush=True)
    w = synth.bf16_from_f32((rng.standard_normal((rows, cols)) * np.ldexp(1.0, rng.integers(-20, 10, (rows, cols))))
                            .astype(np.float32))
    dw = to_dev(w)
    packed = torch.empty((rows, cols // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((rows, cols // 32), dtype=torch.uint8, device="cuda")
    fq = torch.empty((rows, cols), dtype=torch.int16, device="cuda")
    moe.moe_mxfp4_quantize(rows, cols, dw, packed, scales)
    moe.moe_mxfp4_fakequant(rows, cols, dw, fq)
    torch.cuda.synchronize()
    o = oracle.get()
    rq, rs = o.mxfp4_quantize(w)
    assert np.array_equal(packed.cpu().numpy(), rq) and np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(fq.cpu().numpy().view(np.uint16), o.mxfp4_fakequant(w))
