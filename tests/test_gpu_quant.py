"""HIP MXFP4 quantiser and fake quantiser against the oracle, byte for byte.

Both decide integers (codes, scale bytes) from exact arithmetic, so the bar is
bit equality of packed bytes, scale bytes and fake-quantised bf16 bits.

Inputs (seeded): per 32-element block one of
  - N(0, 0.02) weights (the experts' generator distribution),
  - N(0, 1) times 2^U(-30, 30) per element (dynamic range inside a block),
  - E2M1 midpoints times 2^X with the block's amax pinned to 4 or 6 times 2^X
    (every element an exact tie; X across the whole scale range),
  - zeros and negative zeros,
  - bf16 subnormals and the smallest normals (scale byte clamped to 0),
  - random finite bf16 bit patterns;
at a size below one workgroup, at several workgroups with a ragged tail, on
every finite bf16 pattern, and on the 20b gate/up tensor ([32*5760][2880],
1.06 GB) in the launch the benchmark times, checked on 512 seeded rows and by
properties of the whole tensor.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

import mixture_experts_ffn_05_amd as moe
import oracle
import synth
from tests.gpu_layer import to_dev

pytestmark = pytest.mark.gpu

_MID = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])


def _edge_matrix(seed: int, rows: int, cols: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    nb = rows * cols // 32
    kinds = rng.integers(0, 6, size=nb)
    out = np.empty((nb, 32), np.uint16)
    for b, kind in enumerate(kinds):
        if kind == 0:
            v = synth.bf16_from_f32((rng.standard_normal(32) * 0.02).astype(np.float32))
        elif kind == 1:
            v = synth.bf16_from_f32((rng.standard_normal(32) * np.ldexp(1.0, rng.integers(-30, 30, 32)))
                                    .astype(np.float32))
        elif kind == 2:
            X = int(rng.integers(-127, 124))
            m = rng.choice(_MID, 32) * rng.choice([-1.0, 1.0], 32)
            m[rng.integers(32)] = rng.choice([4.0, 6.0, -4.0, -6.0])
            f = (m * np.ldexp(1.0, X)).astype(np.float32)
            v = (f.view(np.uint32) >> 16).astype(np.uint16)  # exact: at most 3 significant bits
        elif kind == 3:
            v = rng.choice(np.array([0x0000, 0x8000], np.uint16), 32)
        elif kind == 4:
            v = (rng.integers(0, 0x180, 32) | (rng.integers(0, 2, 32) << 15)).astype(np.uint16)
        else:
            v = rng.integers(0, 0x10000, 32).astype(np.uint16)
            bad = ((v >> 7) & 0xFF) == 0xFF  # Inf / NaN: undefined codes
            v[bad] &= 0x807F
        out[b] = v
    return out.reshape(rows, cols)


def _gpu(w: np.ndarray):
    rows, cols = w.shape
    dw = to_dev(w)
    packed = torch.empty((rows, cols // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((rows, cols // 32), dtype=torch.uint8, device="cuda")
    fq = torch.empty((rows, cols), dtype=torch.int16, device="cuda")
    moe.moe_mxfp4_quantize(rows, cols, dw, packed, scales)
    moe.moe_mxfp4_fakequant(rows, cols, dw, fq)
    torch.cuda.synchronize()
    return packed.cpu().numpy(), scales.cpu().numpy(), fq.cpu().numpy().view(np.uint16)


def _check(w: np.ndarray):
    o = oracle.get()
    q, s, fq = _gpu(w)
    rq, rs = o.mxfp4_quantize(w)
    rfq = o.mxfp4_fakequant(w)
    bad_s = np.argwhere(s != rs)
    assert bad_s.size == 0, f"{len(bad_s)} scale bytes differ, first at {bad_s[0]}"
    bad_q = np.argwhere(q != rq)
    assert bad_q.size == 0, f"{len(bad_q)} packed bytes differ, first at {bad_q[0]}: got {q[tuple(bad_q[0])]:02x} " \
                            f"want {rq[tuple(bad_q[0])]:02x}"
    bad_f = np.argwhere(fq != rfq)
    assert bad_f.size == 0, f"{len(bad_f)} fake-quant values differ, first at {bad_f[0]}"


@pytest.mark.parametrize("rows,cols,seed", [(3, 96, 1), (37, 2880, 2), (64, 4096, 3)],
                         ids=["sub_workgroup", "ragged_2880", "aligned_4096"])
def test_quantize_matches_oracle(rows, cols, seed):
    print(f"quantize parity rows={rows} cols={cols} seed={seed}", flush=True)
    _check(_edge_matrix(seed, rows, cols))


def test_every_finite_bf16_pattern():
    """Each finite bf16 pattern once, in random blocks, so every input value
    meets many scale bytes across the tensor."""
    print("quantize parity: all finite bf16 patterns", flush=True)
    rng = np.random.default_rng(4)
    pats = np.arange(0x10000, dtype=np.uint32)
    pats = pats[((pats >> 7) & 0xFF) != 0xFF].astype(np.uint16)
    pats = rng.permutation(pats)
    pats = pats[: (pats.size // 32) * 32]
    _check(pats.reshape(-1, 1024) if pats.size % 1024 == 0 else pats.reshape(1, -1))


def test_empty_tensor_is_a_no_op():
    dw = torch.zeros(64, dtype=torch.int16, device="cuda")
    moe.moe_mxfp4_quantize(0, 64, dw, dw, dw)
    moe.moe_mxfp4_fakequant(2, 0, dw, dw)
    torch.cuda.synchronize()


@pytest.mark.slow
def test_full_20b_gate_up_tensor():
    """[32*5760][2880] bf16 N(0, 0.02), drawn on the device from a seeded
    generator: 512 seeded rows against the oracle; over the whole tensor, the
    fake-quantised tensor equals the quantised one decoded (E2M1 table times
    2^(S-127) in torch), fake quantisation is idempotent, and re-quantising
    it gives the same bytes."""
    rows, cols = 32 * 5760, 2880
    print(f"quantize full size rows={rows} cols={cols}", flush=True)
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    w = (torch.randn((rows, cols), generator=g, device="cuda") * 0.02).to(torch.bfloat16).view(torch.int16)
    packed = torch.empty((rows, cols // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((rows, cols // 32), dtype=torch.uint8, device="cuda")
    fq = torch.empty_like(w)
    moe.moe_mxfp4_quantize(rows, cols, w, packed, scales)
    moe.moe_mxfp4_fakequant(rows, cols, w, fq)
    torch.cuda.synchronize()

    sel = np.sort(np.random.default_rng(6).choice(rows, 512, replace=False))
    idx = torch.from_numpy(sel).cuda()
    ws = w.index_select(0, idx).cpu().numpy().view(np.uint16)
    o = oracle.get()
    rq, rs = o.mxfp4_quantize(ws)
    assert np.array_equal(packed.index_select(0, idx).cpu().numpy(), rq)
    assert np.array_equal(scales.index_select(0, idx).cpu().numpy(), rs)
    assert np.array_equal(fq.index_select(0, idx).cpu().numpy().view(np.uint16), o.mxfp4_fakequant(ws))

    table = torch.tensor([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0],
                         device="cuda")
    for r0 in range(0, rows, 16384):  # decode in row chunks
        p = packed[r0:r0 + 16384]
        codes = torch.stack([p & 15, p >> 4], dim=-1).reshape(p.shape[0], cols).long()
        unit = torch.ldexp(torch.ones((), device="cuda"), scales[r0:r0 + 16384].int() - 127)
        dec = (table[codes] * unit.repeat_interleave(32, dim=1)).to(torch.bfloat16).view(torch.int16)
        assert torch.equal(dec, fq[r0:r0 + 16384]), f"decode(quantize) != fake-quant in rows {r0}.."
    fq2 = torch.empty_like(fq)
    moe.moe_mxfp4_fakequant(rows, cols, fq, fq2)
    packed2 = torch.empty_like(packed)
    scales2 = torch.empty_like(scales)
    moe.moe_mxfp4_quantize(rows, cols, fq, packed2, scales2)
    torch.cuda.synchronize()
    assert torch.equal(fq2, fq)
    assert torch.equal(packed2, packed) and torch.equal(scales2, scales)


@pytest.mark.parametrize("name", ["tiny", "20b_decode"])
def test_fake_quant_forward(name):
    """The forward of training through quantisation: bf16 expert weights
    fake-quantised on the GPU, then the bf16 layer; and the MXFP4 layer on the
    GPU-quantised bytes.  Both compute the oracle's MXFP4 layer on the
    oracle-quantised weights (the two forms are the same reals, a pin of the
    oracle), within the layer tolerance."""
    from tests.gpu_layer import GpuLayer, bf16_dev_to_f64, rel_err
    print(f"fake-quant forward {name}", flush=True)
    layer = synth.make_layer(name)
    c = layer.cfg
    gu = layer.weights.gate_up.reshape(c.E * 2 * c.I, c.H)
    dn = layer.weights.down.reshape(c.E * c.H, c.I)
    o = oracle.get()
    qgu, sgu = o.mxfp4_quantize(gu)
    qdn, sdn = o.mxfp4_quantize(dn)
    wq = synth.Weights(1, qgu.reshape(c.E, 2 * c.I, c.H // 2), qdn.reshape(c.E, c.H, c.I // 2),
                       sgu.reshape(c.E, 2 * c.I, c.H // 32), sdn.reshape(c.E, c.H, c.I // 32))
    tokens = synth.sample_tokens(c.T, 512, c.seed + 1)
    ref = o.forward_tokens(layer.x, layer.w_router, wq, c.k, c.I, tokens)[0]

    # bf16 layer on fake-quantised weights
    g = GpuLayer(layer)
    fgu = torch.empty_like(g.gate_up)
    fdn = torch.empty_like(g.down)
    moe.moe_mxfp4_fakequant(gu.shape[0], c.H, g.gate_up, fgu)
    moe.moe_mxfp4_fakequant(dn.shape[0], c.I, g.down, fdn)
    g.gate_up, g.down = fgu, fdn
    g.set_path(moe.MOE_PATH_AUTO)
    g.forward()
    torch.cuda.synchronize()
    err = rel_err(bf16_dev_to_f64(g.y)[tokens], ref)
    assert err <= 1e-2, f"fake-quant bf16 layer: max err {err:.3g} of max|ref|"

    # MXFP4 layer on GPU-quantised bytes
    cq = dataclasses.replace(c, wfmt=1)
    lq = synth.Layer(cq, layer.x, layer.w_router, wq)
    g4 = GpuLayer(lq)
    # quantise the bf16 weights on the GPU into the MXFP4 layer's buffers
    # (gate/up from the original weights; down from its fake-quantised copy,
    # whose re-quantisation gives the same bytes)
    moe.moe_mxfp4_quantize(gu.shape[0], c.H, to_dev(gu), g4.gate_up, g4.gate_up_scale)
    moe.moe_mxfp4_quantize(dn.shape[0], c.I, fdn, g4.down, g4.down_scale)
    g4.forward()
    torch.cuda.synchronize()
    assert np.array_equal(g4.gate_up.cpu().numpy(), wq.gate_up) and np.array_equal(g4.down.cpu().numpy(), wq.down)
    err4 = rel_err(bf16_dev_to_f64(g4.y)[tokens], ref)
    assert err4 <= 1e-2, f"MXFP4 layer on GPU-quantised weights: max err {err4:.3g} of max|ref|"
