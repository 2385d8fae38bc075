"""Packed MXFP4 order on the GPU: moe_mxfp4_pack against the oracle's pack,
byte for byte (a permutation of bytes: bit equality is the bar), and the
layer's prefill (tiled) schedule giving the same bits on packed and on
row-major weights (it decodes the same values in the same order).  Layer
parity of the packed format against the oracle is in test_gpu_parity.py,
test_gpu_edges.py and test_gpu_random_shapes.py.

Inputs: random bytes for the codes and scale bytes (every byte value), at
K-block counts 1, 3, 16, 17 and 90 (below, at and across one 16-block chunk),
several experts, both tensor kinds, and the full 20b tensors."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mixture_experts_ffn_05_amd as moe
import oracle
import synth
from tests.gpu_layer import GpuLayer, to_dev

pytestmark = pytest.mark.gpu


def _pack_gpu(gate_up: bool, E: int, I: int, H: int, w: np.ndarray, s: np.ndarray):
    d = moe.dims(1, H, E, 1, I, moe.MOE_WFMT_MXFP4_PACKED)
    dw, ds = to_dev(w), to_dev(s)
    wp, sp = torch.empty_like(dw), torch.empty_like(ds)
    moe.moe_mxfp4_pack(d, moe.MOE_PACK_GATE_UP if gate_up else moe.MOE_PACK_DOWN, dw, ds, wp, sp)
    torch.cuda.synchronize()
    return wp.cpu().numpy(), sp.cpu().numpy()


def _check(gate_up, E, I, H, seed):
    R, K = (2 * I, H) if gate_up else (H, I)
    print(f"pack parity gate_up={gate_up} E={E} I={I} H={H} (K-blocks {K // 32})", flush=True)
    rng = np.random.default_rng(seed)
    w = rng.integers(0, 256, (E, R, K // 2), dtype=np.uint8)
    s = rng.integers(0, 256, (E, R, K // 32), dtype=np.uint8)
    gw, gs = _pack_gpu(gate_up, E, I, H, w, s)
    rw, rs = oracle.get().mxfp4_pack(gate_up, E, I, H, w, s)
    bad = np.argwhere(gw.reshape(-1) != rw.reshape(-1))
    assert bad.size == 0, f"{bad.size} packed bytes differ, first at {bad[0]}"
    assert np.array_equal(gs.reshape(-1), rs.reshape(-1)), "packed scales differ"


@pytest.mark.parametrize("gate_up,E,I,H", [(True, 3, 32, 32), (True, 2, 64, 96), (False, 2, 512, 64),
                                           (False, 3, 544, 32), (True, 4, 96, 2880), (False, 2, 2880, 96)],
                         ids=["gu_kb1", "gu_kb3", "dn_kb16", "dn_kb17", "gu_kb90", "dn_kb90"])
def test_pack_matches_oracle(gate_up, E, I, H):
    _check(gate_up, E, I, H, seed=E * 1000 + I + H)


@pytest.mark.slow
@pytest.mark.parametrize("gate_up", [True, False], ids=["gate_up", "down"])
def test_pack_full_20b(gate_up):
    _check(gate_up, 32, 2880, 2880, seed=20)


def test_tiled_packed_equals_row_major_bitwise():
    """20b MXFP4 shape at 1024 tokens on the tiled schedule."""
    print("tiled packed vs row-major, 20b MXFP4, T=1024", flush=True)
    layer = synth.make_layer("20b_mxfp4_decode", T=1024)
    ys = []
    for packed in (False, True):
        g = GpuLayer(layer, moe.MOE_PATH_TILED, packed=packed)
        g.forward()
        torch.cuda.synchronize()
        ys.append(g.y.clone())
        del g
    assert torch.equal(ys[0], ys[1])
