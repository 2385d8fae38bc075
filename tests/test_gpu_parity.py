"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Bar (stated for the layer): routing indices and the permutation bit-exact on
every token; routing weights within 1e-5; h, y_sorted and y within
max|gpu - ref| <= 1e-2 * max|ref| (fp32 accumulation, bf16 storage).  Configs
with more than 512 tokens are checked on a seeded sample of 512 tokens (each
token's output depends on that token alone); routing and permutation are
still checked on all tokens.  Both expert-FFN schedules (skinny and tiled)
are forced on every config, and for MXFP4 weights both tiled kernels (MX
matrix cores, and bf16 decode); the MXFP4 configs also run with the weights
in the packed order.
"""
from __future__ import annotations

import functools

import numpy as np
import pytest
import torch

import mixture_experts_ffn_05_amd as moe
import oracle
import synth
from tests.gpu_layer import GpuLayer, bf16_dev_to_f64, rel_err, to_dev

pytestmark = pytest.mark.gpu

TOL = 1e-2
W_TOL = 1e-5
CHECK_TOKENS = 512

# "+packed": the same MXFP4 layer with its weights reordered on the device by
# moe_mxfp4_pack (MOE_WFMT_MXFP4_PACKED), against the oracle on the row-major
# weights; "@1": one token (single-stream decode, few touched experts);
# "120b_mxfp4_T<t>": the 120b shape with MXFP4 experts, as the decode sweep
# times it (packed order).
CASES = ["tiny", "20b_decode"] + [f"120b_T{t}" for t in synth.SWEEP_120B] + [
    "20b_prefill_zipf", "20b_mxfp4_decode", "20b_mxfp4_prefill", "20b_mxfp4_decode+packed",
    "20b_mxfp4_prefill+packed", "20b_mxfp4_decode@1+packed"] + [
    f"120b_mxfp4_T{t}+packed" for t in synth.SWEEP_120B]


@functools.lru_cache(maxsize=1)
def _weights(cfg_name: str):
    return synth.make_weights(synth.CONFIGS[cfg_name])


def make_case(name: str) -> synth.Layer:
    name = name.split("+")[0]
    if "@" in name:  # "<config>@T": the config's layer at T tokens
        base, T = name.split("@")
        cfg = synth.CONFIGS[base].with_T(int(T))
        return synth.Layer(cfg, synth.make_x(cfg), synth.make_router(cfg),
                           _weights("20b_mxfp4_decode" if cfg.wfmt == 1 else base))
    if name.startswith("120b_T"):
        cfg = synth.CONFIGS["120b_sweep"].with_T(int(name[len("120b_T"):]))
        wkey = "120b_sweep"
    elif name.startswith("120b_mxfp4_T"):
        cfg = synth.CONFIGS["120b_mxfp4_sweep"].with_T(int(name[len("120b_mxfp4_T"):]))
        wkey = "120b_mxfp4_sweep"
    else:
        cfg = synth.CONFIGS[name]
        wkey = "20b_mxfp4_decode" if cfg.wfmt == 1 else name
    if cfg.wfmt == 0 and not name.startswith("120b"):
        return synth.make_layer(cfg)
    return synth.Layer(cfg, synth.make_x(cfg), synth.make_router(cfg), _weights(wkey))


class Case:
    """One config: inputs, the oracle's answers, and the device copies."""

    def __init__(self, name):
        print(f"[case] {name}", flush=True)
        self.name = name
        self.layer = make_case(name)
        c = self.cfg = self.layer.cfg
        orc = oracle.get()
        _, self.idx, self.w = orc.route(self.layer.x, self.layer.w_router, c.k)
        self.off, self.sp, self.pr = orc.permute(self.idx, c.E)
        self.tokens = synth.sample_tokens(c.T, CHECK_TOKENS, c.seed + 1)
        self.y, _, _, self.o, self.h = orc.forward_tokens(self.layer.x, self.layer.w_router, self.layer.weights, c.k,
                                                          c.I, self.tokens, want_pairs=True)
        self.gpu = GpuLayer(self.layer, packed=name.endswith("+packed"))
        # pair ids of the checked tokens, in (token, slot) order
        self.pairs = (self.tokens[:, None] * c.k + np.arange(c.k)[None, :]).ravel()


@pytest.fixture(scope="module", params=CASES)
def case(request):
    c = Case(request.param)
    yield c
    del c.gpu
    torch.cuda.empty_cache()


def _load_oracle_routing(case):
    g = case.gpu
    g.topk_idx.copy_(torch.from_numpy(case.idx))
    g.topk_w.copy_(torch.from_numpy(case.w.astype(np.float32)))
    g.offsets.copy_(torch.from_numpy(case.off))
    g.sorted_pairs.copy_(torch.from_numpy(case.sp))
    g.pair_rank.copy_(torch.from_numpy(case.pr))


def test_route(case):
    g = case.gpu
    g.route()
    torch.cuda.synchronize()
    idx = g.topk_idx.cpu().numpy()
    mism = np.nonzero((idx != case.idx).any(1))[0]
    assert mism.size == 0, f"{mism.size} tokens routed differently, first {mism[:5]}"
    werr = float(np.max(np.abs(g.topk_w.cpu().numpy().astype(np.float64) - case.w)))
    assert werr <= W_TOL, werr


def test_permute(case):
    g = case.gpu
    g.topk_idx.copy_(torch.from_numpy(case.idx))
    g.permute()
    torch.cuda.synchronize()
    assert np.array_equal(g.offsets.cpu().numpy(), case.off)
    assert np.array_equal(g.sorted_pairs.cpu().numpy(), case.sp)
    assert np.array_equal(g.pair_rank.cpu().numpy(), case.pr)


# For MXFP4 weights TILED_MX runs the MX-core kernel (so does TILED, where the
# MX kernel applies) and TILED_DEQUANT the bf16-decode one; for bf16 weights
# TILED is the only tiled kernel.
STAGE_PATHS = [moe.MOE_PATH_SKINNY, moe.MOE_PATH_TILED, moe.MOE_PATH_TILED_DEQUANT, moe.MOE_PATH_TILED_MX]
STAGE_IDS = ["skinny", "tiled", "tiled_dequant", "tiled_mx"]


def _skip_duplicate(case, path):
    if case.cfg.wfmt == 0 and path in (moe.MOE_PATH_TILED_DEQUANT, moe.MOE_PATH_TILED_MX):
        pytest.skip("bf16 weights: one tiled kernel (TILED)")
    if case.cfg.wfmt != 0 and path == moe.MOE_PATH_TILED:
        pytest.skip("MXFP4 weights: TILED runs the TILED_MX kernel")


@pytest.mark.parametrize("path", STAGE_PATHS, ids=STAGE_IDS)
def test_expert_stages(case, path):
    """gate/up+SwiGLU -> h, down -> y_sorted, combine -> y, each against the oracle."""
    _skip_duplicate(case, path)
    g = case.gpu
    c = case.cfg
    g.set_path(path)
    _load_oracle_routing(case)
    g.gate_up_stage()
    g.down_stage()
    g.combine()
    torch.cuda.synchronize()
    rows = torch.from_numpy(case.pr[case.pairs].astype(np.int64)).to(g.device)
    h = bf16_dev_to_f64(g.h.index_select(0, rows))
    e_h = rel_err(h, case.h.reshape(-1, c.I))
    ys = bf16_dev_to_f64(g.y_sorted.index_select(0, rows))
    e_o = rel_err(ys, case.o.reshape(-1, c.H))
    y = bf16_dev_to_f64(g.y.index_select(0, torch.from_numpy(case.tokens.astype(np.int64)).to(g.device)))
    e_y = rel_err(y, case.y)
    print(f"[{case.name} path={path}] rel err h {e_h:.2e} y_sorted {e_o:.2e} y {e_y:.2e}")
    assert e_h <= TOL and e_o <= TOL and e_y <= TOL, (e_h, e_o, e_y)


@pytest.mark.parametrize("path", [moe.MOE_PATH_AUTO] + STAGE_PATHS, ids=["auto"] + STAGE_IDS)
def test_forward(case, path):
    _skip_duplicate(case, path)
    g = case.gpu
    g.set_path(path)
    g.y.fill_(0)
    g.forward()
    torch.cuda.synchronize()
    assert np.array_equal(g.topk_idx.cpu().numpy(), case.idx)
    y = bf16_dev_to_f64(g.y.index_select(0, torch.from_numpy(case.tokens.astype(np.int64)).to(g.device)))
    e_y = rel_err(y, case.y)
    print(f"[{case.name} forward path={path}] rel err y {e_y:.2e}")
    assert e_y <= TOL, e_y


def test_forward_deterministic(case):
    g = case.gpu
    g.set_path(moe.MOE_PATH_AUTO)
    g.forward()
    y1 = g.y.clone()
    g.y.fill_(0)
    g.forward()
    torch.cuda.synchronize()
    assert torch.equal(y1, g.y)
