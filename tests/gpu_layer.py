"""Upload a synthetic layer to the GPU and drive the library's C-ABI stages.

Used by the GPU parity tests, ``__graft_entry__.smoke()`` and ``bench.py``.
Every compute step is a call into libmoe.so through the binding; torch only
allocates device memory and supplies the stream.
"""
from __future__ import annotations

import numpy as np
import torch

import mixture_experts_ffn_05_amd as moe
import synth


def to_dev(a: np.ndarray, device="cuda") -> torch.Tensor:
    """Host array -> device tensor with the same bytes (uint16 travels as int16)."""
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


class GpuLayer:
    """Device copies of one synthetic layer plus the buffers of every stage."""

    def __init__(self, layer: synth.Layer, path: int = moe.MOE_PATH_AUTO, device="cuda", packed: bool = False,
                 weights_dev=None):
        """packed: MXFP4 weights are reordered on the device by moe_mxfp4_pack
        and the layer runs with MOE_WFMT_MXFP4_PACKED.  weights_dev: device
        tensors (gate_up, down, gate_up_scale, down_scale) to use instead of
        uploading layer.weights (in the layer's format, row-major)."""
        c = layer.cfg
        self.cfg = c
        self.layer = layer
        self.device = device
        self.wfmt = c.wfmt
        self.x = to_dev(layer.x, device)
        self.w_router = to_dev(layer.w_router, device)
        if weights_dev is not None:
            self.gate_up, self.down, self.gate_up_scale, self.down_scale = weights_dev
        else:
            w = layer.weights
            self.gate_up = to_dev(w.gate_up, device)
            self.down = to_dev(w.down, device)
            self.gate_up_scale = to_dev(w.gate_up_scale, device) if w.wfmt == 1 else None
            self.down_scale = to_dev(w.down_scale, device) if w.wfmt == 1 else None
        if packed:
            assert c.wfmt == 1, "only MXFP4 weights have a packed order"
            self.pack_weights()
        self.set_path(path)
        P = c.T * c.k
        i32 = dict(dtype=torch.int32, device=device)
        self.topk_idx = torch.empty((c.T, c.k), **i32)
        self.topk_w = torch.empty((c.T, c.k), dtype=torch.float32, device=device)
        self.offsets = torch.empty(c.E + 1, **i32)
        self.sorted_pairs = torch.empty(P, **i32)
        self.pair_rank = torch.empty(P, **i32)
        self.h = torch.empty((P, c.I), dtype=torch.int16, device=device)
        self.y_sorted = torch.empty((P, c.H), dtype=torch.int16, device=device)
        self.y = torch.empty((c.T, c.H), dtype=torch.int16, device=device)

    def pack_weights(self):
        """Reorder the device MXFP4 weights into the packed order (C ABI)."""
        c = self.cfg
        d = moe.dims(c.T, c.H, c.E, c.k, c.I, moe.MOE_WFMT_MXFP4_PACKED)
        out = []
        for which, w, s in ((moe.MOE_PACK_GATE_UP, self.gate_up, self.gate_up_scale),
                            (moe.MOE_PACK_DOWN, self.down, self.down_scale)):
            wp, sp = torch.empty_like(w), torch.empty_like(s)
            moe.moe_mxfp4_pack(d, which, w, s, wp, sp)
            out += [wp, sp]
        self.gate_up, self.gate_up_scale, self.down, self.down_scale = out
        self.wfmt = moe.MOE_WFMT_MXFP4_PACKED

    def set_path(self, path: int):
        c = self.cfg
        self.dims = moe.dims(c.T, c.H, c.E, c.k, c.I, self.wfmt, path)
        self.ws_bytes = moe.moe_workspace_size(self.dims)
        self.ws = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=self.device)
        self.weights = moe.expert_weights(self.gate_up, self.down, self.gate_up_scale, self.down_scale)

    # ---- stages, each one C-ABI call
    def route(self):
        moe.moe_route(self.dims, self.x, self.w_router, self.topk_idx, self.topk_w, self.ws, self.ws_bytes)

    def permute(self):
        moe.moe_permute(self.dims, self.topk_idx, self.offsets, self.sorted_pairs, self.pair_rank, self.ws,
                        self.ws_bytes)

    def gate_up_stage(self):
        moe.moe_gate_up(self.dims, self.x, self.offsets, self.sorted_pairs, self.weights, self.h, self.ws,
                        self.ws_bytes)

    def down_stage(self):
        moe.moe_down(self.dims, self.h, self.offsets, self.weights, self.y_sorted, self.ws, self.ws_bytes)

    def grouped_ffn(self):
        moe.moe_grouped_ffn(self.dims, self.x, self.offsets, self.sorted_pairs, self.weights, self.y_sorted, self.ws,
                            self.ws_bytes)

    def combine(self):
        moe.moe_combine(self.dims, self.y_sorted, self.pair_rank, self.topk_w, self.y)

    def stages(self):
        self.route()
        self.permute()
        self.gate_up_stage()
        self.down_stage()
        self.combine()

    def forward(self, want_routing=True):
        moe.moe_forward(self.dims, self.x, self.w_router, self.weights, self.y,
                        self.topk_idx if want_routing else None, self.topk_w if want_routing else None, self.ws,
                        self.ws_bytes)


def bf16_dev_to_f64(t: torch.Tensor) -> np.ndarray:
    """Device bf16 bit patterns -> float64 host array."""
    return synth.f32_from_bf16(t.cpu().numpy().view(np.uint16)).astype(np.float64)


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max|got - ref| / max|ref| (the parity metric)."""
    denom = float(np.max(np.abs(ref)))
    return float(np.max(np.abs(got - ref))) / (denom if denom > 0 else 1.0)
