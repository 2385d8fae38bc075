"""A device-resident MoE layer: its inputs uploaded once, the buffers of every
stage allocated once, and one method per C-ABI entry point.

Argument marshalling only: torch allocates device memory and supplies the
stream; every step of the layer runs in libmoe.so's kernels.  Host inputs are
numpy arrays in the layouts of include/moe.h (bf16 as uint16 bit patterns,
MXFP4 as uint8 bytes and scales).
"""
from __future__ import annotations

import numpy as np
import torch

from . import (MOE_PATH_AUTO, MOE_WFMT_MXFP4, MOE_WFMT_MXFP4_PACKED, MOE_PACK_DOWN, MOE_PACK_GATE_UP, dims,
               expert_weights, moe_combine, moe_down, moe_forward, moe_gate_up, moe_grouped_ffn, moe_mxfp4_pack,
               moe_permute, moe_route, moe_workspace_size)


def to_dev(a: np.ndarray, device="cuda") -> torch.Tensor:
    """Host array -> device tensor with the same bytes (uint16 travels as int16)."""
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


class DeviceLayer:
    """Device copies of one layer (T tokens, hidden H, E experts, top-k, width
    I, weight format wfmt) plus the buffers of every stage."""

    def __init__(self, T: int, H: int, E: int, k: int, I: int, wfmt: int, x: np.ndarray, w_router: np.ndarray,
                 gate_up=None, down=None, gate_up_scale=None, down_scale=None, path: int = MOE_PATH_AUTO,
                 device="cuda", packed: bool = False, weights_dev=None):
        """gate_up .. down_scale: host weight arrays; or weights_dev: device
        tensors (gate_up, down, gate_up_scale, down_scale) already in the
        layer's format, row-major.  packed: MXFP4 weights are reordered on the
        device by moe_mxfp4_pack and the layer runs with MOE_WFMT_MXFP4_PACKED."""
        self.T, self.H, self.E, self.k, self.I = T, H, E, k, I
        self.device = device
        self.wfmt = wfmt
        self.x = to_dev(x, device)
        self.w_router = to_dev(w_router, device)
        if weights_dev is not None:
            self.gate_up, self.down, self.gate_up_scale, self.down_scale = weights_dev
        else:
            self.gate_up = to_dev(gate_up, device)
            self.down = to_dev(down, device)
            self.gate_up_scale = to_dev(gate_up_scale, device) if wfmt == MOE_WFMT_MXFP4 else None
            self.down_scale = to_dev(down_scale, device) if wfmt == MOE_WFMT_MXFP4 else None
        if packed:
            assert wfmt == MOE_WFMT_MXFP4, "only MXFP4 weights have a packed order"
            self.pack_weights()
        self.set_path(path)
        P = T * k
        i32 = dict(dtype=torch.int32, device=device)
        self.topk_idx = torch.empty((T, k), **i32)
        self.topk_w = torch.empty((T, k), dtype=torch.float32, device=device)
        self.offsets = torch.empty(E + 1, **i32)
        self.sorted_pairs = torch.empty(P, **i32)
        self.pair_rank = torch.empty(P, **i32)
        self.h = torch.empty((P, I), dtype=torch.int16, device=device)
        self.y_sorted = torch.empty((P, H), dtype=torch.int16, device=device)
        self.y = torch.empty((T, H), dtype=torch.int16, device=device)

    def pack_weights(self):
        """Reorder the device MXFP4 weights into the packed order (C ABI)."""
        d = dims(self.T, self.H, self.E, self.k, self.I, MOE_WFMT_MXFP4_PACKED)
        out = []
        for which, w, s in ((MOE_PACK_GATE_UP, self.gate_up, self.gate_up_scale),
                            (MOE_PACK_DOWN, self.down, self.down_scale)):
            wp, sp = torch.empty_like(w), torch.empty_like(s)
            moe_mxfp4_pack(d, which, w, s, wp, sp)
            out += [wp, sp]
        self.gate_up, self.gate_up_scale, self.down, self.down_scale = out
        self.wfmt = MOE_WFMT_MXFP4_PACKED

    def set_path(self, path: int):
        self.dims = dims(self.T, self.H, self.E, self.k, self.I, self.wfmt, path)
        self.ws_bytes = moe_workspace_size(self.dims)
        self.ws = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=self.device)
        self.weights = expert_weights(self.gate_up, self.down, self.gate_up_scale, self.down_scale)

    # ---- stages, each one C-ABI call
    def route(self):
        moe_route(self.dims, self.x, self.w_router, self.topk_idx, self.topk_w, self.ws, self.ws_bytes)

    def permute(self):
        moe_permute(self.dims, self.topk_idx, self.offsets, self.sorted_pairs, self.pair_rank, self.ws, self.ws_bytes)

    def gate_up_stage(self, weights=None):
        moe_gate_up(self.dims, self.x, self.offsets, self.sorted_pairs, weights or self.weights, self.h, self.ws,
                    self.ws_bytes)

    def down_stage(self, weights=None):
        moe_down(self.dims, self.h, self.offsets, weights or self.weights, self.y_sorted, self.ws, self.ws_bytes)

    def grouped_ffn(self):
        moe_grouped_ffn(self.dims, self.x, self.offsets, self.sorted_pairs, self.weights, self.y_sorted, self.ws,
                        self.ws_bytes)

    def combine(self):
        moe_combine(self.dims, self.y_sorted, self.pair_rank, self.topk_w, self.y)

    def stages(self):
        self.route()
        self.permute()
        self.gate_up_stage()
        self.down_stage()
        self.combine()

    def forward(self, want_routing=True, weights=None):
        moe_forward(self.dims, self.x, self.w_router, weights or self.weights, self.y,
                    self.topk_idx if want_routing else None, self.topk_w if want_routing else None, self.ws,
                    self.ws_bytes)
