"""Synthetic layers on the GPU for the parity tests and the smoke check.

``GpuLayer`` is the package's DeviceLayer built from a ``synth.Layer``; every
compute step is a call into libmoe.so through the binding.
"""
from __future__ import annotations

import numpy as np
import torch

import mixture_experts_ffn_05_amd as moe
import synth
from mixture_experts_ffn_05_amd.layer import DeviceLayer, to_dev  # noqa: F401  (to_dev re-exported)


class GpuLayer(DeviceLayer):
    """Device copies of one synthetic layer plus the buffers of every stage."""

    def __init__(self, layer: synth.Layer, path: int = moe.MOE_PATH_AUTO, device="cuda", packed: bool = False,
                 weights_dev=None):
        c = layer.cfg
        self.cfg = c
        self.layer = layer
        w = layer.weights
        host = {} if weights_dev is not None else dict(gate_up=w.gate_up, down=w.down, gate_up_scale=w.gate_up_scale,
                                                       down_scale=w.down_scale)
        super().__init__(c.T, c.H, c.E, c.k, c.I, c.wfmt, layer.x, layer.w_router, path=path, device=device,
                         packed=packed, weights_dev=weights_dev, **host)


def bf16_dev_to_f64(t: torch.Tensor) -> np.ndarray:
    """Device bf16 bit patterns -> float64 host array."""
    return synth.f32_from_bf16(t.cpu().numpy().view(np.uint16)).astype(np.float64)


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max|got - ref| / max|ref| (the parity metric)."""
    denom = float(np.max(np.abs(ref)))
    return float(np.max(np.abs(got - ref))) / (denom if denom > 0 else 1.0)
