"""Expert weights in pinned host memory, for the host-streamed decode path.

The pages describe serving engines that keep expert weights in pinned host
memory and stream them to the GPU, which pays off only for models larger
than the GPU's memory ("gpt-oss-20b" model page, section "llama-swap.yaml
entry": the 12 GB model fits one 16 GB card, so keeping every expert
resident is faster than streaming them from pinned host banks).  The library
takes plain pointers, so its skinny kernels read such weights directly: only
the touched experts' rows cross the host link, each once per layer.

Here: torch's pinned allocation (hipHostMalloc) for the bytes, and the device
address of that mapping from hipHostGetDevicePointer (the documented
zero-copy route).  Pass ``PinnedArray.dev`` wherever the C ABI takes an
expert-weight pointer (moe_expert_weights); keep the PinnedArray alive until
the stream has run the work.  This module only allocates and maps memory; it
runs none of the layer.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np


def _hip():
    import torch
    lib = ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
    lib.hipHostGetDevicePointer.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p, ctypes.c_uint]
    lib.hipHostGetDevicePointer.restype = ctypes.c_int
    return lib


class PinnedArray:
    """A host array copied into pinned memory; .dev is its device address
    (None when the runtime does not map pinned memory for the device)."""

    def __init__(self, a: np.ndarray):
        import torch
        a = np.ascontiguousarray(a)
        self.host = torch.empty(a.nbytes, dtype=torch.uint8, pin_memory=True)
        self.host.numpy()[:] = a.view(np.uint8).reshape(-1)
        dev = ctypes.c_void_p(0)
        rc = _hip().hipHostGetDevicePointer(ctypes.byref(dev), ctypes.c_void_p(self.host.data_ptr()), 0)
        self.dev = dev.value if rc == 0 and dev.value else None


def pinned_weights(gate_up: np.ndarray, down: np.ndarray, gate_up_scale: np.ndarray | None = None,
                   down_scale: np.ndarray | None = None):
    """[gate_up, down] (+ [gate_up_scale, down_scale] for MXFP4) copied into
    pinned host memory, in the layouts of include/moe.h; None if any of them
    cannot be mapped for the device."""
    arrays = [gate_up, down] + ([gate_up_scale, down_scale] if gate_up_scale is not None else [])
    parts = [PinnedArray(a) for a in arrays]
    if any(p.dev is None for p in parts):
        return None
    return parts
