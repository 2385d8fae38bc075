"""Python binding of libmoe.so, the MI355X MoE FFN layer library.

Argument marshalling only: every function below packs its arguments and calls
the C entry point of the same name (declared in include/moe.h); all of the
layer's work runs in the library's HIP kernels.  PyTorch supplies device
memory and the stream.  Tensors are passed by ``data_ptr()``; bf16 tensors may
be torch.bfloat16 or raw uint16/int16 bit patterns, MXFP4 tensors uint8.

If the library is not built the import still succeeds, but every call raises
``MoeLibraryMissing`` (there is no fallback path).
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_MISALIGNED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(6)
MOE_WFMT_BF16, MOE_WFMT_MXFP4, MOE_WFMT_MXFP4_PACKED = 0, 1, 2
MOE_PACK_GATE_UP, MOE_PACK_DOWN = 0, 1
MOE_PATH_AUTO, MOE_PATH_SKINNY, MOE_PATH_TILED, MOE_PATH_TILED_DEQUANT, MOE_PATH_TILED_MX = 0, 1, 2, 3, 4

EXPORTED = ("moe_workspace_size", "moe_route", "moe_permute", "moe_gate_up", "moe_down", "moe_grouped_ffn",
            "moe_combine", "moe_forward", "moe_forward_noalloc", "moe_backward_workspace_size", "moe_backward",
            "moe_mxfp4_quantize", "moe_mxfp4_fakequant", "moe_mxfp4_pack", "moe_mx_split", "moe_strerror",
            "moe_last_error")


class MoeLibraryMissing(RuntimeError):
    pass


class MoeError(RuntimeError):
    def __init__(self, fn: str, code: int, text: str):
        super().__init__(f"{fn} failed: {text} (code {code})")
        self.code = code


class moe_dims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("E", ctypes.c_int32), ("k", ctypes.c_int32),
                ("I", ctypes.c_int32), ("wfmt", ctypes.c_int32), ("path", ctypes.c_int32)]


class moe_expert_weights(ctypes.Structure):
    _fields_ = [("gate_up", ctypes.c_void_p), ("gate_up_scale", ctypes.c_void_p), ("down", ctypes.c_void_p),
                ("down_scale", ctypes.c_void_p)]


_lib = None


def library(path: str | None = None):
    """Load libmoe.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    # torch ships its own libamdhip64 (same soname): load it first so the
    # process holds a single HIP runtime and torch's streams are valid here.
    import torch  # noqa: F401
    if not os.path.exists(p):
        raise MoeLibraryMissing(f"{p} is not built; run `python -m mixture_experts_ffn_05_amd.build`")
    lib = ctypes.CDLL(p)
    V, I32, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    D, W = ctypes.POINTER(moe_dims), ctypes.POINTER(moe_expert_weights)
    sig = {
        "moe_workspace_size": [D, ctypes.POINTER(SZ)],
        "moe_route": [D, V, V, V, V, V, SZ, V],
        "moe_permute": [D, V, V, V, V, V, SZ, V],
        "moe_gate_up": [D, V, V, V, W, V, V, SZ, V],
        "moe_down": [D, V, V, W, V, V, SZ, V],
        "moe_grouped_ffn": [D, V, V, V, W, V, V, SZ, V],
        "moe_combine": [D, V, V, V, V, V],
        "moe_forward": [D, V, V, W, V, V, V, V, SZ, V],
        "moe_forward_noalloc": [D, V, V, W, V, V, V, V],
        "moe_backward_workspace_size": [D, ctypes.POINTER(SZ)],
        "moe_backward": [D, V, V, W, V, V, V, V, V, V, SZ, V],
        "moe_mxfp4_quantize": [ctypes.c_int64, ctypes.c_int32, V, V, V, V],
        "moe_mxfp4_fakequant": [ctypes.c_int64, ctypes.c_int32, V, V, V],
        "moe_mxfp4_pack": [D, ctypes.c_int32, V, V, V, V, V],
        "moe_mx_split": [ctypes.c_int64, ctypes.c_int32, V, V, V, V],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = I32
    lib.moe_strerror.argtypes = [I32]
    lib.moe_strerror.restype = ctypes.c_char_p
    lib.moe_last_error.argtypes = []
    lib.moe_last_error.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn: str, rc: int):
    if rc != MOE_OK:
        lib = library()
        text = lib.moe_strerror(rc).decode()
        if rc == MOE_ERR_HIP:
            text += ": " + lib.moe_last_error().decode()
        raise MoeError(fn, rc, text)


def dims(T: int, H: int, E: int, k: int, I: int, wfmt: int = MOE_WFMT_BF16, path: int = MOE_PATH_AUTO) -> moe_dims:
    return moe_dims(T, H, E, k, I, wfmt, path)


def expert_weights(gate_up, down, gate_up_scale=None, down_scale=None) -> moe_expert_weights:
    return moe_expert_weights(_ptr(gate_up), _ptr(gate_up_scale), _ptr(down), _ptr(down_scale))


def strerror(code: int) -> str:
    return library().moe_strerror(code).decode()


def moe_workspace_size(d: moe_dims) -> int:
    n = ctypes.c_size_t(0)
    _check("moe_workspace_size", library().moe_workspace_size(ctypes.byref(d), ctypes.byref(n)))
    return n.value


def moe_route(d, x, w_router, topk_idx, topk_w, ws, ws_bytes, stream=None):
    _check("moe_route", library().moe_route(ctypes.byref(d), _ptr(x), _ptr(w_router), _ptr(topk_idx), _ptr(topk_w),
                                           _ptr(ws), ws_bytes, _stream(stream)))


def moe_permute(d, topk_idx, expert_offsets, sorted_pairs, pair_rank, ws, ws_bytes, stream=None):
    _check("moe_permute", library().moe_permute(ctypes.byref(d), _ptr(topk_idx), _ptr(expert_offsets),
                                               _ptr(sorted_pairs), _ptr(pair_rank), _ptr(ws), ws_bytes,
                                               _stream(stream)))


def moe_gate_up(d, x, expert_offsets, sorted_pairs, weights: moe_expert_weights, h, ws, ws_bytes, stream=None):
    _check("moe_gate_up", library().moe_gate_up(ctypes.byref(d), _ptr(x), _ptr(expert_offsets), _ptr(sorted_pairs),
                                               ctypes.byref(weights), _ptr(h), _ptr(ws), ws_bytes, _stream(stream)))


def moe_down(d, h, expert_offsets, weights: moe_expert_weights, y_sorted, ws, ws_bytes, stream=None):
    _check("moe_down", library().moe_down(ctypes.byref(d), _ptr(h), _ptr(expert_offsets), ctypes.byref(weights),
                                         _ptr(y_sorted), _ptr(ws), ws_bytes, _stream(stream)))


def moe_grouped_ffn(d, x, expert_offsets, sorted_pairs, weights: moe_expert_weights, y_sorted, ws, ws_bytes,
                    stream=None):
    _check("moe_grouped_ffn", library().moe_grouped_ffn(ctypes.byref(d), _ptr(x), _ptr(expert_offsets),
                                                       _ptr(sorted_pairs), ctypes.byref(weights), _ptr(y_sorted),
                                                       _ptr(ws), ws_bytes, _stream(stream)))


def moe_combine(d, y_sorted, pair_rank, topk_w, y, stream=None):
    _check("moe_combine", library().moe_combine(ctypes.byref(d), _ptr(y_sorted), _ptr(pair_rank), _ptr(topk_w),
                                               _ptr(y), _stream(stream)))


def moe_forward(d, x, w_router, weights: moe_expert_weights, y, topk_idx_out, topk_w_out, ws, ws_bytes, stream=None):
    _check("moe_forward", library().moe_forward(ctypes.byref(d), _ptr(x), _ptr(w_router), ctypes.byref(weights),
                                               _ptr(y), _ptr(topk_idx_out), _ptr(topk_w_out), _ptr(ws), ws_bytes,
                                               _stream(stream)))


def moe_forward_noalloc(d, x, w_router, weights: moe_expert_weights, y, topk_idx_out, topk_w_out, stream=None):
    _check("moe_forward_noalloc", library().moe_forward_noalloc(ctypes.byref(d), _ptr(x), _ptr(w_router),
                                                               ctypes.byref(weights), _ptr(y), _ptr(topk_idx_out),
                                                               _ptr(topk_w_out), _stream(stream)))


MOE_NOALLOC_SCRATCH_BYTES = 32 << 20


def moe_backward_workspace_size(d: moe_dims) -> int:
    n = ctypes.c_size_t(0)
    _check("moe_backward_workspace_size", library().moe_backward_workspace_size(ctypes.byref(d), ctypes.byref(n)))
    return n.value


def moe_backward(d, x, w_router, weights: moe_expert_weights, dy, dx, dw_router, dgate_up, ddown, ws, ws_bytes,
                 stream=None):
    _check("moe_backward", library().moe_backward(ctypes.byref(d), _ptr(x), _ptr(w_router), ctypes.byref(weights),
                                                 _ptr(dy), _ptr(dx), _ptr(dw_router), _ptr(dgate_up), _ptr(ddown),
                                                 _ptr(ws), ws_bytes, _stream(stream)))


def moe_mxfp4_quantize(rows: int, cols: int, w, packed, scales, stream=None):
    _check("moe_mxfp4_quantize", library().moe_mxfp4_quantize(rows, cols, _ptr(w), _ptr(packed), _ptr(scales),
                                                             _stream(stream)))


def moe_mxfp4_fakequant(rows: int, cols: int, w, out, stream=None):
    _check("moe_mxfp4_fakequant", library().moe_mxfp4_fakequant(rows, cols, _ptr(w), _ptr(out), _stream(stream)))


def moe_mxfp4_pack(d: moe_dims, which: int, w, scales, w_packed, scales_packed, stream=None):
    _check("moe_mxfp4_pack", library().moe_mxfp4_pack(ctypes.byref(d), which, _ptr(w), _ptr(scales), _ptr(w_packed),
                                                     _ptr(scales_packed), _stream(stream)))


def moe_mx_split(rows: int, cols: int, x, codes, scales, stream=None):
    _check("moe_mx_split", library().moe_mx_split(rows, cols, _ptr(x), _ptr(codes), _ptr(scales), _stream(stream)))


__all__ = ["library", "dims", "expert_weights", "strerror", "moe_workspace_size", "moe_route", "moe_permute",
           "moe_gate_up", "moe_down", "moe_grouped_ffn", "moe_combine", "moe_forward", "moe_forward_noalloc",
           "MOE_NOALLOC_SCRATCH_BYTES", "moe_backward_workspace_size",
           "moe_backward", "moe_mxfp4_quantize",
           "moe_mxfp4_fakequant", "moe_mxfp4_pack", "moe_mx_split", "moe_dims",
           "moe_expert_weights", "MoeError", "MoeLibraryMissing", "EXPORTED", "LIB_PATH"]
