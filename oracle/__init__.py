"""CPU oracle for the MoE FFN layer (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its binding) never does; the two share no code.

The arithmetic lives in ``moe_oracle.c`` (plain C, IEEE double, loop order as
written); this module only compiles it with gcc and marshals numpy arrays
through ctypes.  Array conventions: bf16 tensors are ``numpy.uint16`` bit
patterns, MXFP4 tensors are ``numpy.uint8`` packed bytes plus ``numpy.uint8``
E8M0 scales, all C-contiguous.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")


def build(plant: int = 0, out: str | None = None) -> str:
    """Compile the oracle with gcc.  ``plant`` > 0 builds a variant with one
    planted mistake (used only by the oracle's own pin tests)."""
    out = out or LIB_PATH
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-shared", "-fPIC",
           "-std=c11", "-Wall", "-Wextra", "-Wno-unused-parameter", f"-DORC_PLANT={int(plant)}",
           _SRC, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64


def _bind(lib):
    lib.orc_bf16_value.restype = ctypes.c_double
    lib.orc_bf16_value.argtypes = [ctypes.c_uint16]
    lib.orc_e2m1_value.restype = ctypes.c_double
    lib.orc_e2m1_value.argtypes = [ctypes.c_uint]
    lib.orc_e8m0_value.restype = ctypes.c_double
    lib.orc_e8m0_value.argtypes = [ctypes.c_uint]
    lib.orc_mxfp4_value.restype = ctypes.c_double
    lib.orc_mxfp4_value.argtypes = [_P, _P, _I64]
    lib.orc_decode_expert_matrix.restype = _I
    lib.orc_decode_expert_matrix.argtypes = [_I, _P, _P, _I64, _I64, _I64, _P]
    lib.orc_route.restype = _I
    lib.orc_route.argtypes = [_I, _I, _I, _I, _P, _P, _P, _P, _P, _I]
    lib.orc_permute.restype = _I
    lib.orc_permute.argtypes = [_I, _I, _I, _P, _P, _P, _P]
    lib.orc_ffn_pairs.restype = _I
    lib.orc_ffn_pairs.argtypes = [_I, _I, _I, _I, _P, _P, _P, _P, _P, _I, _P, _P, _P, _P, _I]
    lib.orc_forward_tokens.restype = _I
    lib.orc_forward_tokens.argtypes = [_I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _I, _P, _P, _P, _P, _P, _P,
                                        _I]
    lib.orc_backward.restype = _I
    lib.orc_backward.argtypes = [_I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I]
    lib.orc_backward_f64.restype = _I
    lib.orc_backward_f64.argtypes = [_I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]
    lib.orc_mxfp4_quantize.restype = _I
    lib.orc_mxfp4_quantize.argtypes = [_I64, _I64, _P, _P, _P]
    lib.orc_mxfp4_fakequant.restype = _I
    lib.orc_mxfp4_fakequant.argtypes = [_I64, _I64, _P, _P]
    lib.orc_max_threads.restype = _I
    lib.orc_mxfp4_pack.argtypes = [_I, _I64, _I64, _I64, _P, _P, _P, _P]
    lib.orc_mxfp4_pack.restype = _I
    lib.orc_mxfp4_unpack.argtypes = [_I, _I64, _I64, _I64, _P, _P, _P, _P]
    lib.orc_mxfp4_unpack.restype = _I
    lib.orc_max_threads.argtypes = []
    return lib


class Oracle:
    """ctypes view of one build of the oracle library."""

    def __init__(self, path: str | None = None):
        path = path or LIB_PATH
        if not os.path.exists(path):
            build(out=path)
        self.path = path
        self.lib = _bind(ctypes.CDLL(path))

    # ------------------------------------------------------------ helpers
    @staticmethod
    def _ptr(a):
        if a is None:
            return None
        assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
        return a.ctypes.data

    def _check(self, rc, what):
        if rc != 0:
            raise RuntimeError(f"oracle {what} failed with code {rc}")

    # ------------------------------------------------------------ decode
    def bf16_value(self, bits: int) -> float:
        return self.lib.orc_bf16_value(int(bits))

    def e2m1_value(self, code: int) -> float:
        return self.lib.orc_e2m1_value(int(code))

    def e8m0_value(self, s: int) -> float:
        return self.lib.orc_e8m0_value(int(s))

    def decode_matrix(self, wfmt: int, data, scales, rows: int, cols: int, expert: int) -> np.ndarray:
        out = np.empty((rows, cols), np.float64)
        self._check(self.lib.orc_decode_expert_matrix(int(wfmt), self._ptr(data), self._ptr(scales), rows, cols,
                                                      expert, self._ptr(out)), "decode")
        return out

    # ------------------------------------------------------------ stages
    def route(self, x, w_router, k: int, threads: int = 0):
        """Returns (logits [T][E] f64, topk_idx [T][k] i32, topk_w [T][k] f64)."""
        T, H = x.shape
        E = w_router.shape[0]
        logits = np.empty((T, E), np.float64)
        idx = np.empty((T, k), np.int32)
        w = np.empty((T, k), np.float64)
        self._check(self.lib.orc_route(T, H, E, k, self._ptr(x), self._ptr(w_router), self._ptr(logits),
                                       self._ptr(idx), self._ptr(w), threads), "route")
        return logits, idx, w

    def permute(self, topk_idx, E: int):
        """Returns (expert_offsets [E+1], sorted_pairs [P], pair_rank [P]), all int32."""
        topk_idx = np.ascontiguousarray(topk_idx, np.int32)
        T, k = topk_idx.shape
        off = np.empty(E + 1, np.int32)
        sp = np.empty(T * k, np.int32)
        pr = np.empty(T * k, np.int32)
        self._check(self.lib.orc_permute(T, k, E, self._ptr(topk_idx), self._ptr(off), self._ptr(sp), self._ptr(pr)),
                    "permute")
        return off, sp, pr

    def ffn_pairs(self, x, weights, I: int, E: int, pair_token, pair_expert, want_h=False, threads: int = 0):
        """Expert outputs for (token, expert) pairs: returns o [n][H] (and h [n][I])."""
        T, H = x.shape
        pt = np.ascontiguousarray(pair_token, np.int32)
        pe = np.ascontiguousarray(pair_expert, np.int32)
        n = pt.shape[0]
        o = np.empty((n, H), np.float64)
        h = np.empty((n, I), np.float64) if want_h else None
        self._check(self.lib.orc_ffn_pairs(H, I, E, weights.wfmt, self._ptr(x), self._ptr(weights.gate_up),
                                           self._ptr(weights.gate_up_scale), self._ptr(weights.down),
                                           self._ptr(weights.down_scale), n, self._ptr(pt), self._ptr(pe),
                                           self._ptr(h), self._ptr(o), threads), "ffn_pairs")
        return (o, h) if want_h else o

    def forward_tokens(self, x, w_router, weights, k: int, I: int, tokens, threads: int = 0, want_pairs=False):
        """Layer output for the listed tokens: returns (y [n][H], idx [n][k], w [n][k]), and with
        want_pairs also the per-slot expert outputs o [n][k][H] and SwiGLU activations h [n][k][I]."""
        T, H = x.shape
        E = w_router.shape[0]
        tok = np.ascontiguousarray(tokens, np.int32)
        n = tok.shape[0]
        y = np.empty((n, H), np.float64)
        idx = np.empty((n, k), np.int32)
        w = np.empty((n, k), np.float64)
        o = np.empty((n, k, H), np.float64) if want_pairs else None
        h = np.empty((n, k, I), np.float64) if want_pairs else None
        self._check(self.lib.orc_forward_tokens(T, H, E, k, I, weights.wfmt, self._ptr(x), self._ptr(w_router),
                                                self._ptr(weights.gate_up), self._ptr(weights.gate_up_scale),
                                                self._ptr(weights.down), self._ptr(weights.down_scale), n,
                                                self._ptr(tok), self._ptr(y), self._ptr(idx), self._ptr(w),
                                                self._ptr(o), self._ptr(h), threads),
                    "forward_tokens")
        return (y, idx, w, o, h) if want_pairs else (y, idx, w)

    # ------------------------------------------------------------ backward
    def backward(self, x, w_router, gate_up, down, dy, k: int, threads: int = 0):
        """bf16 bits: x, dy [T][H], w_router [E][H], gate_up [E][2I][H], down [E][H][I].
        Returns (dx [T][H], dw_router [E][H], dgate_up [E][2I][H], ddown [E][H][I]) in float64."""
        T, H = x.shape
        E, twoI, _ = gate_up.shape
        I = twoI // 2
        out = (np.empty((T, H)), np.empty((E, H)), np.empty((E, 2 * I, H)), np.empty((E, H, I)))
        args = [np.ascontiguousarray(a, np.uint16) for a in (x, w_router, gate_up, down, dy)]
        self._check(self.lib.orc_backward(T, H, E, k, I, *[self._ptr(a) for a in args], *[self._ptr(o) for o in out],
                                          threads), "backward")
        return out

    def backward_f64(self, x, w_router, gate_up, down, dy, k: int):
        """Double inputs; returns (dx, dw_router, dgate_up, ddown, loss, topk_idx)."""
        T, H = x.shape
        E, twoI, _ = gate_up.shape
        I = twoI // 2
        out = (np.empty((T, H)), np.empty((E, H)), np.empty((E, 2 * I, H)), np.empty((E, H, I)))
        loss = np.zeros(1)
        idx = np.empty((T, k), np.int32)
        args = [np.ascontiguousarray(a, np.float64) for a in (x, w_router, gate_up, down, dy)]
        self._check(self.lib.orc_backward_f64(T, H, E, k, I, *[self._ptr(a) for a in args],
                                              *[self._ptr(o) for o in out], self._ptr(loss), self._ptr(idx)),
                    "backward_f64")
        return (*out, float(loss[0]), idx)

    # ------------------------------------------------------------ quantize
    def mxfp4_quantize(self, w):
        """bf16 bits [rows][cols] -> (packed u8 [rows][cols/2], scales u8 [rows][cols/32])."""
        w = np.ascontiguousarray(w, np.uint16)
        rows, cols = w.shape
        q = np.empty((rows, cols // 2), np.uint8)
        s = np.empty((rows, cols // 32), np.uint8)
        self._check(self.lib.orc_mxfp4_quantize(rows, cols, self._ptr(w), self._ptr(q), self._ptr(s)), "quantize")
        return q, s

    def mxfp4_fakequant(self, w):
        """bf16 bits [rows][cols] -> bf16 bits of decode(quantize(w))."""
        w = np.ascontiguousarray(w, np.uint16)
        rows, cols = w.shape
        out = np.empty((rows, cols), np.uint16)
        self._check(self.lib.orc_mxfp4_fakequant(rows, cols, self._ptr(w), self._ptr(out)), "fakequant")
        return out

    # ------------------------------------------------------------ packed order
    def _pack_io(self, gate_up: bool, E: int, I: int, H: int, w, s):
        R, K = (2 * I, H) if gate_up else (H, I)
        w = np.ascontiguousarray(w, np.uint8).reshape(E, R, K // 2)
        s = np.ascontiguousarray(s, np.uint8).reshape(E, R, K // 32)
        return w, s, np.empty_like(w), np.empty_like(s)

    def mxfp4_pack(self, gate_up: bool, E: int, I: int, H: int, w, s):
        """Row-major MXFP4 expert tensor (bytes, scales) -> the packed order."""
        w, s, wp, sp = self._pack_io(gate_up, E, I, H, w, s)
        self._check(self.lib.orc_mxfp4_pack(int(gate_up), E, I, H, self._ptr(w), self._ptr(s), self._ptr(wp),
                                            self._ptr(sp)), "mxfp4_pack")
        return wp, sp

    def mxfp4_unpack(self, gate_up: bool, E: int, I: int, H: int, wp, sp):
        """Packed MXFP4 expert tensor -> row-major (bytes, scales)."""
        wp, sp, w, s = self._pack_io(gate_up, E, I, H, wp, sp)
        self._check(self.lib.orc_mxfp4_unpack(int(gate_up), E, I, H, self._ptr(wp), self._ptr(sp), self._ptr(w),
                                              self._ptr(s)), "mxfp4_unpack")
        return w, s

    def max_threads(self) -> int:
        return self.lib.orc_max_threads()


_DEFAULT = None


def get() -> Oracle:
    """The default (mistake-free) oracle build, compiled on first use."""
    global _DEFAULT
    if _DEFAULT is None:
        _DEFAULT = Oracle()
    return _DEFAULT
