"""CPU oracle for the MoE glue path (numpy front end over the plain-C library).

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and
the benchmark's ``cpu_baseline`` leg may import this package.  It shares no code
with ``moe_glue_amd`` (the HIP path) and neither imports the other; the seeded
input generator is the only thing both sides consume.

All arrays are host numpy arrays; bf16 tensors are ``uint16`` arrays of raw
bits.  Shapes follow the C header ``oracle/moe_oracle.h``.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_i32p = ctypes.POINTER(ctypes.c_int32)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)


def _ptr(a: np.ndarray, t):
    return a.ctypes.data_as(t)


class Oracle:
    """ctypes binding of one build of the oracle library (the real one or a test mutant)."""

    def __init__(self, lib_path: str | None = None):
        if lib_path is None:
            if _build.is_stale():
                _build.build()
            lib_path = _build.LIB
        self.lib_file = lib_path
        lib = ctypes.CDLL(os.path.abspath(lib_path))
        lib.moe_ref_route.restype = ctypes.c_int
        lib.moe_ref_route.argtypes = [_f32p, _f32p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      _i32p, _f32p, _i32p, _i32p, _i32p, _i32p]
        lib.moe_ref_route_padded.restype = ctypes.c_int
        lib.moe_ref_route_padded.argtypes = [_f32p, _f32p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                             _i32p, _f32p, _i32p, _i32p, _i32p, _i32p]
        lib.moe_ref_expand_rows.restype = None
        lib.moe_ref_expand_rows.argtypes = [_u16p, _i32p, ctypes.c_int, ctypes.c_int, ctypes.c_int, _u16p]
        lib.moe_ref_expand_rows_fp8.restype = None
        lib.moe_ref_expand_rows_fp8.argtypes = [_u16p, _i32p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                ctypes.c_int, ctypes.POINTER(ctypes.c_uint8), _f32p]
        lib.moe_ref_expand_rows_mxfp8.restype = None
        lib.moe_ref_expand_rows_mxfp8.argtypes = [_u16p, _i32p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                  ctypes.POINTER(ctypes.c_uint8), ctypes.POINTER(ctypes.c_uint8)]
        lib.moe_ref_e4m3_from_f32.restype = ctypes.c_uint8
        lib.moe_ref_e4m3_from_f32.argtypes = [ctypes.c_float]
        lib.moe_ref_f64_from_e4m3.restype = ctypes.c_double
        lib.moe_ref_f64_from_e4m3.argtypes = [ctypes.c_uint8]
        lib.moe_ref_swiglu.restype = None
        lib.moe_ref_swiglu.argtypes = [_u16p, ctypes.c_int, ctypes.c_int, _u16p]
        lib.moe_ref_combine.restype = None
        lib.moe_ref_combine.argtypes = [_u16p, _f32p, _i32p, ctypes.c_int, ctypes.c_int, ctypes.c_int, _u16p]
        lib.moe_ref_bf16_from_f64.restype = ctypes.c_uint16
        lib.moe_ref_bf16_from_f64.argtypes = [ctypes.c_double]
        lib.moe_ref_f64_from_bf16.restype = ctypes.c_double
        lib.moe_ref_f64_from_bf16.argtypes = [ctypes.c_uint16]
        lib.moe_ref_bf16_from_f64_n.restype = None
        lib.moe_ref_bf16_from_f64_n.argtypes = [_f64p, ctypes.c_int64, _u16p]
        self.lib = lib

    # ------------------------------------------------------------ the four steps
    def route(self, logits: np.ndarray, k: int, bias: np.ndarray | None = None) -> dict:
        logits = np.ascontiguousarray(logits, dtype=np.float32)
        T, E = logits.shape
        R = T * k
        ids = np.zeros((T, k), np.int32)
        w = np.zeros((T, k), np.float32)
        offsets = np.zeros(E + 1, np.int32)
        counts = np.zeros(E, np.int32)
        dest = np.zeros(R, np.int32)
        src = np.zeros(R, np.int32)
        b = None
        if bias is not None:
            bias = np.ascontiguousarray(bias, dtype=np.float32)
            assert bias.shape == (E,)
            b = _ptr(bias, _f32p)
        rc = self.lib.moe_ref_route(_ptr(logits, _f32p), b, T, E, k, _ptr(ids, _i32p), _ptr(w, _f32p),
                                    _ptr(offsets, _i32p), _ptr(counts, _i32p), _ptr(dest, _i32p),
                                    _ptr(src, _i32p))
        if rc != 0:
            raise ValueError(f"moe_ref_route rejected T={T} E={E} k={k} (rc={rc})")
        return {"topk_ids": ids, "topk_weights": w, "expert_offsets": offsets, "expert_counts": counts,
                "dest_of_src": dest, "src_of_dest": src}

    def route_padded(self, logits: np.ndarray, k: int, pad_to: int, bias: np.ndarray | None = None) -> dict:
        """Route with each expert's segment padded to a multiple of pad_to rows;
        src_of_dest has expert_offsets[E] entries, -1 on padding rows."""
        logits = np.ascontiguousarray(logits, dtype=np.float32)
        T, E = logits.shape
        R = T * k
        bound = R + E * (pad_to - 1)
        ids = np.zeros((T, k), np.int32)
        w = np.zeros((T, k), np.float32)
        offsets = np.zeros(E + 1, np.int32)
        counts = np.zeros(E, np.int32)
        dest = np.zeros(R, np.int32)
        src = np.full(max(bound, 1), -7, np.int32)
        b = None
        if bias is not None:
            bias = np.ascontiguousarray(bias, dtype=np.float32)
            b = _ptr(bias, _f32p)
        rc = self.lib.moe_ref_route_padded(_ptr(logits, _f32p), b, T, E, k, pad_to, _ptr(ids, _i32p),
                                           _ptr(w, _f32p), _ptr(offsets, _i32p), _ptr(counts, _i32p),
                                           _ptr(dest, _i32p), _ptr(src, _i32p))
        if rc != 0:
            raise ValueError(f"moe_ref_route_padded rejected T={T} E={E} k={k} pad_to={pad_to} (rc={rc})")
        return {"topk_ids": ids, "topk_weights": w, "expert_offsets": offsets, "expert_counts": counts,
                "dest_of_src": dest, "src_of_dest": src[:offsets[E]]}

    def expand_rows(self, x: np.ndarray, dest_of_src: np.ndarray, k: int, rows: int | None = None) -> np.ndarray:
        """rows: height of the expanded buffer (T*k, or the padded total)."""
        x = np.ascontiguousarray(x, dtype=np.uint16)
        dest_of_src = np.ascontiguousarray(dest_of_src, dtype=np.int32).reshape(-1)
        T, H = x.shape
        assert dest_of_src.size == T * k
        out = np.zeros((T * k if rows is None else rows, H), np.uint16)
        self.lib.moe_ref_expand_rows(_ptr(x, _u16p), _ptr(dest_of_src, _i32p), T, H, k, _ptr(out, _u16p))
        return out

    def expand_rows_fp8(self, x: np.ndarray, dest_of_src: np.ndarray, k: int, group: int,
                        rows: int | None = None):
        """FP8 quantising expand; returns (codes uint8 [rows, H], scales fp32 [rows, H/group])."""
        x = np.ascontiguousarray(x, dtype=np.uint16)
        dest_of_src = np.ascontiguousarray(dest_of_src, dtype=np.int32).reshape(-1)
        T, H = x.shape
        assert dest_of_src.size == T * k and H % group == 0
        n = T * k if rows is None else rows
        q = np.zeros((n, H), np.uint8)
        sc = np.zeros((n, H // group), np.float32)
        self.lib.moe_ref_expand_rows_fp8(_ptr(x, _u16p), _ptr(dest_of_src, _i32p), T, H, k, group,
                                         q.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)), _ptr(sc, _f32p))
        return q, sc

    def expand_rows_mxfp8(self, x: np.ndarray, dest_of_src: np.ndarray, k: int, rows: int | None = None):
        """MXFP8 quantising expand; returns (codes uint8 [rows, H], E8M0 scale bytes uint8 [rows, H/32])."""
        x = np.ascontiguousarray(x, dtype=np.uint16)
        dest_of_src = np.ascontiguousarray(dest_of_src, dtype=np.int32).reshape(-1)
        T, H = x.shape
        assert dest_of_src.size == T * k and H % 32 == 0
        n = T * k if rows is None else rows
        q = np.zeros((n, H), np.uint8)
        sc = np.zeros((n, H // 32), np.uint8)
        u8p = ctypes.POINTER(ctypes.c_uint8)
        self.lib.moe_ref_expand_rows_mxfp8(_ptr(x, _u16p), _ptr(dest_of_src, _i32p), T, H, k,
                                           q.ctypes.data_as(u8p), sc.ctypes.data_as(u8p))
        return q, sc

    def e4m3_from_f32(self, v: np.ndarray) -> np.ndarray:
        return np.array([self.lib.moe_ref_e4m3_from_f32(float(a)) for a in np.asarray(v, np.float32).reshape(-1)],
                        np.uint8)

    def swiglu(self, h: np.ndarray) -> np.ndarray:
        h = np.ascontiguousarray(h, dtype=np.uint16)
        R, I2 = h.shape
        assert I2 % 2 == 0
        out = np.zeros((R, I2 // 2), np.uint16)
        self.lib.moe_ref_swiglu(_ptr(h, _u16p), R, I2 // 2, _ptr(out, _u16p))
        return out

    def combine(self, y: np.ndarray, topk_weights: np.ndarray, dest_of_src: np.ndarray) -> np.ndarray:
        y = np.ascontiguousarray(y, dtype=np.uint16)
        w = np.ascontiguousarray(topk_weights, dtype=np.float32)
        T, k = w.shape
        dest_of_src = np.ascontiguousarray(dest_of_src, dtype=np.int32).reshape(-1)
        R, H = y.shape
        assert R >= T * k and dest_of_src.size == T * k
        out = np.zeros((T, H), np.uint16)
        self.lib.moe_ref_combine(_ptr(y, _u16p), _ptr(w, _f32p), _ptr(dest_of_src, _i32p), T, H, k,
                                 _ptr(out, _u16p))
        return out

    # ------------------------------------------------------------------ helpers
    def bf16_from_f64(self, v: np.ndarray) -> np.ndarray:
        v = np.ascontiguousarray(v, dtype=np.float64)
        out = np.zeros(v.shape, np.uint16)
        self.lib.moe_ref_bf16_from_f64_n(_ptr(v, _f64p), v.size, _ptr(out, _u16p))
        return out

    def path(self, inp: dict) -> dict:
        """Run the whole path on one input dict from moe_glue_amd.inputs.make_inputs."""
        cfg = inp["cfg"]
        r = self.route(inp["logits"], cfg.k, inp.get("bias"))
        r["x_expanded"] = self.expand_rows(inp["x"], r["dest_of_src"], cfg.k)
        r["act"] = self.swiglu(inp["h"])
        r["out"] = self.combine(inp["y"], r["topk_weights"], r["dest_of_src"])
        return r


_default: Oracle | None = None


def get() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default
