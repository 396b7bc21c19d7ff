"""The CPU oracle run on several host threads, for the benchmark's all-cores
CPU baseline.

TEST INFRASTRUCTURE ONLY (like the rest of ``oracle``): only the benchmark's
``cpu_baseline`` leg and the test suite use it.  It adds no arithmetic of the
method: it calls the plain oracle functions of ``moe_oracle.c`` unchanged on
ranges of tokens or rows from a thread pool (ctypes releases the GIL during
each call), so the results are the oracle's own:

* route: one call on the whole batch (the histogram, scan and maps are
  global; the per-token top-k inside it is the same work either way);
* expand: token ranges (every destination row comes from ``dest_of_src``);
* SwiGLU: row ranges;
* combine: token ranges (``y`` whole, since any token may read any row).
"""
from __future__ import annotations

import ctypes
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import Oracle, _f32p, _i32p, _u16p, get


def _at(a: np.ndarray, offset_elems: int, t):
    return ctypes.cast(a.ctypes.data + offset_elems * a.itemsize, t)


def _ranges(n: int, parts: int):
    parts = max(1, min(parts, n)) if n > 0 else 1
    cuts = [n * i // parts for i in range(parts + 1)]
    return [(cuts[i], cuts[i + 1]) for i in range(parts) if cuts[i + 1] > cuts[i]]


def usable_cores() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        return os.cpu_count() or 1


def path(inp: dict, workers: int, o: Oracle | None = None) -> dict:
    """The whole path on one input dict from moe_glue_amd.inputs.make_inputs,
    split over `workers` threads; the same results as Oracle.path."""
    o = o or get()
    lib = o.lib
    cfg = inp["cfg"]
    T, H, k = cfg.T, cfg.H, cfg.k
    x = np.ascontiguousarray(inp["x"], dtype=np.uint16)
    h = np.ascontiguousarray(inp["h"], dtype=np.uint16)
    y = np.ascontiguousarray(inp["y"], dtype=np.uint16)
    R, I2 = h.shape
    I = I2 // 2
    r = o.route(inp["logits"], k, inp.get("bias"))
    dest = np.ascontiguousarray(r["dest_of_src"], dtype=np.int32)
    w = np.ascontiguousarray(r["topk_weights"], dtype=np.float32)
    x_exp = np.zeros((T * k, H), np.uint16)
    act = np.zeros((R, I), np.uint16)
    out = np.zeros((T, H), np.uint16)
    jobs = []
    for t0, t1 in _ranges(T, workers):
        jobs.append(lambda t0=t0, t1=t1: lib.moe_ref_expand_rows(_at(x, t0 * H, _u16p), _at(dest, t0 * k, _i32p),
                                                                 t1 - t0, H, k, _at(x_exp, 0, _u16p)))
    for r0, r1 in _ranges(R, workers):
        jobs.append(lambda r0=r0, r1=r1: lib.moe_ref_swiglu(_at(h, r0 * I2, _u16p), r1 - r0, I,
                                                            _at(act, r0 * I, _u16p)))
    for t0, t1 in _ranges(T, workers):
        jobs.append(lambda t0=t0, t1=t1: lib.moe_ref_combine(_at(y, 0, _u16p), _at(w, t0 * k, _f32p),
                                                             _at(dest, t0 * k, _i32p), t1 - t0, H, k,
                                                             _at(out, t0 * H, _u16p)))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        for f in [ex.submit(j) for j in jobs]:
            f.result()
    r["x_expanded"] = x_exp
    r["act"] = act
    r["out"] = out
    return r
