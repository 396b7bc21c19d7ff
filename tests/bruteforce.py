"""Pure-Python brute force for tiny inputs, used to pin the oracle.

Nothing here shares code with the oracle or with the HIP path.  The algorithms
are deliberately different from the oracle's:

* top-k: k rounds of a linear argmax scan (the oracle sorts the whole row);
* destinations: counted directly, O(R^2) (the oracle keeps per-expert cursors);
* bf16 rounding: exact search in the table of all finite bf16 values (the
  oracle scales by a power of two and calls nearbyint);
* combine: exact rational arithmetic (fractions.Fraction) before one rounding.
"""
from __future__ import annotations

import bisect
import struct
from fractions import Fraction

import numpy as np


# ------------------------------------------------------------------ bf16 table
def _bf16_value(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (bits & 0xFFFF) << 16))[0]


# all finite non-negative bf16 values, ascending with the bit pattern
_POS_BITS = list(range(0x0000, 0x7F80))
_POS_VALS = [_bf16_value(b) for b in _POS_BITS]
_POS_VALS_NP = np.array(_POS_VALS, dtype=np.float64)
_OVERFLOW_STEP = 2.0 ** 128  # the (unrepresentable) next value above the largest finite bf16


def bf16_round_exact(v) -> int:
    """Nearest bf16 to v (a float or an exact Fraction), ties to the even bit
    pattern; returns raw bits.  No intermediate rounding happens."""
    if isinstance(v, Fraction):
        sign = 0x8000 if v < 0 else 0
        a = abs(v)
    else:
        if v != v:
            return 0x7FC0
        sign = 0x8000 if (v < 0 or (v == 0 and struct.pack("<d", v)[7] & 0x80)) else 0
        a = abs(v)
        if a == float("inf"):
            return sign | 0x7F80
    i = bisect.bisect_right(_POS_VALS, a) - 1
    lo_bits, lo = _POS_BITS[i], _POS_VALS[i]
    if lo == a:
        return sign | lo_bits
    if i + 1 < len(_POS_VALS):
        hi_bits, hi = _POS_BITS[i + 1], _POS_VALS[i + 1]
    else:
        hi_bits, hi = 0x7F80, _OVERFLOW_STEP
    d_lo = Fraction(a) - Fraction(lo)
    d_hi = Fraction(hi) - Fraction(a)
    if d_lo < d_hi:
        return sign | lo_bits
    if d_hi < d_lo:
        return sign | hi_bits
    return sign | (lo_bits if lo_bits % 2 == 0 else hi_bits)


def bf16_round_exact_np(v: np.ndarray) -> np.ndarray:
    """Vectorised bf16_round_exact for finite doubles (uses exact fp64 subtraction:
    the neighbours bracket |v| within a factor of two, so both distances are exact)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    i = np.searchsorted(_POS_VALS_NP, a, side="right") - 1
    lo = _POS_VALS_NP[i]
    hi = np.where(i + 1 < len(_POS_VALS_NP), _POS_VALS_NP[np.minimum(i + 1, len(_POS_VALS_NP) - 1)],
                  _OVERFLOW_STEP)
    lo_bits = i.astype(np.int64)
    hi_bits = np.where(i + 1 < len(_POS_VALS_NP), i + 1, 0x7F80).astype(np.int64)
    d_lo = a - lo
    d_hi = hi - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (lo_bits % 2 == 1))
    bits = np.where(pick_hi, hi_bits, lo_bits)
    sign = np.where(np.signbit(v), 0x8000, 0)
    return (bits | sign).astype(np.uint16)


def bf16_to_float(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


# ------------------------------------------------------------------ route
def fp32_key(logit: float, bias: float | None) -> float:
    if bias is None:
        return float(np.float32(logit))
    return float(np.float32(logit) + np.float32(bias))


def topk_argmax_rounds(keys: list[float], k: int) -> list[int]:
    """k rounds of: scan every expert not yet taken, keep the first strictly larger key."""
    taken = [False] * len(keys)
    picked = []
    for _ in range(k):
        best = -1
        for e, v in enumerate(keys):
            if taken[e]:
                continue
            if best < 0 or v > keys[best]:
                best = e
        taken[best] = True
        picked.append(best)
    return picked


def route_ids(logits: np.ndarray, k: int, bias: np.ndarray | None = None) -> np.ndarray:
    T, E = logits.shape
    out = np.zeros((T, k), np.int32)
    for t in range(T):
        keys = [fp32_key(logits[t, e], None if bias is None else bias[e]) for e in range(E)]
        out[t] = topk_argmax_rounds(keys, k)
    return out


def counts_offsets_dest(ids: np.ndarray, E: int):
    """Counts, exclusive offsets and stable destinations by direct counting."""
    flat = [int(v) for v in np.asarray(ids).reshape(-1)]
    R = len(flat)
    counts = [sum(1 for v in flat if v == e) for e in range(E)]
    offsets = [sum(counts[:e]) for e in range(E + 1)]
    dest = []
    for s in range(R):
        e = flat[s]
        earlier_same = sum(1 for s2 in range(s) if flat[s2] == e)
        dest.append(offsets[e] + earlier_same)
    return np.array(counts, np.int32), np.array(offsets, np.int32), np.array(dest, np.int32)


# ------------------------------------------------------------------ combine
def combine_exact(y: np.ndarray, w: np.ndarray, dest: np.ndarray):
    """Exact rational sum_j w*y, then one rounding.  Returns (bits, exact sums)."""
    T, k = w.shape
    H = y.shape[1]
    yv = bf16_to_float(y)
    out = np.zeros((T, H), np.uint16)
    exact = [[None] * H for _ in range(T)]
    for t in range(T):
        for c in range(H):
            s = Fraction(0)
            for j in range(k):
                s += Fraction(float(w[t, j])) * Fraction(float(yv[dest[t * k + j], c]))
            exact[t][c] = s
            out[t, c] = bf16_round_exact(s)
    return out, exact


def padded_layout(ids: np.ndarray, E: int, pad_to: int):
    """Build the padded expert-contiguous layout constructively: for each
    expert in turn append its slots in ascending order, then append padding
    (-1) until the segment length is a multiple of pad_to.  Returns
    (offsets, dest_of_src, src_of_dest)."""
    flat = [int(v) for v in np.asarray(ids).reshape(-1)]
    layout = []
    offsets = [0]
    for e in range(E):
        seg = [s for s in range(len(flat)) if flat[s] == e]
        while len(seg) % pad_to != 0:
            seg.append(-1)
        layout.extend(seg)
        offsets.append(len(layout))
    dest = [0] * len(flat)
    for p, s in enumerate(layout):
        if s >= 0:
            dest[s] = p
    return np.array(offsets, np.int32), np.array(dest, np.int32), np.array(layout, np.int32)
