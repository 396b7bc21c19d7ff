"""Comparators for HIP results against the oracle (host numpy arrays).

Tolerances:
* integer outputs (ids, counts, offsets, maps) and copies: bit-exact;
* bf16 activations and combined outputs: |got - ref| <= 1e-2*|ref| + 1e-3;
* fp32 routing weights: |got - ref| <= 1e-5*|ref| + 1e-6 and |sum_j w - 1| <= 1e-6.
"""
from __future__ import annotations

import numpy as np

BF16_RTOL, BF16_ATOL = 1e-2, 1e-3
W_RTOL, W_ATOL = 1e-5, 1e-6


def bf16_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits).view(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def bf16_mismatch(got_bits, ref_bits, rtol=BF16_RTOL, atol=BF16_ATOL):
    """Return (number of elements outside tolerance, worst excess, index of worst)."""
    g, r = bf16_to_f64(got_bits), bf16_to_f64(ref_bits)
    with np.errstate(invalid="ignore"):
        err = np.abs(g - r)
        lim = rtol * np.abs(r) + atol
        # a finite reference takes the tolerance; an infinite one must be matched exactly; NaN never agrees
        bad = ~np.where(np.isfinite(r), err <= lim, g == r)
    if not bad.any():
        return 0, 0.0, None
    with np.errstate(invalid="ignore"):
        excess = np.where(bad, np.nan_to_num(err - lim, nan=np.inf), 0.0)
    idx = np.unravel_index(int(np.argmax(excess)), excess.shape)
    return int(bad.sum()), float(excess[idx]), idx


def assert_bf16_close(got_bits, ref_bits, what: str):
    n, worst, idx = bf16_mismatch(got_bits, ref_bits)
    assert n == 0, (f"{what}: {n} elements outside |err| <= 1e-2|ref| + 1e-3; worst at {idx}: "
                    f"got {bf16_to_f64(got_bits)[idx]} ref {bf16_to_f64(ref_bits)[idx]}")


def assert_equal(got, ref, what: str):
    got, ref = np.asarray(got), np.asarray(ref)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} != {ref.shape}"
    if not np.array_equal(got, ref):
        bad = np.argwhere(got != ref)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} mismatches, first at {i}: got {got[i]} ref {ref[i]}")


def weights_mismatch(got, ref) -> int:
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    return int((~(np.abs(got - ref) <= W_RTOL * np.abs(ref) + W_ATOL)).sum())


def assert_weights_close(got, ref, what="topk_weights"):
    n = weights_mismatch(got, ref)
    assert n == 0, f"{what}: {n} weights outside 1e-5|ref| + 1e-6"
    s = np.asarray(got, np.float64).sum(axis=-1)
    if s.size:
        assert np.max(np.abs(s - 1.0)) <= 1e-6, f"{what}: row sums deviate from 1 by {np.max(np.abs(s - 1.0))}"


def assert_route_equal(got: dict, ref: dict, what: str = "route"):
    for key in ("topk_ids", "expert_offsets", "expert_counts", "dest_of_src", "src_of_dest"):
        assert_equal(got[key], ref[key], f"{what}.{key}")
    assert_weights_close(got["topk_weights"], ref["topk_weights"], f"{what}.topk_weights")
