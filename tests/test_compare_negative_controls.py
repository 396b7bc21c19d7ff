"""Negative controls: a mistake planted in the oracle's expected values (on the
CPU) must make the comparators fail.  A tolerance that lets these through
would pass whatever the kernels compute."""
import numpy as np
import pytest

import compare
from moe_glue_amd import inputs as I


@pytest.fixture(scope="module")
def tiny(oracle_lib):
    cfg = I.CONFIGS["tiny"]
    inp = I.make_inputs(cfg, 0)
    return inp, oracle_lib.path(inp)


def test_identical_results_pass(tiny):
    _, ref = tiny
    compare.assert_route_equal(ref, ref)
    compare.assert_bf16_close(ref["act"], ref["act"], "act")
    compare.assert_bf16_close(ref["out"], ref["out"], "out")


def _bump_ulps(bits, idx, n):
    b = bits.copy()
    b[idx] = np.uint16(int(b[idx]) + n)
    return b


@pytest.mark.parametrize("key", ["act", "out"])
def test_four_ulp_error_is_caught(tiny, key):
    _, ref = tiny
    vals = compare.bf16_to_f64(ref[key])
    idx = np.unravel_index(int(np.argmax(np.abs(vals))), vals.shape)  # a large value: 4 ulps = 2-3%
    planted = _bump_ulps(ref[key], idx, 4)
    with pytest.raises(AssertionError):
        compare.assert_bf16_close(planted, ref[key], key)


def test_one_ulp_error_is_within_tolerance(tiny):
    _, ref = tiny
    planted = _bump_ulps(ref["act"], (0, 0), 1)
    compare.assert_bf16_close(planted, ref["act"], "act")


@pytest.mark.parametrize("key", ["topk_ids", "dest_of_src", "src_of_dest", "expert_offsets", "expert_counts"])
def test_swapped_index_is_caught(tiny, key):
    _, ref = tiny
    bad = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in ref.items()}
    flat = bad[key].reshape(-1)
    flat[0], flat[-1] = flat[-1], flat[0] + (1 if flat[0] == flat[-1] else 0)
    with pytest.raises(AssertionError):
        compare.assert_route_equal(bad, ref)


def test_weight_error_is_caught(tiny):
    _, ref = tiny
    bad = dict(ref)
    w = ref["topk_weights"].copy()
    w[3, 0] *= 1.0 + 5e-5
    bad["topk_weights"] = w
    with pytest.raises(AssertionError):
        compare.assert_route_equal(bad, ref)


def test_copy_error_is_caught(tiny):
    _, ref = tiny
    planted = _bump_ulps(ref["x_expanded"], (5, 7), 1)
    with pytest.raises(AssertionError):
        compare.assert_equal(planted, ref["x_expanded"], "x_expanded")


def test_equal_infinities_agree_but_nan_and_sign_do_not():
    inf, ninf, nan = np.uint16(0x7F80), np.uint16(0xFF80), np.uint16(0x7FC0)
    compare.assert_bf16_close(np.array([inf, ninf]), np.array([inf, ninf]), "inf")
    for got, ref in ((ninf, inf), (nan, nan), (np.uint16(0x3F80), inf)):
        with pytest.raises(AssertionError):
            compare.assert_bf16_close(np.array([got]), np.array([ref]), "special")
