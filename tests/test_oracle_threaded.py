"""The threaded oracle harness (oracle/threaded.py, the benchmark's all-cores
CPU baseline) gives exactly the plain oracle's results: it only splits the
oracle's own calls over token and row ranges."""
import numpy as np
import pytest

from moe_glue_amd import inputs


@pytest.mark.parametrize("name,workers", [("tiny", 3), ("skewed", 4), ("skewed", 16)])
def test_threaded_path_equals_plain_path(oracle_lib, name, workers):
    from oracle import threaded

    cfg = inputs.CONFIGS[name]
    if name == "skewed":
        cfg = cfg.with_tokens(97)
    inp = inputs.make_inputs(cfg, 3)
    want = oracle_lib.path(inp)
    got = threaded.path(inp, workers, oracle_lib)
    for key in want:
        assert np.array_equal(got[key], want[key]), key
