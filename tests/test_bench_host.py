"""Host-side logic of bench.py (no GPU): the input-set rotation and the
algorithmic byte counts it reports."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from moe_glue_amd import inputs  # noqa: E402


def test_rotation_keeps_x_out_of_the_infinity_cache():
    for name in inputs.CONFIG_ORDER:
        cfg = inputs.CONFIGS[name]
        n = bench.default_sets(cfg)
        assert 4 <= n <= bench.MAX_SETS
        assert n * bench.set_bytes(cfg) <= bench.MAX_SET_BYTES or n == 4
        x_total = n * cfg.T * cfg.H * 2
        # either the copies of x exceed the cache twice over, or a cap decided
        assert x_total >= 2 * bench.INFINITY_CACHE_BYTES or n == bench.MAX_SETS, name


def test_rotation_at_the_benchmark_shapes():
    c = inputs.CONFIGS
    assert bench.default_sets(c["qwen3_30b_a3b"]) == 32      # 32 x 16 MiB of x
    assert bench.default_sets(c["deepseek_v3"]) == 5         # 5 x 112 MiB
    assert bench.default_sets(c["decode"]) == bench.MAX_SETS


def test_set_bytes_covers_every_tensor_of_a_set():
    for name in inputs.CONFIG_ORDER:
        cfg = inputs.CONFIGS[name]
        T, H, E, k, I, R = cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.R
        tensors = (T * H * 2 + T * E * 4 + R * 2 * I * 2 + R * H * 2  # x, logits, h, y
                   + R * 4 * 4                                      # ids, weights, two maps
                   + R * H * 2 + R * I * 2 + T * H * 2)             # x_exp, act, out
        assert bench.set_bytes(cfg) >= tensors, name
        assert bench.set_bytes(cfg, pad_to=128) > bench.set_bytes(cfg), name


def test_algorithmic_bytes_at_the_qwen_shape():
    ab = bench.algorithmic_bytes(inputs.CONFIGS["qwen3_30b_a3b"])
    assert ab["expand"] == 151126016
    assert ab["swiglu"] == 150994944
    assert ab["combine"] == 151257088
    assert ab["route_expand"] == ab["route"] + ab["expand"]


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err
