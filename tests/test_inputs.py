"""Seeded synthetic input generator: determinism, shapes, distributions."""
import numpy as np

from moe_glue_amd import inputs as I


def test_same_seed_same_tensors():
    cfg = I.CONFIGS["tiny"]
    a, b = I.make_inputs(cfg, 3), I.make_inputs(cfg, 3)
    for key in ("x", "logits", "h", "y"):
        assert np.array_equal(a[key], b[key])
    c = I.make_inputs(cfg, 4)
    assert not np.array_equal(a["x"], c["x"])


def test_partial_draws_match_full_draws():
    cfg = I.CONFIGS["decode"]
    full = I.make_inputs(cfg, 1)
    only_y = I.make_inputs(cfg, 1, parts=("y",))
    assert np.array_equal(full["y"], only_y["y"])


def test_shapes_and_dtypes():
    for name in I.CONFIG_ORDER:
        cfg = I.CONFIGS[name]
        if cfg.T * cfg.H > 5_000_000:
            continue
        d = I.make_inputs(cfg, 0)
        assert d["x"].shape == (cfg.T, cfg.H) and d["x"].dtype == np.uint16
        assert d["logits"].shape == (cfg.T, cfg.E) and d["logits"].dtype == np.float32
        assert d["h"].shape == (cfg.R, 2 * cfg.I) and d["h"].dtype == np.uint16
        assert d["y"].shape == (cfg.R, cfg.H) and d["y"].dtype == np.uint16
        assert (d["bias"] is not None) == (cfg.bias_std > 0)


def test_bf16_draws_are_standard_normal():
    cfg = I.CONFIGS["decode"]
    v = I.bf16_bits_to_f32(I.make_x(cfg, 0)).astype(np.float64)
    assert abs(v.mean()) < 0.02 and abs(v.std() - 1.0) < 0.02


def test_bf16_conversion_rounds_to_nearest_even():
    f = np.array([1.0, 1.00390625, 1.01171875, -2.5, 1.0 + 2 ** -8 + 2 ** -20], np.float32)
    bits = I.f32_to_bf16_bits(f)
    assert bits.tolist() == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x3F81]


def test_bias_std():
    cfg = I.CONFIGS["deepseek_v3"]
    _, bias = I.make_logits(cfg.with_tokens(4), 0)
    assert bias.shape == (256,) and 0.35 < bias.std() < 0.65


def test_chunked_generation_is_thread_independent():
    a = I._normal_f32(5, 77, 3 * I.CHUNK + 11, threads=1)
    b = I._normal_f32(5, 77, 3 * I.CHUNK + 11, threads=8)
    assert np.array_equal(a, b)
