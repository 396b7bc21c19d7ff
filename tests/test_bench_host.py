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


# ---------------------------------------------------------------- rocprofv3
def _write_counters(d, rows):
    """A counter_collection CSV as rocprofv3 writes it (the columns used)."""
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w") as f:
        f.write('"Dispatch_Id","Grid_Size","Kernel_Name","Counter_Name","Counter_Value"\n')
        for disp, grid, name, ctr, val in rows:
            f.write(f'{disp},{grid},"{name}","{ctr}",{val}\n')


def test_request_bytes_by_size():
    c = {"TCC_EA0_RDREQ_sum": 10, "TCC_EA0_RDREQ_32B_sum": 1, "TCC_EA0_RDREQ_64B_sum": 2,
         "TCC_EA0_RDREQ_128B_sum": 7, "TCC_EA0_WRREQ_sum": 5, "TCC_EA0_WRREQ_64B_sum": 3}
    rd, wr, miss = bench.pmc_request_bytes(c)
    assert rd == 32 + 2 * 64 + 7 * 128
    assert wr == 3 * 64 + 2 * 32
    assert miss == 0
    rd, _, miss = bench.pmc_request_bytes({**c, "TCC_EA0_RDREQ_sum": 12})
    assert miss == 2  # requests of no counted size are reported, not guessed


def test_traffic_report_sums_each_call(tmp_path):
    cfg = inputs.CONFIGS["tiny"]
    probe = "void moe::(anonymous namespace)::copy_probe_kernel(x)"
    kern = {"r": "void moe::(anonymous namespace)::route_expand_small_kernel<2, 4, 1>(a)",
            "s": "void moe::(anonymous namespace)::swiglu_kernel<1>(b)",
            "c": "void moe::(anonymous namespace)::combine_kernel<true>(c)",
            "f": "void at::native::fill(d)"}
    seq = [(probe, bench.COPY_PROBE_LANES, (1 << 30) // 128, (1 << 30) // 64), (kern["f"], 64, 3, 3)]
    for _ in range(2):  # two steps
        seq += [(kern["r"], 1024, 40, 30), (kern["s"], 512, 20, 10), (kern["c"], 512, 25, 5)]
    rd_rows, wr_rows = [], []
    for i, (name, grid, r128, w64) in enumerate(seq):
        rd_rows += [(i, grid, name, "TCC_EA0_RDREQ_sum", r128), (i, grid, name, "TCC_EA0_RDREQ_128B_sum", r128),
                    (i, grid, name, "TCC_EA0_RDREQ_32B_sum", 0), (i, grid, name, "TCC_EA0_RDREQ_64B_sum", 0)]
        wr_rows += [(i, grid, name, "TCC_EA0_WRREQ_sum", w64), (i, grid, name, "TCC_EA0_WRREQ_64B_sum", w64)]
    _write_counters(tmp_path / "rd", rd_rows)
    _write_counters(tmp_path / "wr", wr_rows)
    text = bench.traffic_report(str(tmp_path / "rd"), str(tmp_path / "wr"), cfg)
    assert "read 1.00000 GiB, write 1.00000 GiB" in text
    import json
    block = json.loads(text[text.index("```json") + 7:text.rindex("```")])
    assert block["steps"] == 2
    k = block["kernels"]
    assert k["route_expand"]["traffic_bytes"] == 40 * 128 + 30 * 64
    assert k["swiglu"]["traffic_bytes"] == 20 * 128 + 10 * 64
    assert k["combine"]["traffic_bytes"] == 25 * 128 + 5 * 64
    assert k["swiglu"]["source_digest"] == bench.source_digest("swiglu")


def test_traffic_report_refuses_mismatched_passes(tmp_path):
    _write_counters(tmp_path / "rd", [(0, 64, "a(x)", "TCC_EA0_RDREQ_sum", 1)])
    _write_counters(tmp_path / "wr", [(0, 64, "b(x)", "TCC_EA0_WRREQ_sum", 1)])
    import pytest

    with pytest.raises(RuntimeError):
        bench.traffic_report(str(tmp_path / "rd"), str(tmp_path / "wr"), inputs.CONFIGS["tiny"])


def test_trace_summary_drops_warmup(tmp_path):
    p = tmp_path / "trace.csv"
    with open(p, "w") as f:
        f.write('"Kernel_Name","Grid_Size_X","Start_Timestamp","End_Timestamp"\n')
        for i, d in enumerate([1000, 900, 10, 20, 30, 40, 50]):  # two warm-up dispatches first
            f.write(f'"void moe::(anonymous namespace)::swiglu_kernel<1>(a)",64,{i * 10000},{i * 10000 + d}\n')
    out = bench.summarize_trace(str(p), 2)
    assert "| `swiglu_kernel<1>` | 5 | 30 | 30 | 10 | 50 |" in out


def test_variant_names():
    assert bench.variant_name("qwen3_30b_a3b") == "qwen3_30b_a3b"
    assert bench.variant_name("qwen3_30b_a3b", 128, 128) == "qwen3_30b_a3b_pad128_fp8g128"
    assert bench.variant_name("qwen3_30b_a3b", mxfp8=True) == "qwen3_30b_a3b_mxfp8"


def test_read_write_split_matches_the_totals():
    for name in inputs.CONFIG_ORDER:
        cfg = inputs.CONFIGS[name]
        for g in (0, 128):
            ab = bench.algorithmic_bytes(cfg, g)
            for call, (rd, wr) in bench.rw_bytes(cfg, g).items():
                if call == "route_expand_fp8" and not g:
                    continue
                assert rd + wr == ab[call], (name, g, call)
    assert bench.mix_of(8 * 10, 10) == (8, 1)
    assert bench.mix_of(10, 79) == (1, 8)
    assert bench.mix_of(2, 1) == (2, 1)
