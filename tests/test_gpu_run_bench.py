"""bench.py's own paths on the GPU: each option runs a few steps and prints
one JSON line with the fields the benchmark contract asks for."""
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("extra", [[], ["--pad", "16"], ["--fp8-group", "32"], ["--mxfp8"], ["--mxfp8", "--pad", "16"]])
@pytest.mark.parametrize("config", ["tiny", "decode"])
def test_bench_line(capsys, config, extra):
    import bench

    print(f"[bench] {config} {' '.join(extra)}", file=sys.stderr, flush=True)
    rc = bench.main(["--config", config, "--steps", "4", "--warmup", "2", "--sets", "4", "--no-cpu-baseline",
                     "--no-graph"] + extra)
    assert rc == 0
    lines = [ln for ln in capsys.readouterr().out.splitlines() if ln.startswith("{")]
    assert len(lines) == 1
    r = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
                "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in r, key
    assert r["n_gpus"] == 1 and r["steps"] == 4 and r["warmup"] == 2
    assert r["value"] > 0 and r["ms_per_step"] > 0
    assert r["config"]["workload"] == config
    assert r["roofline"]["bound"] == "hbm" and r["roofline"]["peak"] == 8000.0
    assert 0 < r["roofline"]["frac"] < 1.0
    assert all(k["us"] > 0 for k in r["kernels"].values())
