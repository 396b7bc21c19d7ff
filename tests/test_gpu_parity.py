"""HIP path vs the CPU oracle on the same seeded inputs (runs on an MI355X).

Integer outputs and copies are compared bit for bit; bf16 activations and
combined outputs within |err| <= 1e-2*|ref| + 1e-3; routing weights within
1e-5*|ref| + 1e-6.  Covered: the five workloads at full size (the launch
configuration the benchmark times), three seeds of the small ones, the token
sweep {1, 7, 32, 257, 1023} at the Qwen3-30B-A3B shape, both route variants,
and the edge cases of the method (T = 0, k = 1, k = E, E not a multiple of 4,
E = 512 with k = 16, exact ties, signed zeros, constant rows, rows that are not
a whole number of waves, every finite bf16 gate value), and seeded random
shapes across the size rule's boundaries for the benchmark's calls and for
the padded, FP8 and MXFP8 route + expand calls."""
import os
import sys

import numpy as np
import pytest

import compare
import gpu_util as G
from moe_glue_amd import inputs

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    return G.device()


def check_path(got, ref, cfg, what):
    compare.assert_route_equal(got, ref, what)
    if "x_expanded" in got:
        compare.assert_equal(got["x_expanded"], ref["x_expanded"], f"{what}.x_expanded")
    if "act" in got:
        compare.assert_bf16_close(got["act"], ref["act"], f"{what}.act")
    if "out" in got:
        compare.assert_bf16_close(got["out"], ref["out"], f"{what}.out")


# ------------------------------------------------------------------ workloads
@pytest.mark.parametrize("name", inputs.CONFIG_ORDER)
def test_workload_full_size(dev, oracle_lib, name):
    cfg = inputs.CONFIGS[name]
    _log(f"[parity] {inputs.describe(cfg)} seed=0")
    inp = inputs.make_inputs(cfg, 0)
    got = G.run_path(inp, dev)
    ref = oracle_lib.path(inp)
    check_path(got, ref, cfg, name)


@pytest.mark.parametrize("order", ["auto", "placed", "grouped", "fused"])
@pytest.mark.parametrize("name", inputs.CONFIG_ORDER)
def test_workload_full_size_route_expand(dev, oracle_lib, force, name, order):
    """Route + expand as one moe_route_expand call at full size (the form the
    benchmark times): the one-launch dispatch for decode, the grouped
    destination-order expand or the token-major one above it."""
    force.order(order)
    cfg = inputs.CONFIGS[name]
    _log(f"[parity] route_expand {inputs.describe(cfg)} seed=0 order={order}")
    inp = inputs.make_inputs(cfg, 0, parts=("x", "logits"))
    got = G.run_path(inp, dev, parts=("route", "expand"), fused=True)
    ref = oracle_lib.route(inp["logits"], cfg.k, inp["bias"])
    compare.assert_route_equal(got, ref, f"{name} route_expand")
    compare.assert_equal(got["x_expanded"], oracle_lib.expand_rows(inp["x"], ref["dest_of_src"], cfg.k),
                         f"{name} route_expand x_expanded")


@pytest.mark.parametrize("name", inputs.CONFIG_ORDER)
def test_workload_full_size_bench_path(dev, oracle_lib, name):
    """The calls the benchmark times, in its order: moe_route_expand, then
    SwiGLU and combine on the result."""
    cfg = inputs.CONFIGS[name]
    _log(f"[parity] bench path {inputs.describe(cfg)} seed=0")
    inp = inputs.make_inputs(cfg, 0)
    check_path(G.run_path(inp, dev, fused=True), oracle_lib.path(inp), cfg, f"{name} bench path")


@pytest.mark.parametrize("seed", [1, 2])
@pytest.mark.parametrize("name", ["tiny", "decode", "skewed", "qwen3_30b_a3b"])
def test_workload_more_seeds(dev, oracle_lib, name, seed):
    cfg = inputs.CONFIGS[name]
    _log(f"[parity] {inputs.describe(cfg)} seed={seed}")
    inp = inputs.make_inputs(cfg, seed)
    check_path(G.run_path(inp, dev), oracle_lib.path(inp), cfg, f"{name}/seed{seed}")


@pytest.mark.parametrize("T", [1, 7, 32, 257, 1023])
def test_token_sweep_qwen_shape(dev, oracle_lib, T):
    cfg = inputs.CONFIGS["qwen3_30b_a3b"].with_tokens(T)
    _log(f"[parity] {inputs.describe(cfg)}")
    inp = inputs.make_inputs(cfg, 0)
    check_path(G.run_path(inp, dev), oracle_lib.path(inp), cfg, cfg.name)


def _random_configs(n=40, seed=20261203):
    """Seeded random shapes across the size rule's boundaries, a quarter each
    with T in [1, 64] (the one-launch dispatch), [65, 1500], [1500, 6000],
    and [1200, 6000] with wide rows (H >= 1024, k >= 4: the placing and
    grouped expands); H a multiple of 8, log-uniform up to 8800; E in [1,
    512]; k in [1, min(E, 16)]; I a multiple of 8 up to 2048; a router bias,
    Zipf skew or tie rows now and then; at most 48M expanded elements, so
    the oracle stays quick."""
    rng = np.random.default_rng(seed)
    bands = [(1, 64, 8, 1), (65, 1500, 8, 1), (1500, 6000, 8, 1), (1200, 6000, 1024, 4)]
    out = []
    while len(out) < n:
        lo, hi, hmin, kmin = bands[len(out) % 4]
        T = int(rng.integers(lo, hi + 1))
        H = 8 * int(np.exp(rng.uniform(np.log(hmin / 8), np.log(1100.0))))
        E = int(rng.integers(kmin, 513))
        k = int(rng.integers(kmin, min(E, 16) + 1))
        I = 8 * int(rng.integers(1, 257))
        if T * k * H > 48_000_000 or T * k * 2 * I > 24_000_000:
            continue
        kind = int(rng.integers(0, 4))
        out.append(inputs.Config(f"rand{len(out)}", T=T, H=H, E=E, k=k, I=I,
                                 bias_std=0.5 if kind == 1 else 0.0, zipf_s=1.2 if kind == 2 else 0.0,
                                 tie_frac=0.05 if kind == 3 else 0.0))
    return out


@pytest.mark.parametrize("cfg", _random_configs(), ids=lambda c: c.name)
def test_random_shapes_bench_path(dev, oracle_lib, cfg):
    """The benchmark's calls (moe_route_expand in the order the size rule
    picks, then SwiGLU and combine) on seeded random shapes."""
    _log(f"[parity] random {inputs.describe(cfg)} bias={cfg.bias_std} zipf={cfg.zipf_s} ties={cfg.tie_frac}")
    inp = inputs.make_inputs(cfg, 3)
    check_path(G.run_path(inp, dev, fused=True), oracle_lib.path(inp), cfg, cfg.name)


# ------------------------------------------------------------------ route
def _route_gpu(dev, logits, k, bias=None):
    import moe_glue_amd as mg

    r = mg.route(G.to_dev(logits, dev), k, None if bias is None else G.to_dev(bias, dev))
    return G.route_host(r)


ROUTE_SHAPES = [  # (T, E, k): every lanes-per-token width, odd E, limits
    (5, 1, 1), (9, 3, 2), (33, 4, 4), (70, 8, 8), (100, 17, 5), (64, 16, 3), (65, 33, 7), (130, 64, 6),
    (200, 100, 9), (300, 128, 8), (129, 200, 2), (257, 256, 8), (1000, 300, 16), (96, 512, 16), (50, 512, 1),
]


@pytest.mark.parametrize("variant", ["auto", "single", "two", "three"])
@pytest.mark.parametrize("T,E,k", ROUTE_SHAPES)
def test_route_shapes_and_variants(dev, oracle_lib, force, variant, T, E, k):
    if variant == "single" and T > 256:
        pytest.skip("single-workgroup route covers T <= 256")
    force.route(variant)
    _log(f"[route] T={T} E={E} k={k} variant={variant}")
    rng = np.random.default_rng([T, E, k])
    logits = rng.standard_normal((T, E)).astype(np.float32)
    bias = (0.5 * rng.standard_normal(E)).astype(np.float32) if E % 2 == 0 else None
    compare.assert_route_equal(_route_gpu(dev, logits, k, bias), oracle_lib.route(logits, k, bias),
                               f"route T={T} E={E} k={k}")


@pytest.mark.parametrize("variant", ["single", "two", "three"])
@pytest.mark.parametrize("kind", ["quantized", "signed_zero", "constant", "wide"])
def test_route_ties_and_special_rows(dev, oracle_lib, force, variant, kind):
    force.route(variant)
    T, E, k = 200, 64, 6
    _log(f"[route] {kind} rows T={T} E={E} k={k} variant={variant}")
    logits = {"quantized": lambda: inputs.quantized_logits(T, E, 3),
              "signed_zero": lambda: inputs.signed_zero_logits(T, E, 3),
              "constant": lambda: inputs.constant_logits(T, E),
              "wide": lambda: inputs.wide_logits(T, E, 3)}[kind]()
    compare.assert_route_equal(_route_gpu(dev, logits, k), oracle_lib.route(logits, k), f"route {kind}")


def test_route_empty_batch(dev, oracle_lib):
    import torch
    import moe_glue_amd as mg

    _log("[route] T=0")
    out = mg.alloc_route_outputs(0, 16, 4, dev)
    out["expert_offsets"].fill_(-7)
    out["expert_counts"].fill_(-7)
    mg.route(torch.empty((0, 16), dtype=torch.float32, device=dev), 4, out=out)
    torch.cuda.synchronize()
    assert G.to_host(out["expert_offsets"]).tolist() == [0] * 17
    assert G.to_host(out["expert_counts"]).tolist() == [0] * 16


def test_route_variants_bit_identical_and_deterministic(dev, force):
    T, E, k = 256, 128, 8
    _log("[route] determinism and variants")
    logits = inputs.quantized_logits(T, E, 9)
    results = []
    for variant in ("single", "two", "three", "two", "three", "single"):
        force.route(variant)
        results.append(_route_gpu(dev, logits, k))
    for r in results[1:]:
        for key in results[0]:
            compare.assert_equal(r[key], results[0][key], f"variant/determinism {key}")


def test_skewed_tie_rows(dev, oracle_lib):
    cfg = inputs.CONFIGS["skewed"]
    _log("[route] skewed workload, injected tie rows")
    logits, bias = inputs.make_logits(cfg, 0)
    got, ref = _route_gpu(dev, logits, cfg.k, bias), oracle_lib.route(logits, cfg.k, bias)
    rows = inputs.tie_rows(cfg, 0)
    compare.assert_equal(got["topk_ids"][rows], ref["topk_ids"][rows], "tie rows")
    compare.assert_route_equal(got, ref, "skewed")


# ------------------------------------------------------------------ expand / combine
@pytest.mark.parametrize("T,H,E,k", [(1, 8, 4, 1), (3, 8, 4, 4), (77, 520, 17, 5), (300, 2048, 128, 8),
                                     (65, 4096, 64, 16), (513, 264, 8, 2), (50, 32768, 16, 4),
                                     (257, 1024, 8, 2), (130, 512, 12, 6), (33, 512, 9, 3),
                                     (64, 1536, 16, 4), (512, 16384, 16, 4), (2048, 4096, 8, 2),
                                     (1100, 8192, 32, 6), (600, 4096, 64, 8), (1023, 2048, 64, 2),
                                     (1024, 2048, 64, 2)])
def test_expand_combine_shapes(dev, oracle_lib, T, H, E, k):
    cfg = inputs.Config("adhoc", T=T, H=H, E=E, k=k, I=8)
    _log(f"[rows] T={T} H={H} E={E} k={k}")
    inp = inputs.make_inputs(cfg, 4)
    got = G.run_path(inp, dev, parts=("route", "expand", "combine"))
    ref = oracle_lib.route(inp["logits"], k)
    compare.assert_equal(got["x_expanded"], oracle_lib.expand_rows(inp["x"], ref["dest_of_src"], k), "x_expanded")
    compare.assert_bf16_close(got["out"], oracle_lib.combine(inp["y"], ref["topk_weights"], ref["dest_of_src"]),
                              "out")


@pytest.mark.parametrize("name", ["tiny", "qwen3_30b_a3b", "skewed"])
def test_combine_of_expand_is_identity(dev, name):
    """Identity experts: combine(expand(x), w) == x exactly on the GPU (as
    values: -0 and +0 are the same sum)."""
    import torch
    import moe_glue_amd as mg

    cfg = inputs.CONFIGS[name]
    _log(f"[identity] {name}")
    inp = inputs.make_inputs(cfg, 5, parts=("x", "logits"))
    x = G.to_dev(inp["x"], dev)
    r = mg.route(G.to_dev(inp["logits"], dev), cfg.k,
                 None if inp["bias"] is None else G.to_dev(inp["bias"], dev))
    assert np.array_equal(np.sort(G.to_host(r["dest_of_src"])), np.arange(cfg.R)), "dest_of_src not a permutation"
    out = mg.combine(mg.expand_rows(x, r["dest_of_src"], cfg.k), r["topk_weights"], r["dest_of_src"])
    torch.cuda.synchronize()
    # exact as values: the fp32 sum starts from +0, so a -0 in x comes back as +0
    compare.assert_equal(compare.bf16_to_f64(G.to_host(out)), compare.bf16_to_f64(inp["x"]), "combine(expand(x))")


def test_combine_unnormalised_weights(dev, oracle_lib):
    import torch
    import moe_glue_amd as mg

    T, H, E, k = 129, 1024, 32, 4
    _log("[combine] unnormalised weights")
    rng = np.random.default_rng(11)
    ref = oracle_lib.route(rng.standard_normal((T, E)).astype(np.float32), k)
    y = inputs.normal_bf16(3, 99, (T * k, H))
    w = inputs.make_weights(T, k, 3)
    got = mg.combine(G.to_dev(y, dev), G.to_dev(w, dev), G.to_dev(ref["dest_of_src"], dev))
    torch.cuda.synchronize()
    compare.assert_bf16_close(G.to_host(got), oracle_lib.combine(y, w, ref["dest_of_src"]), "combine")


# ------------------------------------------------------------------ SwiGLU
def test_swiglu_every_finite_bf16_gate(dev, oracle_lib):
    import torch
    import moe_glue_amd as mg

    _log("[swiglu] every finite bf16 gate x u in {1, -1, 0.5, 3}")
    gate = np.array([b for b in range(0x10000) if (b & 0x7F80) != 0x7F80], dtype=np.uint16)
    n = gate.size - gate.size % 8
    gate = gate[:n]
    for u_bits in (0x3F80, 0xBF80, 0x3F00, 0x4040):
        I8 = 64
        rows = n // (8 * I8)
        g = gate[: rows * 8 * I8].reshape(rows, 8 * I8)
        h = np.concatenate([g, np.full_like(g, u_bits)], axis=1)
        got = G.to_host(mg.swiglu(G.to_dev(h, dev)))
        torch.cuda.synchronize()
        compare.assert_bf16_close(got, oracle_lib.swiglu(h), f"swiglu u={u_bits:#06x}")


def test_swiglu_every_finite_bf16_gate_wide_batch(dev, oracle_lib):
    """The same on a batch large enough for the 8-byte-lane kernel (R x I =
    32768 x 2048, 2^23 16-byte items): the finite gate values tiled over the
    rows (63488 = 31 rows of 2048, so every value meets every row residue),
    u in {1, -1, 0.5, 3} by row mod 4."""
    import torch
    import moe_glue_amd as mg

    _log("[swiglu] every finite bf16 gate, 32768 x 2048 (8-byte lanes)")
    gate = np.array([b for b in range(0x10000) if (b & 0x7F80) != 0x7F80], dtype=np.uint16)
    R, I = 32768, 2048
    g = np.resize(gate, R * I).reshape(R, I)
    u_row = np.array([0x3F80, 0xBF80, 0x3F00, 0x4040], dtype=np.uint16)[np.arange(R) % 4]
    h = np.concatenate([g, np.broadcast_to(u_row[:, None], (R, I))], axis=1)
    got = G.to_host(mg.swiglu(G.to_dev(h, dev)))
    torch.cuda.synchronize()
    compare.assert_bf16_close(got, oracle_lib.swiglu(h), "swiglu every gate, wide batch")


@pytest.mark.parametrize("R,I", [(1, 8), (3, 16), (257, 768), (1023, 1408), (64, 2048), (7, 2056), (5, 16384),
                                 (1367, 6152), (32767, 2048), (32768, 2048), (40000, 1736)])
def test_swiglu_shapes(dev, oracle_lib, R, I):
    import torch
    import moe_glue_amd as mg

    _log(f"[swiglu] R={R} I={I}")
    hb = inputs.normal_bf16(R, 21, (R, 2 * I))
    got = G.to_host(mg.swiglu(G.to_dev(hb, dev)))
    torch.cuda.synchronize()
    compare.assert_bf16_close(got, oracle_lib.swiglu(hb), f"swiglu R={R} I={I}")


# ------------------------------------------------------------------ route + expand
@pytest.mark.parametrize("T,E,k,H", [(0, 16, 4, 256), (1, 8, 2, 8), (7, 128, 8, 2048), (32, 128, 8, 2048),
                                     (64, 256, 8, 7168), (64, 512, 16, 264), (33, 64, 6, 4096), (20, 3, 3, 520),
                                     (65, 128, 8, 2048), (300, 64, 6, 256), (100, 17, 5, 8), (777, 8, 2, 264),
                                     (1023, 64, 6, 4096), (2000, 256, 8, 7168), (130, 512, 16, 264),
                                     (5000, 3, 3, 8), (4096, 128, 8, 2048), (9000, 300, 4, 64),
                                     (40, 16, 4, 32768), (300, 16, 4, 32768), (150, 64, 6, 4104),
                                     (90, 128, 8, 8800)])
@pytest.mark.parametrize("order", ["auto", "placed", "grouped", "token", "fused"])
def test_route_expand_matches_oracle(dev, oracle_lib, force, order, T, E, k, H):
    import torch
    import moe_glue_amd as mg

    force.order(order)
    _log(f"[route_expand] T={T} E={E} k={k} H={H} order={order}")
    cfg = inputs.Config("adhoc", T=T, H=H, E=E, k=k, I=8, bias_std=0.5 if E % 2 == 0 else 0.0)
    inp = inputs.make_inputs(cfg, 6, parts=("x", "logits"))
    bias = None if inp["bias"] is None else G.to_dev(inp["bias"], dev)
    r = mg.route_expand(G.to_dev(inp["logits"], dev), k, G.to_dev(inp["x"], dev), bias)
    torch.cuda.synchronize()
    got = G.route_host(r)
    ref = oracle_lib.route(inp["logits"], k, inp["bias"])
    compare.assert_route_equal(got, ref, f"route_expand T={T} E={E} k={k}")
    compare.assert_equal(got["x_expanded"], oracle_lib.expand_rows(inp["x"], ref["dest_of_src"], k), "x_expanded")


@pytest.mark.parametrize("order", ["placed", "grouped", "fused"])
@pytest.mark.parametrize("variant", ["two", "three"])
def test_route_expand_workspace_needs_no_initialisation(dev, oracle_lib, force, variant, order):
    """The workspace (histogram rows, row list or slot ranks) may hold
    anything: fill it with 0xFF bytes, then with zeros, and get the same
    results both times."""
    import torch
    import moe_glue_amd as mg

    force.route(variant)
    force.order(order)
    T, E, k, H = 1500, 96, 6, 256
    _log(f"[route_expand] garbage workspace T={T} E={E} k={k} variant={variant} order={order}")
    cfg = inputs.Config("adhoc", T=T, H=H, E=E, k=k, I=8)
    inp = inputs.make_inputs(cfg, 15, parts=("x", "logits"))
    logits, x = G.to_dev(inp["logits"], dev), G.to_dev(inp["x"], dev)
    results = []
    for fill in (0xFF, 0x00):
        out = mg.alloc_route_outputs(T, E, k, dev)
        out["workspace"].fill_(fill)
        results.append(G.route_host(mg.route_expand(logits, k, x, out=out)))
    torch.cuda.synchronize()
    ref = oracle_lib.route(inp["logits"], k)
    for got in results:
        compare.assert_route_equal(got, ref, f"route_expand garbage workspace ({variant})")
        compare.assert_equal(got["x_expanded"], oracle_lib.expand_rows(inp["x"], ref["dest_of_src"], k),
                             "x_expanded")


@pytest.mark.parametrize("order", ["placed", "grouped", "fused"])
@pytest.mark.parametrize("variant", ["auto", "two", "three"])
@pytest.mark.parametrize("T,E,k,H", [(70000, 64, 2, 64), (65535, 8, 2, 16), (20000, 512, 16, 8)])
def test_route_expand_large_batches(dev, oracle_lib, force, variant, T, E, k, H, order):
    """Batches past the two-launch route's 2^16-token limit (a forced two-launch
    request falls back to three launches), many token groups, E = 512 with
    k = 16; grouped destination order, or the copy fused into the place step
    (token order after three launches)."""
    import torch
    import moe_glue_amd as mg

    force.route(variant)
    force.order(order)
    _log(f"[route_expand] large T={T} E={E} k={k} H={H} variant={variant} order={order}")
    cfg = inputs.Config("adhoc", T=T, H=H, E=E, k=k, I=8)
    inp = inputs.make_inputs(cfg, 13, parts=("x", "logits"))
    r = mg.route_expand(G.to_dev(inp["logits"], dev), k, G.to_dev(inp["x"], dev))
    torch.cuda.synchronize()
    got = G.route_host(r)
    ref = oracle_lib.route(inp["logits"], k)
    compare.assert_route_equal(got, ref, f"route_expand large T={T}")
    compare.assert_equal(got["x_expanded"], oracle_lib.expand_rows(inp["x"], ref["dest_of_src"], k), "x_expanded")


@pytest.mark.parametrize("wpg", [1, 2, 7, 64, 300])
@pytest.mark.parametrize("T,E,k,H,M", [(4096, 128, 8, 2048, 1), (1500, 96, 6, 256, 1), (3000, 64, 6, 8, 1),
                                       (777, 256, 8, 16392, 1), (5000, 16, 4, 520, 1), (2500, 128, 8, 1024, 128),
                                       (4100, 200, 6, 264, 7)])
def test_route_expand_placed_slicing(dev, oracle_lib, force, wpg, T, E, k, H, M):
    """The placing destination-order expand with the number of workgroups per
    token group forced (1 to more than the group has row chunks), rows of one
    16-byte vector up to more than one pass of a workgroup, E not a multiple
    of 16, padded segments: the maps and every copied row match the oracle,
    padding rows stay untouched."""
    import torch
    import moe_glue_amd as mg

    force.order("placed")
    force.workgroups_per_group(wpg)
    _log(f"[placed] T={T} E={E} k={k} H={H} pad_to={M} workgroups/group={wpg}")
    cfg = inputs.Config("adhoc", T=T, H=H, E=E, k=k, I=8, bias_std=0.5)
    inp = inputs.make_inputs(cfg, 17, parts=("x", "logits"))
    ref = oracle_lib.route_padded(inp["logits"], k, M, inp["bias"])
    P = int(ref["expert_offsets"][E])
    rows = mg.padded_rows(T, E, k, M) if M > 1 else T * k
    out = mg.alloc_route_outputs(T, E, k, dev)
    out["src_of_dest"] = torch.empty((rows,), dtype=torch.int32, device=dev)
    out["x_expanded"] = torch.full((rows, H), 0x7F7F, dtype=torch.int16, device=dev).view(torch.bfloat16)
    out["workspace"].fill_(0xEE)
    bias = G.to_dev(inp["bias"], dev)
    r = mg.route_expand_padded(G.to_dev(inp["logits"], dev), k, M, G.to_dev(inp["x"], dev), bias, out=out)
    torch.cuda.synchronize()
    got = G.route_host(r)
    got["src_of_dest"] = got["src_of_dest"][:P]
    xe = got.pop("x_expanded")[:P]
    compare.assert_route_equal(got, ref, f"placed T={T} E={E} k={k} M={M} wpg={wpg}")
    want = oracle_lib.expand_rows(inp["x"], ref["dest_of_src"], k, rows=P)
    pad_rows = ref["src_of_dest"] < 0
    compare.assert_equal(xe[~pad_rows], want[~pad_rows], "placed x_expanded (real rows)")
    assert np.all(xe[pad_rows] == 0x7F7F), "placed: a padding row was written"


@pytest.mark.parametrize("order", ["grouped", "placed"])
@pytest.mark.parametrize("variant", ["single", "two", "three"])
@pytest.mark.parametrize("T", [48, 700])
def test_route_expand_equals_separate_calls(dev, force, variant, T, order):
    import torch
    import moe_glue_amd as mg

    if variant == "single" and T > 256:
        pytest.skip("single-workgroup route covers T <= 256")
    force.order(order)
    E, k, H = 128, 8, 2048
    _log(f"[route_expand] T={T} auto vs forced variant {variant}")
    cfg = inputs.Config("adhoc", T=T, H=H, E=E, k=k, I=8)
    inp = inputs.make_inputs(cfg, 8, parts=("x", "logits"))
    logits, x = G.to_dev(inp["logits"], dev), G.to_dev(inp["x"], dev)
    fused = G.route_host(mg.route_expand(logits, k, x))
    force.route(variant)
    r = mg.route_expand(logits, k, x)
    torch.cuda.synchronize()
    sep = G.route_host(r)
    for key in fused:
        compare.assert_equal(sep[key], fused[key], f"fused vs {variant}: {key}")


# ------------------------------------------------------------------ padded segments
PADDED_CASES = [(1, 8, 2, 4), (33, 8, 2, 16), (100, 17, 5, 8), (300, 128, 8, 128), (64, 512, 16, 32),
                (1023, 64, 6, 64), (257, 256, 8, 3), (4096, 128, 8, 128), (50, 4, 4, 1)]


@pytest.mark.parametrize("variant", ["auto", "single", "two", "three"])
@pytest.mark.parametrize("T,E,k,M", PADDED_CASES)
def test_route_padded_matches_oracle(dev, oracle_lib, force, variant, T, E, k, M):
    import moe_glue_amd as mg

    if variant == "single" and T > 256:
        pytest.skip("single-workgroup route covers T <= 256")
    force.route(variant)
    _log(f"[route_padded] T={T} E={E} k={k} pad_to={M} variant={variant}")
    rng = np.random.default_rng([T, E, k, M])
    logits = rng.standard_normal((T, E)).astype(np.float32)
    r = G.route_host(mg.route_padded(G.to_dev(logits, dev), k, M))
    ref = oracle_lib.route_padded(logits, k, M)
    P = int(ref["expert_offsets"][E])
    r["src_of_dest"] = r["src_of_dest"][:P]
    compare.assert_route_equal(r, ref, f"route_padded T={T} E={E} k={k} M={M}")


@pytest.mark.parametrize("T,E,k,M,H", [(300, 128, 8, 128, 2048), (77, 17, 5, 16, 520), (1023, 64, 6, 64, 4096)])
def test_expand_combine_on_padded_layout(dev, oracle_lib, T, E, k, M, H):
    import torch
    import moe_glue_amd as mg

    _log(f"[padded rows] T={T} E={E} k={k} pad_to={M} H={H}")
    cfg = inputs.Config("adhoc", T=T, H=H, E=E, k=k, I=8)
    inp = inputs.make_inputs(cfg, 9, parts=("x", "logits"))
    ref = oracle_lib.route_padded(inp["logits"], k, M)
    P = int(ref["expert_offsets"][E])
    r = mg.route_padded(G.to_dev(inp["logits"], dev), k, M)
    sentinel = 0x7F7F
    xe = torch.full((mg.padded_rows(T, E, k, M), H), sentinel, dtype=torch.int16, device=dev).view(torch.bfloat16)
    mg.expand_rows(G.to_dev(inp["x"], dev), r["dest_of_src"], k, out=xe)
    torch.cuda.synchronize()
    got = G.to_host(xe)[:P]
    want = oracle_lib.expand_rows(inp["x"], ref["dest_of_src"], k, rows=P)
    pad_rows = ref["src_of_dest"] < 0
    compare.assert_equal(got[~pad_rows], want[~pad_rows], "padded x_expanded (valid rows)")
    assert np.all(got[pad_rows] == sentinel), "expand wrote into padding rows"
    # combine reads only valid rows of a padded y
    y = inputs.normal_bf16(9, 77, (P, H))
    out = mg.combine(G.to_dev(y, dev), r["topk_weights"], r["dest_of_src"])
    torch.cuda.synchronize()
    compare.assert_bf16_close(G.to_host(out), oracle_lib.combine(y, ref["topk_weights"], ref["dest_of_src"]),
                              "combine on padded y")


@pytest.mark.parametrize("order", ["auto", "placed", "grouped", "token", "fused"])
@pytest.mark.parametrize("T,E,k,M,H", [(20, 8, 2, 16, 256), (64, 512, 16, 32, 264), (32, 128, 8, 128, 2048),
                                       (1, 3, 2, 5, 8), (300, 128, 8, 128, 2048), (77, 17, 5, 16, 520),
                                       (1023, 64, 6, 64, 4096), (4096, 128, 8, 128, 2048), (2000, 256, 8, 3, 264)])
def test_route_expand_padded_matches_oracle(dev, oracle_lib, force, order, T, E, k, M, H):
    """moe_route_expand_padded: the padded maps, every real row copied, the
    padding rows untouched (sentinel), in every expand order."""
    import torch
    import moe_glue_amd as mg

    force.order(order)
    _log(f"[route_expand_padded] T={T} E={E} k={k} pad_to={M} H={H} order={order}")
    cfg = inputs.Config("adhoc", T=T, H=H, E=E, k=k, I=8, bias_std=0.5 if E % 2 == 0 else 0.0)
    inp = inputs.make_inputs(cfg, 14, parts=("x", "logits"))
    ref = oracle_lib.route_padded(inp["logits"], k, M, inp["bias"])
    P = int(ref["expert_offsets"][E])
    rows = mg.padded_rows(T, E, k, M)
    out = mg.alloc_route_outputs(T, E, k, dev)
    out["src_of_dest"] = torch.empty((rows,), dtype=torch.int32, device=dev)
    sentinel = 0x7F7F
    out["x_expanded"] = torch.full((rows, H), sentinel, dtype=torch.int16, device=dev).view(torch.bfloat16)
    bias = None if inp["bias"] is None else G.to_dev(inp["bias"], dev)
    r = mg.route_expand_padded(G.to_dev(inp["logits"], dev), k, M, G.to_dev(inp["x"], dev), bias, out=out)
    torch.cuda.synchronize()
    got = G.route_host(r)
    got["src_of_dest"] = got["src_of_dest"][:P]
    xe = got.pop("x_expanded")[:P]
    compare.assert_route_equal(got, ref, f"route_expand_padded T={T} E={E} k={k} M={M}")
    want = oracle_lib.expand_rows(inp["x"], ref["dest_of_src"], k, rows=P)
    pad_rows = ref["src_of_dest"] < 0
    compare.assert_equal(xe[~pad_rows], want[~pad_rows], "padded x_expanded (real rows)")
    assert np.all(xe[pad_rows] == sentinel), "the fused call wrote into padding rows"


# ------------------------------------------------------------------ FP8 quantising expand
@pytest.mark.parametrize("T,H,E,k,group", [(1, 8, 4, 1, 8), (17, 256, 8, 2, 32), (300, 2048, 128, 8, 128),
                                           (77, 520, 17, 5, 8), (65, 4096, 64, 16, 512), (33, 7168, 256, 8, 128),
                                           (129, 1024, 32, 4, 64), (40, 96, 6, 3, 16)])
def test_expand_fp8_matches_oracle(dev, oracle_lib, T, H, E, k, group):
    import torch
    import moe_glue_amd as mg

    _log(f"[expand_fp8] T={T} H={H} E={E} k={k} group={group}")
    cfg = inputs.Config("adhoc", T=T, H=H, E=E, k=k, I=8)
    inp = inputs.make_inputs(cfg, 12, parts=("x", "logits"))
    x = inp["x"].copy()
    x[0, :group] = 0                      # an all-zero group
    x[-1, -group:] = np.uint16(0x3F80)    # a constant group: every code is +448
    r = oracle_lib.route(inp["logits"], k)
    q, sc = mg.expand_rows_fp8(G.to_dev(x, dev), G.to_dev(r["dest_of_src"], dev), k, group)
    torch.cuda.synchronize()
    qr, scr = oracle_lib.expand_rows_fp8(x, r["dest_of_src"], k, group)
    compare.assert_equal(G.to_host(sc), scr, "fp8 scales")
    compare.assert_equal(G.to_host(q), qr, "fp8 codes")


def test_expand_fp8_qwen_workload_and_padded_layout(dev, oracle_lib):
    import torch
    import moe_glue_amd as mg

    cfg = inputs.CONFIGS["qwen3_30b_a3b"]
    _log(f"[expand_fp8] {inputs.describe(cfg)} group=128, padded to 128 rows")
    inp = inputs.make_inputs(cfg, 0, parts=("x", "logits"))
    ref = oracle_lib.route_padded(inp["logits"], cfg.k, 128)
    P = int(ref["expert_offsets"][cfg.E])
    r = mg.route_padded(G.to_dev(inp["logits"], dev), cfg.k, 128)
    q = torch.full((mg.padded_rows(cfg.T, cfg.E, cfg.k, 128), cfg.H), 0xAB, dtype=torch.uint8, device=dev)
    q, sc = mg.expand_rows_fp8(G.to_dev(inp["x"], dev), r["dest_of_src"], cfg.k, 128, rows=q.shape[0], out=q)
    torch.cuda.synchronize()
    qr, scr = oracle_lib.expand_rows_fp8(inp["x"], ref["dest_of_src"], cfg.k, 128, rows=P)
    valid = ref["src_of_dest"] >= 0
    qh, sch = G.to_host(q)[:P], G.to_host(sc)[:P]
    compare.assert_equal(qh[valid], qr[valid], "fp8 codes (valid rows)")
    compare.assert_equal(sch[valid], scr[valid], "fp8 scales (valid rows)")
    assert np.all(qh[~valid] == 0xAB), "fp8 expand wrote into padding rows"


# ------------------------------------------------------------------ MXFP8 quantising expand
def _mx_special_rows(x: np.ndarray, seed: int) -> np.ndarray:
    """Blocks that exercise the MX scale: all zero, saturating (1.875 * 2^8 >
    448), magnitudes spread over +-100 binades, and tiny negatives beside a
    block maximum of 1 (their codes are -0)."""
    import bruteforce as bf

    x = x.copy()
    T, H = x.shape
    rng = np.random.default_rng(seed)
    x[0, :32] = 0
    x[-1, -32:] = np.uint16(0x3FF0)  # bf16 1.875
    if T > 1:
        v = rng.standard_normal(H) * np.repeat(2.0 ** rng.integers(-100, 100, H // 32), 32)
        x[1] = bf.bf16_round_exact_np(v)
    if T > 2:
        v = -np.abs(rng.standard_normal(32)) * 1e-30
        v[5] = 1.0
        x[2, :32] = bf.bf16_round_exact_np(v)
    return x


@pytest.mark.parametrize("T,H,E,k", [(1, 32, 4, 1), (17, 256, 8, 2), (300, 2048, 128, 8), (77, 544, 17, 5),
                                     (65, 4096, 64, 16), (33, 7168, 256, 8), (40, 96, 6, 3), (1023, 1408, 64, 6)])
def test_expand_mxfp8_matches_oracle(dev, oracle_lib, T, H, E, k):
    import torch
    import moe_glue_amd as mg

    _log(f"[expand_mxfp8] T={T} H={H} E={E} k={k}")
    cfg = inputs.Config("adhoc", T=T, H=H, E=E, k=k, I=8)
    inp = inputs.make_inputs(cfg, 13, parts=("x", "logits"))
    x = _mx_special_rows(inp["x"], 13)
    r = oracle_lib.route(inp["logits"], k)
    q, sc = mg.expand_rows_mxfp8(G.to_dev(x, dev), G.to_dev(r["dest_of_src"], dev), k)
    torch.cuda.synchronize()
    qr, scr = oracle_lib.expand_rows_mxfp8(x, r["dest_of_src"], k)
    compare.assert_equal(G.to_host(sc), scr, "mxfp8 scale bytes")
    compare.assert_equal(G.to_host(q), qr, "mxfp8 codes")


def test_expand_mxfp8_qwen_workload(dev, oracle_lib):
    import torch
    import moe_glue_amd as mg

    cfg = inputs.CONFIGS["qwen3_30b_a3b"]
    _log(f"[expand_mxfp8] {inputs.describe(cfg)}")
    inp = inputs.make_inputs(cfg, 0, parts=("x", "logits"))
    r = mg.route(G.to_dev(inp["logits"], dev), cfg.k)
    q, sc = mg.expand_rows_mxfp8(G.to_dev(inp["x"], dev), r["dest_of_src"], cfg.k)
    torch.cuda.synchronize()
    qr, scr = oracle_lib.expand_rows_mxfp8(inp["x"], G.to_host(r["dest_of_src"]), cfg.k)
    compare.assert_equal(G.to_host(sc), scr, "mxfp8 scale bytes")
    compare.assert_equal(G.to_host(q), qr, "mxfp8 codes")


# T, E, k, H, group, pad_to; order auto folds the quantising copy into the
# route's place step for small batches, token never, fused whenever possible
FP8_FUSED_CASES = [(1, 8, 2, 256, 8, 1), (40, 64, 6, 512, 128, 1), (300, 128, 8, 2048, 128, 1),
                   (300, 128, 8, 2048, 128, 128), (1023, 64, 6, 4096, 256, 1), (1023, 64, 6, 4096, 512, 16),
                   (500, 8, 2, 1024, 128, 16), (500, 8, 2, 1024, 256, 1), (500, 4, 2, 512, 64, 1),
                   (500, 4, 2, 512, 128, 3), (77, 17, 5, 520, 8, 16), (4096, 128, 8, 2048, 128, 1),
                   (2000, 512, 16, 264, 8, 1), (32, 128, 8, 2048, 128, 1), (64, 256, 8, 7168, 128, 128),
                   (0, 16, 4, 256, 64, 1), (64, 4, 2, 512, 512, 8)]


@pytest.mark.parametrize("order", ["auto", "token", "fused"])
@pytest.mark.parametrize("T,E,k,H,group,M", FP8_FUSED_CASES)
def test_route_expand_fp8_matches_oracle(dev, oracle_lib, force, order, T, E, k, H, group, M):
    """moe_route_expand_fp8 = route (padded for M > 1) then the quantising
    expand; padding rows of the codes and scales stay untouched."""
    import torch
    import moe_glue_amd as mg

    force.order(order)
    _log(f"[route_expand_fp8] T={T} E={E} k={k} H={H} group={group} pad_to={M} order={order}")
    cfg = inputs.Config("adhoc", T=T, H=H, E=E, k=k, I=8, bias_std=0.5 if E % 2 == 0 else 0.0)
    inp = inputs.make_inputs(cfg, 9, parts=("x", "logits"))
    bias = None if inp["bias"] is None else G.to_dev(inp["bias"], dev)
    P = mg.padded_rows(T, E, k, M) if M > 1 else T * k
    out = mg.alloc_route_outputs(T, E, k, dev)
    out["src_of_dest"] = torch.empty((P,), dtype=torch.int32, device=dev)
    out["x_expanded"] = torch.full((P, H), 0xAB, dtype=torch.uint8, device=dev)
    out["scales"] = torch.full((P, H // group), -7.0, dtype=torch.float32, device=dev)
    r = mg.route_expand_fp8(G.to_dev(inp["logits"], dev), k, G.to_dev(inp["x"], dev), group, M, bias, out=out)
    torch.cuda.synchronize()
    got = G.route_host(r)
    ref = (oracle_lib.route_padded(inp["logits"], k, M, inp["bias"]) if M > 1
           else oracle_lib.route(inp["logits"], k, inp["bias"]))
    n = int(ref["expert_offsets"][E])
    got["src_of_dest"] = got["src_of_dest"][:n]
    compare.assert_route_equal({key: v for key, v in got.items() if key not in ("x_expanded", "scales")}, ref,
                               f"route_expand_fp8 T={T} E={E} k={k} M={M}")
    qr, scr = oracle_lib.expand_rows_fp8(inp["x"], ref["dest_of_src"], k, group, rows=n)
    valid = ref["src_of_dest"] >= 0
    qh, sch = got["x_expanded"][:n], got["scales"][:n]
    compare.assert_equal(qh[valid], qr[valid], "fp8 codes (valid rows)")
    compare.assert_equal(sch[valid], scr[valid], "fp8 scales (valid rows)")
    assert np.all(qh[~valid] == 0xAB) and np.all(got["x_expanded"][n:] == 0xAB), "codes written into padding rows"
    assert np.all(sch[~valid] == -7.0) and np.all(got["scales"][n:] == -7.0), "scales written into padding rows"


def _with_tiny_groups(x, group, seed):
    """x with tiny groups planted in several tokens: maxima of about 1e-37
    (448/amax overflows fp32), about 1e-25 (below 2^-64, no overflow) and
    bf16 subnormals (2^-133 and up), signs mixed; other groups untouched."""
    import bruteforce as bf

    x = x.copy()
    T, H = x.shape
    rng = np.random.default_rng(seed)
    for t in range(0, T, max(1, T // 7)):
        kind = t % 3
        g0 = (t // 3) % max(1, H // group) * group
        if kind == 0:
            x[t, g0:g0 + group] = bf.bf16_round_exact_np(rng.standard_normal(group) * 1e-37)
        elif kind == 1:
            x[t, g0:g0 + group] = bf.bf16_round_exact_np(rng.standard_normal(group) * 1e-25)
        else:
            x[t, g0:g0 + group] = rng.integers(1, 0x80, group).astype(np.uint16) | \
                (rng.integers(0, 2, group).astype(np.uint16) << 15)
    return x


@pytest.mark.parametrize("path", ["expand", "dispatch", "folded", "separate"])
@pytest.mark.parametrize("group", [8, 32, 128])
def test_fp8_tiny_groups(dev, oracle_lib, force, path, group):
    """FP8 groups whose maximum is tiny (448/amax overflows fp32, or amax is a
    bf16 subnormal): codes and scales as the oracle's exponent-unlimited
    reading gives them, through the quantising expand, the one-launch
    dispatch (T <= 64), the copy folded into the route's place launch and
    the route followed by the separate quantising expand."""
    import torch
    import moe_glue_amd as mg

    T = 48 if path == "dispatch" else 300
    E, k, H = 64, 6, 1024
    _log(f"[fp8 tiny groups] path={path} T={T} group={group}")
    cfg = inputs.Config("adhoc", T=T, H=H, E=E, k=k, I=8)
    inp = inputs.make_inputs(cfg, 31, parts=("x", "logits"))
    x = _with_tiny_groups(inp["x"], group, 5)
    ref = oracle_lib.route(inp["logits"], k)
    qr, scr = oracle_lib.expand_rows_fp8(x, ref["dest_of_src"], k, group)
    if path == "expand":
        q, sc = mg.expand_rows_fp8(G.to_dev(x, dev), G.to_dev(ref["dest_of_src"], dev), k, group)
        torch.cuda.synchronize()
        q, sc = G.to_host(q), G.to_host(sc)
    else:
        force.order({"dispatch": "auto", "folded": "fused", "separate": "token"}[path])
        if path != "dispatch":
            force.route("two")
        r = mg.route_expand_fp8(G.to_dev(inp["logits"], dev), k, G.to_dev(x, dev), group)
        torch.cuda.synchronize()
        got = G.route_host(r)
        compare.assert_route_equal({key: v for key, v in got.items() if key not in ("x_expanded", "scales")}, ref,
                                   f"fp8 tiny groups route ({path})")
        q, sc = got["x_expanded"], got["scales"]
    compare.assert_equal(sc, scr, f"fp8 tiny-group scales ({path})")
    compare.assert_equal(q, qr, f"fp8 tiny-group codes ({path})")


MX_FUSED_CASES = [(T, E, k, H, M) for (T, E, k, H, group, M) in FP8_FUSED_CASES if H % 32 == 0]


@pytest.mark.parametrize("order", ["auto", "token", "fused"])
@pytest.mark.parametrize("T,E,k,H,M", MX_FUSED_CASES)
def test_route_expand_mxfp8_matches_oracle(dev, oracle_lib, force, order, T, E, k, H, M):
    """moe_route_expand_mxfp8 = route (padded for M > 1) then the MXFP8
    expand; padding rows of the codes and scale bytes stay untouched."""
    import torch
    import moe_glue_amd as mg

    force.order(order)
    _log(f"[route_expand_mxfp8] T={T} E={E} k={k} H={H} pad_to={M} order={order}")
    cfg = inputs.Config("adhoc", T=T, H=H, E=E, k=k, I=8, bias_std=0.5 if E % 2 == 0 else 0.0)
    inp = inputs.make_inputs(cfg, 10, parts=("x", "logits"))
    x = _mx_special_rows(inp["x"], 10) if T > 0 else inp["x"]
    bias = None if inp["bias"] is None else G.to_dev(inp["bias"], dev)
    P = mg.padded_rows(T, E, k, M) if M > 1 else T * k
    out = mg.alloc_route_outputs(T, E, k, dev)
    out["src_of_dest"] = torch.empty((max(P, 1),), dtype=torch.int32, device=dev)
    out["x_expanded"] = torch.full((max(P, 1), H), 0xAB, dtype=torch.uint8, device=dev)
    out["scales"] = torch.full((max(P, 1), H // 32), 0xCD, dtype=torch.uint8, device=dev)
    r = mg.route_expand_mxfp8(G.to_dev(inp["logits"], dev), k, G.to_dev(x, dev), M, bias, out=out)
    torch.cuda.synchronize()
    got = G.route_host(r)
    ref = (oracle_lib.route_padded(inp["logits"], k, M, inp["bias"]) if M > 1
           else oracle_lib.route(inp["logits"], k, inp["bias"]))
    n = int(ref["expert_offsets"][E])
    got["src_of_dest"] = got["src_of_dest"][:n]
    compare.assert_route_equal({key: v for key, v in got.items() if key not in ("x_expanded", "scales")}, ref,
                               f"route_expand_mxfp8 T={T} E={E} k={k} M={M}")
    qr, scr = oracle_lib.expand_rows_mxfp8(x, ref["dest_of_src"], k, rows=n)
    valid = ref["src_of_dest"] >= 0
    qh, sch = got["x_expanded"][:n], got["scales"][:n]
    compare.assert_equal(qh[valid], qr[valid], "mxfp8 codes (valid rows)")
    compare.assert_equal(sch[valid], scr[valid], "mxfp8 scale bytes (valid rows)")
    assert np.all(qh[~valid] == 0xAB) and np.all(got["x_expanded"][n:] == 0xAB), "codes written into padding rows"
    assert np.all(sch[~valid] == 0xCD) and np.all(got["scales"][n:] == 0xCD), "scales written into padding rows"


@pytest.mark.parametrize("fmt", ["fp8", "mxfp8"])
@pytest.mark.parametrize("variant", ["single", "two", "three"])
@pytest.mark.parametrize("T,E,k,H,M", [(48, 128, 8, 2048, 1), (48, 64, 6, 512, 16), (700, 128, 8, 1024, 1),
                                       (700, 17, 5, 256, 8)])
def test_route_expand_quantised_every_route_variant(dev, oracle_lib, force, fmt, variant, T, E, k, H, M):
    """The combined quantising calls with the route variant forced: the
    single-workgroup route followed by the separate quantising expand, and
    the two- and three-launch routes (folded copy or separate expand)."""
    import torch
    import moe_glue_amd as mg

    if variant == "single" and T > 256:
        pytest.skip("single-workgroup route covers T <= 256")
    force.route(variant)
    _log(f"[route_expand_{fmt}] T={T} E={E} k={k} H={H} pad_to={M} variant={variant}")
    cfg = inputs.Config("adhoc", T=T, H=H, E=E, k=k, I=8)
    inp = inputs.make_inputs(cfg, 11, parts=("x", "logits"))
    x = _mx_special_rows(inp["x"], 11)
    if fmt == "fp8":
        r = mg.route_expand_fp8(G.to_dev(inp["logits"], dev), k, G.to_dev(x, dev), 32, M)
    else:
        r = mg.route_expand_mxfp8(G.to_dev(inp["logits"], dev), k, G.to_dev(x, dev), M)
    torch.cuda.synchronize()
    got = G.route_host(r)
    ref = oracle_lib.route_padded(inp["logits"], k, M) if M > 1 else oracle_lib.route(inp["logits"], k)
    n = int(ref["expert_offsets"][E])
    got["src_of_dest"] = got["src_of_dest"][:n]
    compare.assert_route_equal({key: v for key, v in got.items() if key not in ("x_expanded", "scales")}, ref,
                               f"route_expand_{fmt} T={T} variant={variant}")
    if fmt == "fp8":
        qr, scr = oracle_lib.expand_rows_fp8(x, ref["dest_of_src"], k, 32, rows=n)
    else:
        qr, scr = oracle_lib.expand_rows_mxfp8(x, ref["dest_of_src"], k, rows=n)
    valid = ref["src_of_dest"] >= 0
    compare.assert_equal(got["x_expanded"][:n][valid], qr[valid], f"{fmt} codes (valid rows)")
    compare.assert_equal(got["scales"][:n][valid], scr[valid], f"{fmt} scales (valid rows)")


def _random_variant_cases(n=36, seed=20261204):
    """Seeded random shapes (as for the bench-path sweep) for the padded,
    FP8 and MXFP8 route + expand calls, in turn: pad_to in [2, 256] for the
    padded call, in {1} or [2, 256] for the quantising ones (lowered where
    the padded rows would pass 48M elements); the FP8 group a power of two
    in [8, 512] dividing H; H rounded up to a multiple of 32 for MXFP8."""
    rng = np.random.default_rng(seed)
    out = []
    for i, cfg in enumerate(_random_configs(n, seed)):
        fmt = ("padded", "fp8", "mxfp8")[i % 3]
        M = int(rng.integers(2, 257)) if fmt == "padded" or rng.integers(0, 2) else 1
        H = cfg.H
        # at most T*k + E*(pad_to - 1) padded rows: keep them under 48M elements
        M = max(1, min(M, (48_000_000 // H - cfg.T * cfg.k) // cfg.E + 1))
        group = 0
        if fmt == "fp8":
            groups = [g for g in (8, 16, 32, 64, 128, 256, 512) if H % g == 0]
            group = int(groups[rng.integers(0, len(groups))])
        if fmt == "mxfp8":
            H = (H + 31) // 32 * 32
        c = inputs.Config(cfg.name, T=cfg.T, H=H, E=cfg.E, k=cfg.k, I=8, bias_std=cfg.bias_std,
                          zipf_s=cfg.zipf_s, tie_frac=cfg.tie_frac)
        out.append((c, fmt, M, group))
    return out


@pytest.mark.parametrize("cfg,fmt,M,group", _random_variant_cases(), ids=lambda v: getattr(v, "name", str(v)))
def test_random_shapes_padded_and_quantised(dev, oracle_lib, cfg, fmt, M, group):
    """moe_route_expand_padded / _fp8 / _mxfp8 in the order the size rule
    picks, on seeded random shapes: maps, rows (codes and scales) of every
    real row, padding rows untouched."""
    import torch
    import moe_glue_amd as mg

    T, E, k, H = cfg.T, cfg.E, cfg.k, cfg.H
    _log(f"[random {fmt}] {inputs.describe(cfg)} pad_to={M} group={group} bias={cfg.bias_std} "
         f"zipf={cfg.zipf_s} ties={cfg.tie_frac}")
    inp = inputs.make_inputs(cfg, 5, parts=("x", "logits"))
    bias = None if inp["bias"] is None else G.to_dev(inp["bias"], dev)
    P = mg.padded_rows(T, E, k, M) if M > 1 else T * k
    out = mg.alloc_route_outputs(T, E, k, dev)
    out["src_of_dest"] = torch.empty((max(P, 1),), dtype=torch.int32, device=dev)
    if fmt == "padded":
        out["x_expanded"] = torch.full((max(P, 1), H), 0x7F7F, dtype=torch.int16, device=dev).view(torch.bfloat16)
    else:
        out["x_expanded"] = torch.full((max(P, 1), H), 0xAB, dtype=torch.uint8, device=dev)
        if fmt == "fp8":
            out["scales"] = torch.full((max(P, 1), H // group), -7.0, dtype=torch.float32, device=dev)
        else:
            out["scales"] = torch.full((max(P, 1), H // 32), 0xCD, dtype=torch.uint8, device=dev)
    lg, xd = G.to_dev(inp["logits"], dev), G.to_dev(inp["x"], dev)
    if fmt == "padded":
        r = mg.route_expand_padded(lg, k, M, xd, bias, out=out)
    elif fmt == "fp8":
        r = mg.route_expand_fp8(lg, k, xd, group, M, bias, out=out)
    else:
        r = mg.route_expand_mxfp8(lg, k, xd, M, bias, out=out)
    torch.cuda.synchronize()
    got = G.route_host(r)
    ref = (oracle_lib.route_padded(inp["logits"], k, M, inp["bias"]) if M > 1
           else oracle_lib.route(inp["logits"], k, inp["bias"]))
    n = int(ref["expert_offsets"][E])
    got["src_of_dest"] = got["src_of_dest"][:n]
    rows = {key: got.pop(key) for key in ("x_expanded", "scales") if key in got}
    compare.assert_route_equal(got, ref, f"random {fmt} T={T} E={E} k={k} M={M}")
    valid = ref["src_of_dest"] >= 0
    xe = rows["x_expanded"]
    if fmt == "padded":
        want = oracle_lib.expand_rows(inp["x"], ref["dest_of_src"], k, rows=n)
        compare.assert_equal(xe[:n][valid], want[valid], "padded x_expanded (real rows)")
        assert np.all(xe[:n][~valid] == 0x7F7F) and np.all(xe[n:] == 0x7F7F), "rows written into padding"
        return
    if fmt == "fp8":
        qr, scr = oracle_lib.expand_rows_fp8(inp["x"], ref["dest_of_src"], k, group, rows=n)
        untouched = -7.0
    else:
        qr, scr = oracle_lib.expand_rows_mxfp8(inp["x"], ref["dest_of_src"], k, rows=n)
        untouched = 0xCD
    sc = rows["scales"]
    compare.assert_equal(xe[:n][valid], qr[valid], f"{fmt} codes (real rows)")
    compare.assert_equal(sc[:n][valid], scr[valid], f"{fmt} scales (real rows)")
    assert np.all(xe[:n][~valid] == 0xAB) and np.all(xe[n:] == 0xAB), "codes written into padding rows"
    assert np.all(sc[:n][~valid] == untouched) and np.all(sc[n:] == untouched), "scales written into padding"


@pytest.mark.parametrize("T,E,k,H,I,variant,order", [(32, 128, 8, 2048, 768, "auto", "auto"),
                                                     (4096, 128, 8, 2048, 768, "auto", "auto"),
                                                     (700, 64, 6, 256, 64, "two", "placed"),
                                                     (700, 64, 6, 256, 64, "two", "grouped"),
                                                     (300, 128, 8, 512, 32, "three", "token"),
                                                     (1023, 64, 6, 4096, 1408, "auto", "fused")])
def test_graph_replay_matches_eager(dev, force, T, E, k, H, I, variant, order):
    """route_expand, swiglu and combine captured in one HIP graph: every replay
    (outputs overwritten with garbage by eager work in between) gives exactly
    the eager results."""
    import torch
    import moe_glue_amd as mg

    force.route(variant)
    force.order(order)
    _log(f"[graph] T={T} E={E} k={k} H={H} I={I} variant={variant} order={order}")
    cfg = inputs.Config("adhoc", T=T, H=H, E=E, k=k, I=I)
    inp = inputs.make_inputs(cfg, 21, parts=("x", "logits", "h", "y"))
    logits, x = G.to_dev(inp["logits"], dev), G.to_dev(inp["x"], dev)
    h, y = G.to_dev(inp["h"], dev), G.to_dev(inp["y"], dev)

    def run(out, act, comb):
        mg.route_expand(logits, k, x, out=out)
        mg.swiglu(h, out=act)
        mg.combine(y, out["topk_weights"], out["dest_of_src"], out=comb)

    def alloc():
        out = mg.alloc_route_outputs(T, E, k, dev)
        out["x_expanded"] = torch.empty((T * k, H), dtype=torch.bfloat16, device=dev)
        return out, torch.empty((T * k, I), dtype=torch.bfloat16, device=dev), \
            torch.empty((T, H), dtype=torch.bfloat16, device=dev)

    ref = alloc()
    run(*ref)
    torch.cuda.synchronize()
    want = {key: G.to_host(v) for key, v in ref[0].items() if key != "workspace"}
    want["act"], want["out"] = G.to_host(ref[1]), G.to_host(ref[2])

    bufs = alloc()
    side = torch.cuda.Stream(device=dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        run(*bufs)
    for rep in range(3):
        for key, v in bufs[0].items():
            v.view(torch.uint8).fill_(0xA5 + rep)
        bufs[1].view(torch.uint8).fill_(0x5A)
        bufs[2].view(torch.uint8).fill_(0x3C)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = {key: G.to_host(v) for key, v in bufs[0].items() if key != "workspace"}
        got["act"], got["out"] = G.to_host(bufs[1]), G.to_host(bufs[2])
        for key in want:
            compare.assert_equal(got[key], want[key], f"graph replay {rep}: {key}")


def test_concurrent_streams(dev, oracle_lib):
    """Calls on two streams at once, each with its own buffers (the library
    keeps no state between calls): three batches, one per route + expand form
    (one-launch dispatch, the route's place step copying, the placing
    expand), issued alternately on two streams with no synchronisation in
    between, each result against the oracle."""
    import torch
    import moe_glue_amd as mg

    shapes = [(40, 128, 8, 1024, 64), (500, 64, 6, 512, 96), (900, 128, 8, 1024, 128)]  # T, E, k, H, I
    cases = []
    for n, (T, E, k, H, I) in enumerate(shapes):
        cfg = inputs.Config(f"streams{n}", T=T, H=H, E=E, k=k, I=I)
        cases.append((cfg, inputs.make_inputs(cfg, 30 + n)))
    _log("[streams] " + ", ".join(inputs.describe(c) for c, _ in cases))
    streams = [torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)]
    dev_in = [{key: G.to_dev(inp[key], dev) for key in ("logits", "x", "h", "y")} for _, inp in cases]
    torch.cuda.synchronize()
    results = []
    for it in range(4):
        for n, (cfg, _) in enumerate(cases):
            with torch.cuda.stream(streams[(it + n) % 2]):
                d = dev_in[n]
                r = mg.route_expand(d["logits"], cfg.k, d["x"])
                act = mg.swiglu(d["h"])
                out = mg.combine(d["y"], r["topk_weights"], r["dest_of_src"])
                results.append((n, r, act, out))
    torch.cuda.synchronize()
    refs = [oracle_lib.path(inp) for _, inp in cases]
    for n, r, act, out in results:
        cfg, ref = cases[n][0], refs[n]
        got = G.route_host(r)
        compare.assert_route_equal(got, ref, f"streams {cfg.name}")
        compare.assert_equal(got["x_expanded"], ref["x_expanded"], f"streams {cfg.name} x_expanded")
        compare.assert_bf16_close(G.to_host(act), ref["act"], f"streams {cfg.name} act")
        compare.assert_bf16_close(G.to_host(out), ref["out"], f"streams {cfg.name} out")
