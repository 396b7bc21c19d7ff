"""Planted mistakes in the oracle must be caught by its pins.

Each mutant is the oracle's C source with one plausible mistake written in (a
dropped term, a wrong sign, a wrong index, a transposed operand, a broken tie
rule or rounding), compiled on the CPU into a temporary library.  The pins of
tests/pins.py must report at least one failure for every mutant; this is what
shows the pins can see the kind of mistake they are meant to catch.  A mutant
that the pins drive out of bounds (the pin runner dies with a signal) counts as
caught; each mutant runs in its own process for that reason.
"""
from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest

import oracle
from oracle import build as obuild
import pins

MUTANTS = [
    ("select_smallest",
     "if (a->key > b->key) return -1;\n    if (a->key < b->key) return 1;",
     "if (a->key < b->key) return -1;\n    if (a->key > b->key) return 1;"),
    ("tie_to_higher_index",
     "return (a->expert > b->expert) - (a->expert < b->expert);",
     "return (a->expert < b->expert) - (a->expert > b->expert);"),
    ("bias_dropped", "if (bias) key = key + bias[e];", "(void)bias;"),
    ("bias_subtracted", "if (bias) key = key + bias[e];", "if (bias) key = key - bias[e];"),
    ("softmax_over_all_experts",
     "for (int j = 0; j < k; ++j) denom += exp((double)row[j].key - top);",
     "for (int j = 0; j < E; ++j) denom += exp((double)row[j].key - top);"),
    ("weight_exp_sign",
     "topk_weights[(size_t)t * k + j] = (float)(exp((double)row[j].key - top) / denom);",
     "topk_weights[(size_t)t * k + j] = (float)(exp(top - (double)row[j].key) / denom);"),
    ("weights_unnormalised",
     "topk_weights[(size_t)t * k + j] = (float)(exp((double)row[j].key - top) / denom);",
     "topk_weights[(size_t)t * k + j] = (float)(exp((double)row[j].key - top));"),
    ("selection_off_by_one",
     "topk_ids[(size_t)t * k + j] = row[j].expert;",
     "topk_ids[(size_t)t * k + j] = row[(j + 1) % E].expert;"),
    ("histogram_drops_last_slot",
     "for (int64_t s = 0; s < R; ++s) expert_counts[topk_ids[s]] += 1;",
     "for (int64_t s = 0; s + 1 < R; ++s) expert_counts[topk_ids[s]] += 1;"),
    ("scan_index_off_by_one",
     "expert_offsets[e + 1] = expert_offsets[e] + expert_counts[e];",
     "expert_offsets[e + 1] = expert_offsets[e] + expert_counts[e + 1 < E ? e + 1 : e];"),
    ("segment_order_reversed",
     "for (int e = 0; e < E; ++e) cursor[e] = expert_offsets[e];",
     "for (int e = 0; e < E; ++e) cursor[e] = expert_offsets[e + 1] - 1;",
     "cursor[e] += 1;", "cursor[e] -= 1;"),
    ("src_of_dest_not_inverted",
     "for (int64_t s = 0; s < R; ++s) src_of_dest[dest_of_src[s]] = (int32_t)s;",
     "for (int64_t s = 0; s < R; ++s) src_of_dest[s] = dest_of_src[s];"),
    ("padding_always_adds_a_tile",
     "const int64_t padded = (int64_t)pad_to * ((expert_counts[e] + pad_to - 1) / pad_to);",
     "const int64_t padded = (int64_t)pad_to * (expert_counts[e] / pad_to + 1);"),
    ("padding_rows_not_marked",
     "for (int64_t p = 0; p < expert_offsets[E]; ++p) src_of_dest[p] = -1;",
     "for (int64_t p = 0; p < 0; ++p) src_of_dest[p] = -1;"),
    ("padded_placement_uses_plain_offsets",
     "for (int e = 0; e < E; ++e) next_row[e] = expert_offsets[e];",
     "for (int e = 0; e < E; ++e) next_row[e] = plain_offsets[e];"),
    ("expand_not_permuted",
     "int64_t d = dest_of_src[(size_t)t * k + j];",
     "int64_t d = (int64_t)t * k + j;"),
    ("expand_index_transposed",
     "int64_t d = dest_of_src[(size_t)t * k + j];",
     "int64_t d = dest_of_src[(size_t)j * T + t];"),
    ("e4m3_bias_8", "return sgn | (uint8_t)(((re - 1 + 7) << 3) | mant);",
     "return sgn | (uint8_t)(((re - 1 + 8) << 3) | mant);"),
    ("e4m3_not_saturating", "if (mag > 448.0) mag = 448.0;", "(void)0;"),
    ("e4m3_subnormal_quantum", "const int qe = ex - 4 < -9 ? -9 : ex - 4;", "const int qe = ex - 4 < -10 ? -10 : ex - 4;"),
    ("e4m3_truncates", "const double rounded = ldexp(nearbyint(ldexp(mag, -qe)), qe);",
     "const double rounded = ldexp(floor(ldexp(mag, -qe)), qe);"),
    ("fp8_scale_240", "const float scale = amax / 448.0f;", "const float scale = amax / 240.0f;"),
    ("fp8_divide_by_scale", "q_out[(size_t)dst_row * H + c] = moe_ref_e4m3_from_f32(xv * inv);",
     "q_out[(size_t)dst_row * H + c] = moe_ref_e4m3_from_f32(xv / scale);"),
    ("fp8_scales_by_token", "scales[(size_t)dst_row * G + g] = scale;", "scales[(size_t)t * G + g] = scale;"),
    ("fp8_no_prescale", "const float pre = amax < 0x1p-64f ? 0x1p64f : 1.0f;", "const float pre = 1.0f;"),
    ("fp8_prescale_inverse_only", "const float xv = (float)moe_ref_f64_from_bf16(x[(size_t)t * H + c]) * pre;",
     "const float xv = (float)moe_ref_f64_from_bf16(x[(size_t)t * H + c]);"),
    ("fp8_amax_first_only",
     "for (int c = g * group; c < (g + 1) * group; ++c) {\n                float v = fabsf(",
     "for (int c = g * group; c < g * group + 1; ++c) {\n                float v = fabsf("),
    ("mx_emax_7", "e = ex - 1 - 8;", "e = ex - 1 - 7;"),
    ("mx_ceil_log2", "e = ex - 1 - 8;", "e = ex - 8;"),
    ("mx_e8m0_bias_128", "scales[(size_t)dst_row * B + b] = (uint8_t)(e + 127);",
     "scales[(size_t)dst_row * B + b] = (uint8_t)(e + 128);"),
    ("mx_scales_by_token", "scales[(size_t)dst_row * B + b] = (uint8_t)(e + 127);",
     "scales[(size_t)t * B + b] = (uint8_t)(e + 127);"),
    ("mx_zero_block_scale_one", "int e = -127;\n            if (amax > 0.0) {", "int e = 0;\n            if (amax > 0.0) {"),
    ("mx_multiplies_by_scale", "moe_ref_e4m3_from_f32((float)ldexp(xv, -e));", "moe_ref_e4m3_from_f32((float)ldexp(xv, e));"),
    ("swiglu_gate_up_swapped",
     "double g = moe_ref_f64_from_bf16(h[(size_t)r * 2 * I + i]);\n"
     "            double u = moe_ref_f64_from_bf16(h[(size_t)r * 2 * I + I + i]);",
     "double g = moe_ref_f64_from_bf16(h[(size_t)r * 2 * I + I + i]);\n"
     "            double u = moe_ref_f64_from_bf16(h[(size_t)r * 2 * I + i]);"),
    ("silu_exp_sign", "double silu = g / (1.0 + exp(-g));", "double silu = g / (1.0 + exp(g));"),
    ("sigmoid_instead_of_silu", "double silu = g / (1.0 + exp(-g));", "double silu = 1.0 / (1.0 + exp(-g));"),
    ("up_dropped", "act[(size_t)r * I + i] = moe_ref_bf16_from_f64(silu * u);",
     "act[(size_t)r * I + i] = moe_ref_bf16_from_f64(silu + 0.0 * u);"),
    ("combine_unweighted", "acc += w * moe_ref_f64_from_bf16(y[(size_t)row * H + c]);",
     "acc += (0.0 * w + 1.0) * moe_ref_f64_from_bf16(y[(size_t)row * H + c]);"),
    ("combine_not_permuted", "int64_t row = dest_of_src[(size_t)t * k + j];", "int64_t row = (int64_t)t * k + j;"),
    ("combine_weights_transposed",
     "double w = (double)topk_weights[(size_t)t * k + j];",
     "double w = (double)topk_weights[(size_t)j * T + t];"),
    ("bf16_truncates", "double r = ldexp(nearbyint(ldexp(a, -q)), q);", "double r = ldexp(floor(ldexp(a, -q)), q);"),
    ("bf16_ties_away", "double r = ldexp(nearbyint(ldexp(a, -q)), q);", "double r = ldexp(round(ldexp(a, -q)), q);"),
    ("bf16_nine_bits", "int q = e - 8;", "int q = e - 9;"),
    ("bf16_no_subnormals", "if (q < -133) q = -133;", "if (q < -126) q = -126;"),
    ("bf16_sign_dropped", "return sign | (uint16_t)(u >> 16);", "return (uint16_t)(u >> 16);"),
]


def _pairs(m):
    return list(zip(m[1::2], m[2::2]))


def test_mutant_anchors_exist():
    with open(obuild.SRC) as f:
        src = f.read()
    for m in MUTANTS:
        for old, _new in _pairs(m):
            assert src.count(old) == 1, f"mutant {m[0]}: anchor not found exactly once in moe_oracle.c"


def test_real_oracle_passes_all_pins(oracle_lib):
    fails = pins.run_all(oracle_lib)
    assert not any(fails.values()), {k: v[:3] for k, v in fails.items() if v}


_RUNNER = """
import json, sys
sys.path[:0] = [{root!r}, {tests!r}]
import oracle, pins
res = pins.run_all(oracle.Oracle({lib!r}))
print(json.dumps({{k: v[:2] for k, v in res.items()}}))
"""


@pytest.mark.parametrize("mutant", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, mutant):
    name = mutant[0]
    with open(obuild.SRC) as f:
        src = f.read()
    for old, new in _pairs(mutant):
        assert src.count(old) == 1
        src = src.replace(old, new)
    mutant_src = tmp_path / "moe_oracle_mutant.c"
    mutant_src.write_text(src)
    lib = obuild.build(str(mutant_src), str(tmp_path / f"libmut_{name}.so"), extra_flags=["-w"])
    # separate process: a planted mistake may also write out of bounds
    tests_dir = os.path.dirname(os.path.abspath(__file__))
    code = _RUNNER.format(root=os.path.dirname(tests_dir), tests=tests_dir, lib=lib)
    proc = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    if proc.returncode != 0:
        # the pins drove the mutant out of bounds (e.g. a placement past R): caught, loudly
        assert "Traceback" not in proc.stderr or "pins" not in proc.stderr, proc.stderr[-800:]
        return
    fails = json.loads(proc.stdout.strip().splitlines()[-1])
    caught = {k: v for k, v in fails.items() if v}
    assert caught, f"planted mistake '{name}' was not caught by any pin"
