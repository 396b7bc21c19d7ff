"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each pin takes an ``oracle.Oracle`` (the real library, or a planted mutant
built by the mutation test) and returns a list of failure messages; an empty
list means the pin holds.  The pins are:

* hand-worked routing cases (tests/golden/route_handworked.json);
* pure-Python brute force on tiny inputs (tests/bruteforce.py);
* closed forms and invariants that the mathematics fixes:
  - softmax weights: sum to 1 and log(w_i) - log(w_j) = key_i - key_j;
  - selection: every selected key >= every unselected key, ties to lower index;
  - maps: a bijection on [0, R), stable inside each expert's segment;
  - expand then combine with identity experts returns x bit for bit;
  - SwiGLU: gate = 0 gives 0, silu(g) - silu(-g) = g, limits at +-inf,
    linearity in u, and SciPy's own logistic function over every finite
    bf16 gate value;
  - bf16 rounding: torch's fp32 -> bf16 conversion on fp32 inputs, exact
    table search on fp64 inputs, and the special values.
"""
from __future__ import annotations

import json
import os

import numpy as np

import bruteforce as bf

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(tag: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([20260, tag]))


def _bf16_vals(bits) -> np.ndarray:
    return bf.bf16_to_float(bits)


def _rand_bf16(rng, shape, scale=1.0) -> np.ndarray:
    v = (rng.standard_normal(shape) * scale).astype(np.float32)
    return bf.bf16_round_exact_np(v.astype(np.float64))


# ===================================================================== route
def pin_route_golden(o) -> list:
    fails = []
    with open(os.path.join(GOLDEN, "route_handworked.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        logits = np.array(c["logits"], np.float32)
        bias = None if c["bias"] is None else np.array(c["bias"], np.float32)
        r = o.route(logits, c["k"], bias)
        for key in ("topk_ids", "expert_counts", "expert_offsets", "dest_of_src", "src_of_dest"):
            want = np.array(c[key]).reshape(-1)
            if not np.array_equal(r[key].reshape(-1), want):
                fails.append(f"golden {c['name']}: {key} {r[key].reshape(-1).tolist()} != {want.tolist()}")
        w_want = np.array(c["topk_weights"], np.float64)
        if not np.allclose(r["topk_weights"], w_want, rtol=1e-6, atol=1e-7):
            fails.append(f"golden {c['name']}: weights {r['topk_weights'].tolist()} != {w_want.tolist()}")
    return fails


def _tiny_route_cases():
    rng = _rng(1)
    cases = []
    for E in range(1, 7):
        for k in range(1, E + 1):
            T = 5
            cases.append((rng.standard_normal((T, E)).astype(np.float32), k, None))
            cases.append((rng.integers(-2, 3, (T, E)).astype(np.float32), k, None))  # many ties
    # bias, signed zeros, all-equal rows
    cases.append((rng.standard_normal((7, 8)).astype(np.float32), 3,
                  (0.5 * rng.standard_normal(8)).astype(np.float32)))
    z = np.where(rng.integers(0, 2, (6, 6)) == 0, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
    cases.append((z, 2, None))
    cases.append((np.full((4, 6), 0.75, np.float32), 4, None))
    return cases


def pin_route_bruteforce(o) -> list:
    fails = []
    for logits, k, bias in _tiny_route_cases():
        T, E = logits.shape
        r = o.route(logits, k, bias)
        ids_bf = bf.route_ids(logits, k, bias)
        if not np.array_equal(r["topk_ids"], ids_bf):
            fails.append(f"brute force ids T={T} E={E} k={k}: {r['topk_ids'].tolist()} != {ids_bf.tolist()}")
            continue
        counts, offsets, dest = bf.counts_offsets_dest(ids_bf, E)
        for key, want in (("expert_counts", counts), ("expert_offsets", offsets), ("dest_of_src", dest)):
            if not np.array_equal(r[key], want):
                fails.append(f"brute force {key} E={E} k={k}: {r[key].tolist()} != {want.tolist()}")
        src = np.empty_like(dest)
        src[dest] = np.arange(dest.size, dtype=np.int32)
        if not np.array_equal(r["src_of_dest"], src):
            fails.append(f"brute force src_of_dest E={E} k={k}")
    return fails


def _keys(logits, bias):
    return logits.astype(np.float32) + (bias.astype(np.float32) if bias is not None else np.float32(0))


def check_route_properties(logits, k, bias, r) -> list:
    """Properties any correct routing satisfies (used for the oracle here and
    for sampled checks elsewhere)."""
    fails = []
    T, E = logits.shape
    ids, w = r["topk_ids"], r["topk_weights"].astype(np.float64)
    keys = _keys(logits, bias).astype(np.float64)
    for t in range(T):
        sel = [int(e) for e in ids[t]]
        if len(set(sel)) != k or min(sel) < 0 or max(sel) >= E:
            fails.append(f"row {t}: ids not k distinct experts: {sel}")
            continue
        ks = keys[t, sel]
        if np.any(np.diff(ks) > 0):
            fails.append(f"row {t}: slots not in descending key order")
        for a in range(k - 1):  # equal keys inside the selection: lower index first
            if ks[a] == ks[a + 1] and sel[a] > sel[a + 1]:
                fails.append(f"row {t}: tie inside selection not in index order")
        unsel = [e for e in range(E) if e not in sel]
        if unsel:
            mx = keys[t, unsel].max()
            if ks.min() < mx:
                fails.append(f"row {t}: an unselected key beats a selected one")
            elif ks.min() == mx:
                tied_sel = [e for e in sel if keys[t, e] == mx]
                tied_un = [e for e in unsel if keys[t, e] == mx]
                if max(tied_sel) > min(tied_un):
                    fails.append(f"row {t}: boundary tie not broken toward the lower index")
        s = w[t].sum()
        if abs(s - 1.0) > 1e-6:
            fails.append(f"row {t}: weights sum {s}")
        if np.any(w[t] <= 0):
            # exp underflow to zero needs key gaps > 100; not in these inputs
            fails.append(f"row {t}: non-positive weight")
            continue
        lw = np.log(w[t])
        d = (lw - lw[0]) - (ks - ks[0])
        if np.max(np.abs(d)) > 2e-6 * max(1.0, np.max(np.abs(ks - ks[0]))):
            fails.append(f"row {t}: log-weight differences != key differences (max dev {np.max(np.abs(d))})")
    return fails


def check_maps(ids, E, r) -> list:
    fails = []
    ids = np.asarray(ids).reshape(-1)
    R = ids.size
    counts, offsets = r["expert_counts"], r["expert_offsets"]
    dest, src = r["dest_of_src"].reshape(-1), r["src_of_dest"].reshape(-1)
    if counts.sum() != R:
        fails.append(f"counts sum {counts.sum()} != R {R}")
    if offsets[0] != 0 or offsets[E] != R or np.any(np.diff(offsets) != counts):
        fails.append("offsets are not the exclusive prefix sum of counts")
    if not np.array_equal(np.bincount(ids, minlength=E)[:E], counts):
        fails.append("counts != histogram of ids")
    if R and not np.array_equal(np.sort(dest), np.arange(R)):
        fails.append("dest_of_src is not a permutation of [0,R)")
        return fails
    if R and not np.array_equal(src[dest], np.arange(R)):
        fails.append("src_of_dest is not the inverse of dest_of_src")
    seg = np.searchsorted(offsets, dest, side="right") - 1
    if R and not np.array_equal(seg, ids):
        fails.append("a row lies outside its expert's segment")
    if R:  # inside each segment, source slots ascend
        for e in range(E):
            sl = src[offsets[e]:offsets[e + 1]]
            if np.any(np.diff(sl) <= 0):
                fails.append(f"segment of expert {e} is not in ascending slot order")
                break
    return fails


def pin_route_properties(o) -> list:
    fails = []
    rng = _rng(2)
    for (T, E, k, with_bias) in ((64, 8, 2, False), (40, 128, 8, False), (33, 256, 8, True), (50, 64, 6, False),
                                 (20, 17, 5, True), (30, 512, 16, False)):
        logits = rng.standard_normal((T, E)).astype(np.float32)
        bias = (0.5 * rng.standard_normal(E)).astype(np.float32) if with_bias else None
        r = o.route(logits, k, bias)
        fails += check_route_properties(logits, k, bias, r)
        fails += check_maps(r["topk_ids"], E, r)
    # closed forms: k=1 -> weight exactly 1; all-equal keys -> ids 0..k-1, weights 1/k
    r = o.route(rng.standard_normal((9, 12)).astype(np.float32), 1)
    if not np.all(r["topk_weights"] == 1.0):
        fails.append("k=1 weights are not exactly 1")
    r = o.route(np.full((3, 10), -2.5, np.float32), 4)
    if not (np.all(r["topk_ids"] == np.arange(4)) and np.allclose(r["topk_weights"], 0.25, rtol=0, atol=1e-7)):
        fails.append("all-equal keys: ids != 0..k-1 or weights != 1/k")
    # k=E -> the ids of a row are all experts sorted by key (desc, index asc)
    lg = rng.integers(-3, 4, (6, 7)).astype(np.float32)
    r = o.route(lg, 7)
    for t in range(6):
        want = sorted(range(7), key=lambda e: (-float(lg[t, e]), e))
        if r["topk_ids"][t].tolist() != want:
            fails.append(f"k=E row {t}: {r['topk_ids'][t].tolist()} != {want}")
    # T = 0 is a valid empty batch
    r = o.route(np.zeros((0, 5), np.float32), 2)
    if r["expert_offsets"].tolist() != [0] * 6:
        fails.append("T=0: offsets not all zero")
    return fails


def pin_route_padded(o) -> list:
    """Padded segments: brute-force constructive layout on tiny inputs;
    pad_to = 1 reproduces the unpadded route; segment invariants."""
    fails = []
    rng = _rng(8)
    for (T, E, k, M) in ((5, 4, 2, 1), (5, 4, 2, 4), (7, 6, 3, 3), (9, 8, 2, 16), (3, 5, 5, 2), (0, 4, 2, 8),
                         (12, 3, 1, 5)):
        logits = rng.standard_normal((T, E)).astype(np.float32)
        r = o.route_padded(logits, k, M)
        ids_bf = bf.route_ids(logits, k) if T else np.zeros((0, k), np.int32)
        offs, dest, src = bf.padded_layout(ids_bf, E, M)
        for key, want in (("expert_offsets", offs), ("dest_of_src", dest), ("src_of_dest", src)):
            if not np.array_equal(r[key], want):
                fails.append(f"padded brute force T={T} E={E} k={k} M={M}: {key} {r[key].tolist()} != {want.tolist()}")
        cnt = r["expert_counts"]
        seg = np.diff(r["expert_offsets"])
        if np.any(seg % M) or np.any(seg < cnt) or np.any(seg - cnt >= M):
            fails.append(f"padded segments T={T} E={E} k={k} M={M}: lengths {seg.tolist()} counts {cnt.tolist()}")
        if int((r["src_of_dest"] == -1).sum()) != int(seg.sum() - cnt.sum()):
            fails.append(f"padded T={T} M={M}: padding rows are not all -1")
    # pad_to = 1 is the unpadded route
    logits = rng.standard_normal((40, 16)).astype(np.float32)
    a, b = o.route_padded(logits, 4, 1), o.route(logits, 4)
    for key in ("topk_ids", "expert_offsets", "expert_counts", "dest_of_src", "src_of_dest"):
        if not np.array_equal(a[key], b[key]):
            fails.append(f"pad_to=1 differs from the unpadded route in {key}")
    return fails


# ===================================================================== expand
def pin_expand(o) -> list:
    fails = []
    rng = _rng(3)
    for (T, H, E, k) in ((13, 16, 8, 2), (9, 24, 5, 5), (20, 8, 64, 6), (1, 40, 3, 1)):
        x = _rand_bf16(rng, (T, H))
        r = o.route(rng.standard_normal((T, E)).astype(np.float32), k)
        xe = o.expand_rows(x, r["dest_of_src"], k)
        d = r["dest_of_src"]
        for s in range(T * k):
            if not np.array_equal(xe[d[s]], x[s // k]):
                fails.append(f"expand T={T} H={H} k={k}: row {d[s]} != x[{s // k}]")
                break
        if not np.array_equal(xe, x[r["src_of_dest"] // k]):
            fails.append(f"expand T={T}: x_exp[p] != x[src_of_dest[p] / k]")
    return fails


# ===================================================================== SwiGLU
_FINITE_BF16 = np.array([b for b in range(0x10000) if (b & 0x7F80) != 0x7F80], dtype=np.uint16)


def _swiglu_rows(o, gate_bits, up_bits):
    """Run the oracle with one row per value pair (I=1), return act bits."""
    h = np.stack([gate_bits, up_bits], axis=1).astype(np.uint16)
    return o.swiglu(h).reshape(-1)


def pin_swiglu_layout_and_identities(o) -> list:
    fails = []
    rng = _rng(4)
    R, I = 6, 16
    # gate (first I columns) = 0 -> output 0 whatever up holds; up = 0 -> output 0
    h = _rand_bf16(rng, (R, 2 * I))
    h0 = h.copy()
    h0[:, :I] = 0
    if np.any(_bf16_vals(o.swiglu(h0)) != 0):
        fails.append("swiglu: gate = 0 (first half) does not give 0")
    h1 = h.copy()
    h1[:, I:] = 0
    if np.any(_bf16_vals(o.swiglu(h1)) != 0):
        fails.append("swiglu: up = 0 (second half) does not give 0")
    # linearity in up: doubling up doubles the output exactly (power-of-two scaling)
    up2 = bf.bf16_round_exact_np(2.0 * _bf16_vals(h[:, I:]))
    h2 = h.copy()
    h2[:, I:] = up2
    a1, a2 = _bf16_vals(o.swiglu(h)), _bf16_vals(o.swiglu(h2))
    if not np.array_equal(2.0 * a1, a2):
        fails.append("swiglu: not linear in up")
    # silu(g) - silu(-g) = g  (u = 1), within two bf16 roundings
    g = _FINITE_BF16[(np.abs(_bf16_vals(_FINITE_BF16)) < 64) & (_bf16_vals(_FINITE_BF16) > 0)]
    one = np.full(g.shape, 0x3F80, np.uint16)
    pos = _bf16_vals(_swiglu_rows(o, g, one))
    neg = _bf16_vals(_swiglu_rows(o, g ^ np.uint16(0x8000), one))
    gv = _bf16_vals(g)
    tol = 2.0 ** -8 * (np.abs(pos) + np.abs(neg)) + 1e-38
    bad = np.abs((pos - neg) - gv) > tol
    if np.any(bad):
        i = int(np.argmax(bad))
        fails.append(f"swiglu: silu(g)-silu(-g) != g at g={gv[i]} ({pos[i]} - {neg[i]})")
    # limits: for g >= 32, silu(g) rounds to g; for g <= -128 it is a negative value below 1e-30
    big = np.array([0x4200, 0x4300, 0x4780], np.uint16)  # 32, 128, 65536
    if not np.array_equal(_swiglu_rows(o, big, np.full(3, 0x3F80, np.uint16)), big):
        fails.append("swiglu: silu(g) != g for large g")
    small = np.array([0xC300, 0xC780], np.uint16)  # -128, -65536
    sv = _bf16_vals(_swiglu_rows(o, small, np.full(2, 0x3F80, np.uint16)))
    if np.any(np.abs(sv) > 1e-30) or np.any(~np.signbit(sv)):
        fails.append(f"swiglu: silu(g) for g -> -inf is not -0/-tiny: {sv}")
    # slope 1/2 at 0: silu(g) ~= g/2 for tiny g
    tiny = np.array([0x3A80, 0xBA80], np.uint16)  # +-2^-10
    tv = _bf16_vals(_swiglu_rows(o, tiny, np.full(2, 0x3F80, np.uint16)))
    want = _bf16_vals(tiny) / 2
    if np.any(np.abs(tv - want) > 2.0 ** -8 * np.abs(want)):
        fails.append(f"swiglu: silu'(0) != 1/2: {tv} vs {want}")
    return fails


def pin_swiglu_expit_exhaustive(o) -> list:
    """Every finite bf16 gate value x u in {1, -1, 0.5, 3}: against SciPy's logistic."""
    from scipy.special import expit

    fails = []
    gv = _bf16_vals(_FINITE_BF16)
    for u_val, u_bits in ((1.0, 0x3F80), (-1.0, 0xBF80), (0.5, 0x3F00), (3.0, 0x4040)):
        got = _swiglu_rows(o, _FINITE_BF16, np.full(_FINITE_BF16.shape, u_bits, np.uint16))
        ref = gv * expit(gv) * u_val
        want = bf.bf16_round_exact_np(ref)
        bad = got != want
        if np.any(bad):
            # a mismatch is only acceptable if the fp64 value sits on a rounding midpoint
            gvb, wv = _bf16_vals(got[bad]), _bf16_vals(want[bad])
            mid = 0.5 * (gvb + wv)
            near = np.abs(ref[bad] - mid) <= 1e-12 * np.abs(ref[bad])
            if not np.all(near):
                i = int(np.argmax(~near))
                fails.append(f"swiglu vs expit u={u_val}: {int(np.sum(~near))} mismatches, e.g. g={gv[bad][i]} "
                             f"got {gvb[i]} want {wv[i]}")
    return fails


# ===================================================================== combine
def pin_combine_identity(o) -> list:
    """Identity experts: combine(expand(x), w) == x exactly (sum w = 1 to
    within k fp32 ulps, far below half a bf16 ulp).  Compared as values: the
    sum starts from +0, so a -0 in x comes back as +0."""
    fails = []
    rng = _rng(5)
    for (T, H, E, k) in ((17, 32, 8, 2), (12, 16, 128, 8), (10, 24, 64, 6), (8, 8, 4, 4), (6, 16, 9, 1)):
        x = _rand_bf16(rng, (T, H))
        r = o.route(rng.standard_normal((T, E)).astype(np.float32), k)
        y = o.expand_rows(x, r["dest_of_src"], k)
        out = o.combine(y, r["topk_weights"], r["dest_of_src"])
        if not np.array_equal(_bf16_vals(out), _bf16_vals(x)):  # -0 in x may come back as +0
            fails.append(f"combine(expand(x)) != x for T={T} H={H} E={E} k={k}")
        # doubling the weights doubles the output exactly
        out2 = o.combine(y, 2 * r["topk_weights"], r["dest_of_src"])
        if not np.array_equal(_bf16_vals(out2), 2 * _bf16_vals(x)):
            fails.append(f"combine not linear in w for T={T} k={k}")
    return fails


def pin_combine_bruteforce(o) -> list:
    fails = []
    rng = _rng(6)
    for (T, H, E, k) in ((5, 8, 6, 3), (4, 16, 8, 2), (3, 8, 16, 8)):
        r = o.route(rng.standard_normal((T, E)).astype(np.float32), k)
        y = _rand_bf16(rng, (T * k, H))
        w = (np.abs(rng.standard_normal((T, k))) + 0.1).astype(np.float32)  # not normalised on purpose
        got = o.combine(y, w, r["dest_of_src"])
        want, exact = bf.combine_exact(y, w, r["dest_of_src"])
        bad = np.argwhere(got != want)
        for t, c in bad:
            # fp64 summation may only differ from the exact sum right at a midpoint
            s = exact[t][c]
            gv, wv = float(_bf16_vals(got[t, c])), float(_bf16_vals(want[t, c]))
            if abs(float(s) - 0.5 * (gv + wv)) > 1e-12 * abs(float(s)):
                fails.append(f"combine brute force T={T} k={k} at ({t},{c}): got {gv} want {wv}")
                break
    return fails


# ===================================================================== bf16
def pin_bf16_rounding(o) -> list:
    import torch

    fails = []
    rng = _rng(7)
    # (1) fp32 inputs: torch's fp32 -> bf16 (round to nearest even) is a library routine
    f = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-39).astype(np.float32),            # fp32 subnormals
        (np.clip(rng.standard_normal(2000), -3.3, 3.3) * 1e38).astype(np.float32),  # near overflow
        np.array([0.0, -0.0, 1.0, -1.0, 1.00390625, 1.01171875, 3.3895314e38, 3.3961776e38], np.float32),
        (np.arange(1, 2000, dtype=np.uint32) | np.uint32(0x3F800000)).view(np.float32),  # 1 + tiny ulps
        ((np.arange(0, 4000, dtype=np.uint32) << 15) | np.uint32(0x3F808000)).view(np.float32),  # exact halves
    ]).astype(np.float32)
    f = f[np.isfinite(f)]
    got = o.bf16_from_f64(f.astype(np.float64))
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    if not np.array_equal(got, want):
        i = int(np.argmax(got != want))
        fails.append(f"bf16 rounding vs torch at {f[i]!r}: {got[i]:#06x} != {want[i]:#06x}")
    # (2) fp64 inputs that fp32 cannot hold: exact table search
    d = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-40, 38, 20000),
                        1.0 + (2 * rng.integers(0, 128, 500) + 1) * 2.0 ** -8 + 2.0 ** -40])
    got = o.bf16_from_f64(d)
    want = bf.bf16_round_exact_np(d)
    if not np.array_equal(got, want):
        i = int(np.argmax(got != want))
        fails.append(f"bf16 rounding vs exact at {d[i]!r}: {got[i]:#06x} != {want[i]:#06x}")
    # (3) specials
    specials = {float("inf"): 0x7F80, float("-inf"): 0xFF80, 3.5e38: 0x7F80, -3.5e38: 0xFF80, -0.0: 0x8000,
                2.0 ** -133: 0x0001, 2.0 ** -134: 0x0000, 1.5 * 2.0 ** -133: 0x0002, 2.0 ** -126: 0x0080}
    for v, b in specials.items():
        g = int(o.bf16_from_f64(np.array([v]))[0])
        if g != b:
            fails.append(f"bf16 special {v!r}: {g:#06x} != {b:#06x}")
    nan = int(o.bf16_from_f64(np.array([float("nan")]))[0])
    if (nan & 0x7F80) != 0x7F80 or (nan & 0x7F) == 0:
        fails.append(f"bf16 of NaN is not a NaN: {nan:#06x}")
    # (4) bf16 -> f64 is exact on every finite pattern (round trip)
    back = o.bf16_from_f64(np.array([o.lib.moe_ref_f64_from_bf16(int(b)) for b in _FINITE_BF16[::7]]))
    if not np.array_equal(back, _FINITE_BF16[::7]):
        fails.append("bf16 -> f64 -> bf16 is not the identity")
    return fails


# ===================================================================== FP8
def _torch_e4m3(v: np.ndarray) -> np.ndarray:
    """torch's own fp32 -> float8_e4m3fn conversion (nearest-even) of clamped values."""
    import torch

    c = np.clip(np.asarray(v, np.float32), np.float32(-448.0), np.float32(448.0))
    return torch.from_numpy(c.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


_E4M3_VALUES = None


def _e4m3_table():
    """All non-negative finite e4m3 values with their codes, ascending (independent decode)."""
    global _E4M3_VALUES
    if _E4M3_VALUES is None:
        vals = []
        for code in range(0x7F):
            ex, m = code >> 3, code & 7
            vals.append(m * 2.0 ** -9 if ex == 0 else (1 + m / 8) * 2.0 ** (ex - 7))
        _E4M3_VALUES = np.array(vals)
    return _E4M3_VALUES


def pin_e4m3_rounding(o) -> list:
    fails = []
    rng = _rng(9)
    v = np.concatenate([rng.standard_normal(4000) * 10.0 ** rng.integers(-4, 3, 4000),
                        rng.uniform(-460, 460, 2000), np.array([0.0, -0.0, 448.0, 449.0, 463.0, 465.0, 1e9, -1e9,
                                                                2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -11, 2.0 ** -6])
                        ]).astype(np.float32)
    got = o.e4m3_from_f32(v)
    want = _torch_e4m3(v)
    if not np.array_equal(got, want):
        i = int(np.argmax(got != want))
        fails.append(f"e4m3 vs torch at {v[i]!r}: {got[i]:#04x} != {want[i]:#04x}")
    # exact table search: nearest e4m3 value, ties to the even code
    table = _e4m3_table()
    for x in v[:600]:
        a = min(abs(float(x)), 448.0)
        i = int(np.searchsorted(table, a, side="right")) - 1
        lo, hi = table[i], table[min(i + 1, len(table) - 1)]
        code = i if (a - lo < hi - a or (a - lo == hi - a and i % 2 == 0) or i == len(table) - 1) else i + 1
        code |= 0x80 if np.signbit(x) else 0
        g = int(o.e4m3_from_f32(np.array([x]))[0])
        if g != code:
            fails.append(f"e4m3 vs table at {x!r}: {g:#04x} != {code:#04x}")
            break
    # every finite code decodes and re-encodes to itself
    for code in list(range(0x7F)) + list(range(0x80, 0xFF)):
        back = int(o.e4m3_from_f32(np.array([o.lib.moe_ref_f64_from_e4m3(code)]))[0])
        if back != code:
            fails.append(f"e4m3 code {code:#04x} does not round-trip ({back:#04x})")
            break
    return fails


def _round_sig24(v: np.ndarray) -> np.ndarray:
    """v (float64) rounded to a 24-bit significand, nearest-even, with no
    exponent limits: the significand from frexp goes through float32 (in
    [0.5, 1) it is always normal), the exponent is put back in float64."""
    m, e = np.frexp(np.asarray(v, np.float64))
    return np.ldexp(m.astype(np.float32).astype(np.float64), e)


def _bruteforce_expand_fp8(x_bits, dest, k, group, rows):
    """The FP8 reading with fp32 roundings and no exponent limits: inv =
    448/amax to 24 bits, the product x * inv to 24 bits (exact in float64
    before that rounding), clamped, then torch's own E4M3 conversion."""
    T, H = x_bits.shape
    G = H // group
    xv = bf.bf16_to_float(x_bits).astype(np.float64)
    q = np.zeros((rows, H), np.uint8)
    sc = np.zeros((rows, G), np.float32)
    for t in range(T):
        for g in range(G):
            seg = xv[t, g * group:(g + 1) * group]
            amax = np.max(np.abs(seg))
            scale = np.float32(np.float32(amax) / np.float32(448.0))
            inv = _round_sig24(448.0 / amax) if amax > 0 else 0.0
            prod = np.clip(_round_sig24(seg * inv), -448.0, 448.0)
            codes = _torch_e4m3(prod.astype(np.float32))
            for j in range(k):
                d = dest[t * k + j]
                q[d, g * group:(g + 1) * group] = codes
                sc[d, g] = scale
    return q, sc


def _tiny_groups(x_bits, group):
    """Rows 1 and 2 of x: groups whose maximum is tiny -- row 1 alternates
    groups of about 1e-37 (below 448/FLT_MAX, where 448/amax overflows fp32)
    and of about 1e-25 (below 2^-64, no overflow), row 2 holds bf16
    subnormals (magnitudes 2^-133 and up), signs mixed."""
    T, H = x_bits.shape
    rng = np.random.default_rng(99)
    if T > 1:
        mag = np.where((np.arange(H) // group) % 2 == 0, 1e-37, 1e-25)
        x_bits[1] = bf.bf16_round_exact_np(rng.standard_normal(H) * mag)
    if T > 2:
        sub = rng.integers(1, 0x80, H).astype(np.uint16)  # subnormal magnitudes, 1..127 quanta of 2^-133
        x_bits[2] = sub | (rng.integers(0, 2, H).astype(np.uint16) << 15)
    return x_bits


def pin_expand_fp8(o) -> list:
    fails = []
    rng = _rng(10)
    for (T, H, E, k, group) in ((5, 32, 8, 2, 8), (4, 64, 6, 3, 16), (3, 128, 4, 4, 128), (6, 48, 5, 1, 16)):
        x = _rand_bf16(rng, (T, H), scale=3.0)
        x = _tiny_groups(x, group)
        x[0, :group] = 0  # an all-zero group
        r = o.route(rng.standard_normal((T, E)).astype(np.float32), k)
        q, sc = o.expand_rows_fp8(x, r["dest_of_src"], k, group)
        qb, scb = _bruteforce_expand_fp8(x, r["dest_of_src"], k, group, T * k)
        if not np.array_equal(q, qb):
            fails.append(f"fp8 expand codes differ from brute force T={T} H={H} group={group}")
        if not np.array_equal(sc, scb):
            fails.append(f"fp8 expand scales differ from brute force T={T} H={H} group={group}")
        # properties: the group maximum maps to +-448; dequantised values within half an e4m3 step
        d0 = r["dest_of_src"][0]
        if np.any(q[d0, :group] != 0) or sc[d0, 0] != 0:
            fails.append("fp8 expand: an all-zero group is not all-zero codes with scale 0")
        deq = np.array([[o.lib.moe_ref_f64_from_e4m3(int(c)) for c in row] for row in q]) * \
            np.repeat(sc.astype(np.float64), group, axis=1)
        for s in range(T * k):
            t, dd = s // k, r["dest_of_src"][s]
            ref = bf.bf16_to_float(x[t])
            err = np.abs(deq[dd] - ref)
            lim = np.maximum(np.abs(ref) * 2.0 ** -4, 2.0 ** -10 * np.repeat(sc[dd], group)) * (1 + 1e-6)
            if np.any(err > lim):
                fails.append(f"fp8 expand: dequantised error above half a step (T={T} group={group})")
                break
    return fails


def _bruteforce_expand_mxfp8(x_bits, dest, k, rows):
    """Per block of 32: the smallest power-of-two scale 2^e with amax / 2^e < 512
    found by halving and doubling (no logarithm), codes by torch's own E4M3
    conversion of x / 2^e after the +-448 clamp."""
    T, H = x_bits.shape
    B = H // 32
    xv = bf.bf16_to_float(x_bits).astype(np.float64)
    q = np.zeros((rows, H), np.uint8)
    sc = np.zeros((rows, B), np.uint8)
    for t in range(T):
        for b in range(B):
            seg = xv[t, 32 * b:32 * (b + 1)]
            amax = float(np.max(np.abs(seg)))
            e = -127
            if amax > 0:
                e = 0
                while amax / 2.0 ** e >= 512.0:
                    e += 1
                while amax / 2.0 ** e < 256.0 and e > -127:
                    e -= 1
            codes = _torch_e4m3((seg / 2.0 ** e).astype(np.float32))
            for j in range(k):
                d = dest[t * k + j]
                q[d, 32 * b:32 * (b + 1)] = codes
                sc[d, b] = e + 127
    return q, sc


def pin_expand_mxfp8(o) -> list:
    fails = []
    rng = _rng(12)
    for (T, H, E, k) in ((5, 64, 8, 2), (4, 96, 6, 3), (3, 256, 4, 4), (6, 32, 5, 1)):
        x = _rand_bf16(rng, (T, H), scale=3.0)
        # magnitudes spread over many binades, one block per token
        for t in range(T):
            x[t, 32 * (t % (H // 32)):32 * (t % (H // 32) + 1)] = _rand_bf16(
                rng, (32,), scale=float(10.0 ** rng.integers(-6, 5)))
        x[0, :32] = 0                                      # an all-zero block
        x[1, :32] = bf.bf16_round_exact_np(np.full(32, 1.875))  # saturates: 1.875 * 2^8 > 448
        x[2, -32:] = bf.bf16_round_exact_np(np.full(32, 0.25))  # exact power of two
        x[2, -31] = bf.bf16_round_exact_np(np.array([3e-6]))[0]  # tiny beside its block maximum: a subnormal code
        r = o.route(rng.standard_normal((T, E)).astype(np.float32), k)
        q, sc = o.expand_rows_mxfp8(x, r["dest_of_src"], k)
        qb, scb = _bruteforce_expand_mxfp8(x, r["dest_of_src"], k, T * k)
        if not np.array_equal(q, qb):
            fails.append(f"mxfp8 expand codes differ from brute force T={T} H={H}")
        if not np.array_equal(sc, scb):
            fails.append(f"mxfp8 expand scale bytes differ from brute force T={T} H={H}")
        # format properties, from the OCP MX definition: 2^(byte - 127) is a
        # power-of-two scale with amax / scale in [256, 512); zero blocks get byte 0
        xv = bf.bf16_to_float(x).astype(np.float64)
        for s in range(T * k):
            t, d = s // k, r["dest_of_src"][s]
            for b in range(H // 32):
                seg = xv[t, 32 * b:32 * (b + 1)]
                amax = float(np.max(np.abs(seg)))
                scale = 2.0 ** (int(sc[d, b]) - 127)
                if amax == 0:
                    if sc[d, b] != 0 or np.any(q[d, 32 * b:32 * (b + 1)] != 0):
                        fails.append("mxfp8 expand: an all-zero block is not byte 0 with zero codes")
                    continue
                if not (256.0 <= amax / scale < 512.0):
                    fails.append(f"mxfp8 expand: amax/scale = {amax / scale} outside [256, 512)")
                    break
                vals = np.array([o.lib.moe_ref_f64_from_e4m3(int(c)) for c in q[d, 32 * b:32 * (b + 1)]])
                scaled = seg / scale
                sat = np.abs(scaled) > 448.0
                if np.any(np.abs(vals[sat]) != 448.0):
                    fails.append("mxfp8 expand: a value beyond 448 after scaling does not saturate")
                ok = ~sat
                lim = np.maximum(np.abs(scaled[ok]) * 2.0 ** -4, 2.0 ** -10) * (1 + 1e-9)
                if np.any(np.abs(vals[ok] - scaled[ok]) > lim):
                    fails.append("mxfp8 expand: a code is more than half an E4M3 step from x / scale")
                    break
    return fails


ALL_PINS = [
    pin_route_golden,
    pin_route_bruteforce,
    pin_route_properties,
    pin_route_padded,
    pin_expand,
    pin_e4m3_rounding,
    pin_expand_fp8,
    pin_expand_mxfp8,
    pin_swiglu_layout_and_identities,
    pin_swiglu_expit_exhaustive,
    pin_combine_identity,
    pin_combine_bruteforce,
    pin_bf16_rounding,
]


def run_all(o) -> dict:
    out = {}
    for p in ALL_PINS:
        try:
            out[p.__name__] = p(o)
        except Exception as ex:  # a crash in a mutant counts as a caught mistake
            out[p.__name__] = [f"exception: {type(ex).__name__}: {ex}"]
    return out


__all__ = ["ALL_PINS", "run_all", "check_route_properties", "check_maps"]
