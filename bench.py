"""Benchmark of the MoE glue path on one MI355X.

One step = the whole path on one batch: moe_route_expand (route, then the
expansion of the token rows) -> moe_swiglu -> moe_combine (the GEMM outputs
are seeded stand-ins already in HBM).  With --pad the first call is
moe_route_expand_padded; with --fp8-group it is moe_route_expand_fp8 (the
route and the quantising expand); with --mxfp8 it is moe_route_expand_mxfp8
(the same with E4M3 codes and one E8M0 scale byte per 32 columns).
The default workload is the Qwen3-30B-A3B-shaped prefill batch
(T=4096, H=2048, E=128, k=8, I=768).

Inputs are resident in HBM before the timed region.  Steps rotate over
several complete input/output sets, so that no step finds its inputs in the
256 MiB Infinity Cache left behind by the previous step on the same set.  The
default number of sets is sized from the token rows x: the expand reads them
through the caches (each row is wanted k times), so the copies of x together
must exceed the Infinity Cache twice over, or a step would be served by it.

Prints ONE JSON line: whole-job tokens/s, per-call device times from HIP
events recorded on the launch stream inside the timed region, the roofline of
the dominant kernel, and the CPU oracle timed on the host as a baseline.
`value` and ms_per_step come from eager calls (each pays the host's launch
cost); ms_per_step_graph is the same steps replayed from a HIP graph.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE glue tokens/sec + achieved HBM GB/s (% of MI355X peak), Qwen3-30B-A3B shape"
HBM_PEAK_GBPS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "moe_glue_amd", "csrc")
# Source files each call's kernels are built from (a traffic figure is valid
# only while these are unchanged).
_ROUTE_SOURCES = ("route.hip", "route_common.h", "fp8_common.h", "place_copy.h")
KERNEL_SOURCES = {"route": _ROUTE_SOURCES, "expand": ("expand.hip",), "expand_fp8": ("quant.hip", "fp8_common.h"),
                  "expand_mxfp8": ("quant.hip", "fp8_common.h"),
                  "swiglu": ("swiglu.hip",), "combine": ("combine.hip",),
                  "route_expand": _ROUTE_SOURCES + ("dispatch.hip", "expand.hip", "place_expand.hip"),
                  "route_expand_padded": _ROUTE_SOURCES + ("dispatch.hip", "expand.hip", "place_expand.hip"),
                  "route_expand_fp8": _ROUTE_SOURCES + ("dispatch.hip", "quant.hip"),
                  "route_expand_mxfp8": _ROUTE_SOURCES + ("dispatch.hip", "quant.hip")}


def algorithmic_bytes(cfg, fp8_group: int = 0) -> dict:
    """Bytes each call must move: every input read once, every output written once."""
    T, H, E, k, I, R = cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.R
    route = T * E * 4 + (E * 4 if cfg.bias_std > 0 else 0) + R * 4 + R * 4 + R * 4 + R * 4 + (E + 1) * 4 + E * 4
    expand = T * H * 2 + R * 4 + R * H * 2
    swiglu = R * 2 * I * 2 + R * I * 2
    combine = R * H * 2 + R * 4 + R * 4 + T * H * 2
    expand_fp8 = T * H * 2 + R * 4 + R * H + (R * (H // fp8_group) * 4 if fp8_group else 0)
    expand_mxfp8 = T * H * 2 + R * 4 + R * H + R * (H // 32)
    return {"route": route, "expand": expand, "swiglu": swiglu, "combine": combine, "route_expand": route + expand,
            "expand_mxfp8": expand_mxfp8,
            "route_expand_padded": route + expand, "expand_fp8": expand_fp8, "route_expand_fp8": route + expand_fp8,
            "route_expand_mxfp8": route + expand_mxfp8}


def source_digest(kernel: str) -> str:
    h = hashlib.sha256()
    for f in (*KERNEL_SOURCES[kernel], "device_common.h"):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def variant_name(cfg_name: str, pad_to: int = 1, fp8_group: int = 0, mxfp8: bool = False) -> str:
    """The workload's name with its layout and quantisation options, as the
    profiles name it: qwen3_30b_a3b, qwen3_30b_a3b_pad128_fp8g128, ..."""
    return (cfg_name + (f"_pad{pad_to}" if pad_to > 1 else "") + (f"_fp8g{fp8_group}" if fp8_group else "")
            + ("_mxfp8" if mxfp8 else ""))


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per step of one call from the committed rocprofv3 counter
    summary (profiles/traffic_<workload>.md, workload as variant_name gives
    it), or None when there is none or the call's sources changed since the
    counters were taken."""
    path = os.path.join(PROFILES, f"traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        text = f.read()
    start = text.find("```json")
    if start < 0:
        return None
    end = text.find("```", start + 7)
    rec = json.loads(text[start + 7:end]).get("kernels", {}).get(kernel)
    if not rec or rec.get("source_digest") != source_digest(kernel):
        return None
    return rec.get("traffic_bytes")


class HipEvent:
    """A HIP timing event recorded on the launch stream without the system-scope
    release fence a default event carries (hipEventDisableSystemFence), so the
    markers between kernels stay cheap."""

    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    @classmethod
    def hip(cls):
        if cls._hip is None:
            import ctypes

            lib = ctypes.CDLL("libamdhip64.so")
            lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._hip = lib
        return cls._hip

    def __init__(self, stream: int, flags: int = DISABLE_SYSTEM_FENCE):
        import ctypes

        self.h = ctypes.c_void_p()
        self.stream = ctypes.c_void_p(stream)
        rc = self.hip().hipEventCreateWithFlags(ctypes.byref(self.h), flags)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        self._record = self.hip().hipEventRecord

    def record(self):
        self._record(self.h, self.stream)

    def elapsed_time(self, end: "HipEvent") -> float:
        import ctypes

        ms = ctypes.c_float()
        rc = self.hip().hipEventElapsedTime(ctypes.byref(ms), self.h, end.h)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value


class Sets:
    """NSETS complete input/output sets on the device, with ctypes argument tuples."""

    def __init__(self, inp, nsets, dev, pad_to=1, fp8_group=0, mxfp8=False):
        import torch
        import moe_glue_amd as mg

        cfg = inp["cfg"]
        self.cfg = cfg
        self.lib = mg.load()
        stream = torch.cuda.current_stream(dev).cuda_stream

        def dev_bf16(a):
            return torch.from_numpy(a.view("int16")).to(dev).view(torch.bfloat16)

        base = {
            "x": dev_bf16(inp["x"]),
            "logits": torch.from_numpy(inp["logits"]).to(dev),
            "bias": None if inp["bias"] is None else torch.from_numpy(inp["bias"]).to(dev),
            "h": dev_bf16(inp["h"]),
            "y": dev_bf16(inp["y"]),
        }
        self.sets = []
        T, H, E, k, I, R = cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.R
        P = mg.padded_rows(T, E, k, pad_to) if pad_to > 1 else R  # rows of the expert-contiguous buffers
        for s in range(nsets):
            d = {key: (None if v is None else v.clone()) for key, v in base.items()}
            d.update(mg.alloc_route_outputs(T, E, k, dev))
            if pad_to > 1:
                d["src_of_dest"] = torch.empty((P,), dtype=torch.int32, device=dev)
                y = torch.empty((P, H), dtype=torch.bfloat16, device=dev)
                y[:R].copy_(d["y"])
                d["y"] = y
            d["x_exp"] = torch.empty((P, H), dtype=torch.bfloat16, device=dev)
            if fp8_group:
                d["x_exp"] = torch.empty((P, H), dtype=torch.uint8, device=dev)
                d["x_scales"] = torch.empty((P, H // fp8_group), dtype=torch.float32, device=dev)
            if mxfp8:
                d["x_exp"] = torch.empty((P, H), dtype=torch.uint8, device=dev)
                d["x_scales"] = torch.empty((P, H // 32), dtype=torch.uint8, device=dev)
            d["act"] = torch.empty((R, I), dtype=torch.bfloat16, device=dev)
            d["out"] = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
            p = lambda key: 0 if d[key] is None else d[key].data_ptr()  # noqa: E731
            route_args = (p("topk_ids"), p("topk_weights"), p("expert_offsets"), p("expert_counts"),
                          p("dest_of_src"), p("src_of_dest"), p("workspace"), d["workspace"].numel(), stream)
            d["args"] = {
                "route": ((p("logits"), p("bias"), T, E, k) + route_args if pad_to == 1
                          else (p("logits"), p("bias"), T, E, k, pad_to) + route_args),
                "route_expand": (p("logits"), p("bias"), T, E, k, p("x"), H, p("topk_ids"), p("topk_weights"),
                             p("expert_offsets"), p("expert_counts"), p("dest_of_src"), p("src_of_dest"), p("x_exp"),
                             p("workspace"), d["workspace"].numel(), stream),
                "route_expand_padded": (p("logits"), p("bias"), T, E, k, pad_to, p("x"), H, p("topk_ids"),
                                        p("topk_weights"), p("expert_offsets"), p("expert_counts"),
                                        p("dest_of_src"), p("src_of_dest"), p("x_exp"), p("workspace"),
                                        d["workspace"].numel(), stream),
                "expand": (p("x"), p("dest_of_src"), T, H, k, p("x_exp"), stream),
                "expand_fp8": ((p("x"), p("dest_of_src"), T, H, k, fp8_group, p("x_exp"), p("x_scales"), stream)
                               if fp8_group else None),
                "expand_mxfp8": ((p("x"), p("dest_of_src"), T, H, k, p("x_exp"), p("x_scales"), stream)
                                 if mxfp8 else None),
                "route_expand_mxfp8": ((p("logits"), p("bias"), T, E, k, pad_to, p("x"), H, p("topk_ids"),
                                        p("topk_weights"), p("expert_offsets"), p("expert_counts"),
                                        p("dest_of_src"), p("src_of_dest"), p("x_exp"), p("x_scales"),
                                        p("workspace"), d["workspace"].numel(), stream) if mxfp8 else None),
                "route_expand_fp8": ((p("logits"), p("bias"), T, E, k, pad_to, p("x"), H, fp8_group, p("topk_ids"),
                                      p("topk_weights"), p("expert_offsets"), p("expert_counts"), p("dest_of_src"),
                                      p("src_of_dest"), p("x_exp"), p("x_scales"), p("workspace"),
                                      d["workspace"].numel(), stream) if fp8_group else None),
                "swiglu": (p("h"), R, I, p("act"), stream),
                "combine": (p("y"), p("topk_weights"), p("dest_of_src"), T, H, k, p("out"), stream),
            }
            self.sets.append(d)
        self.fns = {"route": self.lib.moe_route if pad_to == 1 else self.lib.moe_route_padded,
                    "expand": self.lib.moe_expand_rows, "expand_fp8": self.lib.moe_expand_rows_fp8,
                    "expand_mxfp8": self.lib.moe_expand_rows_mxfp8,
                    "route_expand_mxfp8": self.lib.moe_route_expand_mxfp8,
                    "route_expand": self.lib.moe_route_expand,
                    "route_expand_padded": self.lib.moe_route_expand_padded,
                    "route_expand_fp8": self.lib.moe_route_expand_fp8, "swiglu": self.lib.moe_swiglu,
                    "combine": self.lib.moe_combine}
        # Route and expand run as one moe_route_expand(_padded, _fp8) call
        # (one launch for decode batches, destination-order expand for large
        # ones, the copy in the route's place launch in between).
        if mxfp8:
            self.calls = ["route_expand_mxfp8", "swiglu", "combine"]
        elif fp8_group:
            self.calls = ["route_expand_fp8", "swiglu", "combine"]
        elif pad_to == 1:
            self.calls = ["route_expand", "swiglu", "combine"]
        else:
            self.calls = ["route_expand_padded", "swiglu", "combine"]

    def step(self, s, events=None, stream=None):
        """One pass of the path over input set s % nsets; `stream` (a raw
        hipStream_t) replaces the stream the argument tuples were built with."""
        a = self.sets[s % len(self.sets)]["args"]
        f = self.fns
        rc = 0
        if events is not None:
            events[0].record()
        for i, name in enumerate(self.calls):
            rc |= f[name](*(a[name] if stream is None else a[name][:-1] + (stream,)))
            if events is not None:
                events[i + 1].record()
        if rc:
            raise RuntimeError(f"a MoE glue call failed: {self.lib.moe_last_error().decode()}")


INFINITY_CACHE_BYTES = 256 << 20
MAX_SETS = 256
MAX_SET_BYTES = 32 << 30


def set_bytes(cfg, pad_to=1, fp8_group=0) -> int:
    """Device bytes of one input/output set (inputs, route outputs, workspace
    upper bound, expanded rows, activation, output)."""
    T, H, E, k, I, R = cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.R
    inputs = T * H * 2 + T * E * 4 + E * 4 + R * 2 * I * 2 + R * H * 2
    route = R * 16 + (E + 1) * 4 + E * 4 + R * 8 + (T + 1) * E * 4
    rows = R + (pad_to - 1) * E if pad_to > 1 else R
    expanded = rows * H * (1 if fp8_group else 2) + (rows * (H // fp8_group) * 4 if fp8_group else 0)
    return inputs + route + expanded + R * I * 2 + T * H * 2 + (rows * H * 2 if pad_to > 1 else 0)


def default_sets(cfg, pad_to=1, fp8_group=0) -> int:
    """Input sets to rotate: the copies of x together at least twice the
    Infinity Cache, at least 4 sets, at most MAX_SETS and MAX_SET_BYTES."""
    x_bytes = cfg.T * cfg.H * 2
    want = -(-2 * INFINITY_CACHE_BYTES // max(1, x_bytes))
    fit = MAX_SET_BYTES // max(1, set_bytes(cfg, pad_to, fp8_group))
    return max(4, min(want, MAX_SETS, fit))


def rw_bytes(cfg, fp8_group: int = 0) -> dict:
    """Algorithmic bytes of each call split into (read, write)."""
    T, H, E, k, I, R = cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.R
    route = (T * E * 4 + (E * 4 if cfg.bias_std > 0 else 0), R * 4 * 4 + (E + 1) * 4 + E * 4)
    expand = (T * H * 2 + R * 4, R * H * 2)
    expand_fp8 = (T * H * 2 + R * 4, R * H + (R * (H // fp8_group) * 4 if fp8_group else 0))
    expand_mx = (T * H * 2 + R * 4, R * H + R * (H // 32))
    add = lambda a, b: (a[0] + b[0], a[1] + b[1])  # noqa: E731
    return {"route_expand": add(route, expand), "route_expand_padded": add(route, expand),
            "route_expand_fp8": add(route, expand_fp8), "route_expand_mxfp8": add(route, expand_mx),
            "swiglu": (R * 2 * I * 2, R * I * 2), "combine": (R * H * 2 + R * 8, T * H * 2)}


def mix_of(read: int, write: int) -> tuple:
    """Small whole numbers of reads and writes per lane with about the same ratio."""
    if read >= write:
        return (max(1, min(64, round(read / max(write, 1)))), 1)
    return (1, max(1, min(64, round(write / max(read, 1)))))


def _timed_launches(dev, launch, copies: int, reps: int) -> float:
    """Median device time (s) of `reps` launches, launch(i) on copy i % copies,
    each between HIP events without the system fence (as the path's calls)."""
    import torch

    stream = torch.cuda.current_stream(dev).cuda_stream
    for i in range(min(copies, 4)):
        launch(i)
    torch.cuda.synchronize()
    ev = [(HipEvent(stream), HipEvent(stream)) for _ in range(reps)]
    for i, (e0, e1) in enumerate(ev):
        e0.record()
        launch(i % copies)
        e1.record()
    torch.cuda.synchronize()
    times = sorted(e0.elapsed_time(e1) * 1e-3 for e0, e1 in ev)
    return times[len(times) // 2]


def copy_probe_gbps(dev, nbytes=1 << 30, reps=9):
    """Achievable HBM bandwidth: the library's 16 B/lane copy over 1 GiB."""
    import torch
    import moe_glue_amd as mg

    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    t = _timed_launches(dev, lambda i: mg.copy_probe(src, dst), 1, reps)
    del src, dst
    return 2 * nbytes / t / 1e9, t


MIX_PROBE_SHAPES = ((256, 1), (256, 2), (256, 4), (1024, 1), (1024, 2))  # (lanes per workgroup, KiB per wave)


def mix_probe_gbps(dev, reads: int, writes: int, nbytes=1 << 30, reps=5):
    """HBM bandwidth of a plain stream with `reads` read waves per `writes`
    write waves (moe_mix_probe, about nbytes in all, at least one cycle): the
    best over MIX_PROBE_SHAPES, each timed as the path's calls are.  Below
    twice the Infinity Cache the launches rotate over copies of the
    buffers, as the path's calls rotate over input sets, so the reads come
    from HBM there too."""
    import torch
    import moe_glue_amd as mg

    best = 0.0
    for threads, vpl in MIX_PROBE_SHAPES:
        kib = 1024 * vpl
        cycles = max(1, nbytes // ((reads + writes) * kib))
        rb, wb = cycles * reads * kib, max(cycles * writes * kib, 1024)
        copies = max(1, min(MAX_SETS, -(-2 * INFINITY_CACHE_BYTES // (rb + wb))))
        src = torch.empty(max(1, copies * rb), dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty(copies * wb, dtype=torch.uint8, device=dev)
        t = _timed_launches(dev, lambda i: mg.mix_probe(src[i * rb:] if reads else src, dst[i * wb:], cycles, reads,
                                                         writes, vpl, threads), copies, max(reps, min(copies, 64)))
        del src, dst
        best = max(best, cycles * (reads + writes) * kib / t / 1e9)
    return best


def launch_floor_us(dev, n=100):
    """Device time of one tiny kernel (a 16-byte moe_copy_probe) when kernels
    run back to back: n launches captured in a HIP graph and replayed, so the
    host's per-call cost is out of the measurement.  None if capture fails."""
    import torch
    import moe_glue_amd as mg

    try:
        lib = mg.load()
        src = torch.ones(16, dtype=torch.uint8, device=dev)
        dst = torch.empty(16, dtype=torch.uint8, device=dev)
        side = torch.cuda.Stream(device=dev)
        with torch.cuda.stream(side):
            lib.moe_copy_probe(src.data_ptr(), dst.data_ptr(), 16, side.cuda_stream)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            for _ in range(n):
                lib.moe_copy_probe(src.data_ptr(), dst.data_ptr(), 16, side.cuda_stream)
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return round(1e3 * e0.elapsed_time(e1) / (5 * n), 3)
    except Exception as ex:  # capture unsupported: report nothing rather than a wrong floor
        print(f"bench.py: launch floor not measured ({type(ex).__name__}: {ex})", file=sys.stderr)
        return None


def graph_ms_per_step(sets, dev, steps):
    """Device time per step with the host's launch cost taken out: one pass
    over every input set captured in a HIP graph on a side stream, replayed
    back to back for about `steps` steps.  None if capture fails."""
    import torch

    try:
        side = torch.cuda.Stream(device=dev)
        n = len(sets.sets)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            for s in range(n):
                sets.step(s, stream=side.cuda_stream)
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        reps = max(1, steps // n)
        t0 = time.perf_counter()
        for _ in range(reps):
            g.replay()
        torch.cuda.synchronize()
        return round(1e3 * (time.perf_counter() - t0) / (reps * n), 4)
    except Exception as ex:  # capture unsupported: report nothing rather than a wrong time
        print(f"bench.py: graph replay not measured ({type(ex).__name__}: {ex})", file=sys.stderr)
        return None


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def _cpu_leg(config: str, seed: int, leg: str, budget_s: float, max_passes: int = 400) -> dict:
    """One leg of the CPU baseline, run in this (child) process, which never
    touches the GPU: the oracle as it stands on the same seeded workload,
    whole passes for about `budget_s` seconds after one warm pass.  Leg
    "single": the plain oracle on one thread pinned to one core.  Leg "all":
    the oracle's own calls split over token and row ranges on every core
    this process may use (oracle/threaded.py; the route stays one call)."""
    import oracle
    from moe_glue_amd import inputs as I
    from oracle import threaded

    cores = sorted(os.sched_getaffinity(0))
    if leg == "single":
        os.sched_setaffinity(0, {cores[0]})
        workers = 1
        run = oracle.get().path
    else:
        workers = len(cores)
        o = oracle.get()
        run = lambda inp: threaded.path(inp, workers, o)  # noqa: E731
    cfg = I.CONFIGS[config]
    inp = I.make_inputs(cfg, seed)
    t0 = time.perf_counter()
    run(inp)  # warm: page in
    warm = time.perf_counter() - t0
    passes = max(1, min(max_passes, int(budget_s / max(warm, 1e-3))))
    t0 = time.perf_counter()
    for _ in range(passes):
        run(inp)
    total = time.perf_counter() - t0
    return {"leg": leg, "workers": workers, "passes": passes, "seconds": total, "per_pass": total / passes,
            "pinned_core": cores[0] if leg == "single" else None}


def cpu_baseline(cfg, seed, budget_s=10.0):
    """The CPU oracle timed on this host's cores in two legs, each in a child
    process (so no GPU state is involved): one thread pinned to one core, and
    every usable core.  `value` is the all-cores leg."""
    import subprocess

    legs = {}
    for leg in ("single", "all"):
        out = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-leg", leg, "--config", cfg.name,
                              "--seed", str(seed), "--cpu-budget", str(budget_s)],
                             capture_output=True, text=True, check=True)
        legs[leg] = json.loads(out.stdout.strip().splitlines()[-1])
    ab = algorithmic_bytes(cfg)
    path_bytes = ab["route"] + ab["expand"] + ab["swiglu"] + ab["combine"]
    a, s1 = legs["all"], legs["single"]
    return {"value": round(cfg.T / a["per_pass"], 1), "unit": "tokens/s", "cores": a["workers"], "kind": "oracle",
            "GBps": round(path_bytes / a["per_pass"] / 1e9, 3),
            "single_core": {"value": round(cfg.T / s1["per_pass"], 1), "unit": "tokens/s", "cores": 1,
                            "GBps": round(path_bytes / s1["per_pass"] / 1e9, 3), "pinned_core": s1["pinned_core"]},
            "sample": f"the full {cfg.name} batch (T={cfg.T}), route+expand+swiglu+combine on the CPU oracle; "
                      f"all cores: {a['workers']} threads over token/row ranges (route one call), {a['passes']} passes "
                      f"in {a['seconds']:.1f} s, {a['per_pass']:.3f} s per pass; single core (pinned to CPU "
                      f"{s1['pinned_core']}): {s1['passes']} passes in {s1['seconds']:.1f} s, {s1['per_pass']:.3f} s "
                      f"per pass; each after one warm pass; {cpu_model()}, {os.cpu_count()} logical CPUs on the host"}


# ------------------------------------------------- rocprofv3 output summaries
def _short_kernel_name(name: str) -> str:
    name = name.replace("moe::(anonymous namespace)::", "").replace("void ", "")
    return name.split("(")[0]


def summarize_trace(csv_path: str, skip: int) -> str:
    """Per-kernel dispatch durations from a rocprofv3 kernel-trace CSV: the
    first `skip` dispatches of each kernel (the warm-up steps) are dropped,
    then the median, mean, min and max over the rest, as a markdown table."""
    import csv
    import statistics

    durs = {}
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            name = _short_kernel_name(r["Kernel_Name"])
            if name.startswith("copy_probe"):  # the 1 GiB copies and the 16-byte launch-floor copies apart
                name += f" [{int(r['Grid_Size_X'])} lanes]"
            durs.setdefault(name, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    lines = ["| kernel | dispatches timed | median ns | mean ns | min ns | max ns |", "|---|---|---|---|---|---|"]
    for name, d in sorted(durs.items(), key=lambda kv: -statistics.median(kv[1])):
        d = d[skip:] if len(d) > skip else d
        lines.append(f"| `{name}` | {len(d)} | {statistics.median(d):.0f} | {statistics.mean(d):.0f} | {min(d)} | "
                     f"{max(d)} |")
    return "\n".join(lines)


# Counter passes for HBM traffic (each its own rocprofv3 run; at most 4 TCC
# counters per pass).  Every request is counted by its size, so bytes are
# exact sums, not a scale fitted to a copy.
PMC_READ = ("TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_32B_sum", "TCC_EA0_RDREQ_64B_sum", "TCC_EA0_RDREQ_128B_sum")
PMC_WRITE = ("TCC_EA0_WRREQ_sum", "TCC_EA0_WRREQ_64B_sum")
COPY_PROBE_LANES = (1 << 30) // 16  # the 1 GiB copy probe: one 16-byte vector per lane


def _pmc_dispatches(read_dir: str, write_dir: str) -> list:
    """Per-dispatch counters from the two passes, in dispatch order of the
    read pass: [(kernel, grid_size, {counter: value})]."""
    import csv
    import glob

    passes = []
    for d in (read_dir, write_dir):
        rows = {}
        for path in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
            with open(path) as f:
                for r in csv.DictReader(f):
                    key = int(r["Dispatch_Id"])
                    e = rows.setdefault(key, [_short_kernel_name(r["Kernel_Name"]), int(r["Grid_Size"]), {}])
                    e[2][r["Counter_Name"]] = float(r["Counter_Value"])
        passes.append([rows[k] for k in sorted(rows)])
    rd, wr = passes
    if [(n, g) for n, g, _ in rd] != [(n, g) for n, g, _ in wr]:
        raise RuntimeError("the read and write counter passes saw different dispatch sequences")
    return [(n, g, {**a, **b[2]}) for (n, g, a), b in zip(rd, wr)]


def pmc_request_bytes(c: dict) -> tuple:
    """(read bytes, write bytes, read requests unaccounted) of one dispatch:
    reads 32 * RDREQ_32B + 64 * RDREQ_64B + 128 * RDREQ_128B, writes
    64 * WRREQ_64B + 32 * (WRREQ - WRREQ_64B)."""
    r32, r64, r128 = (c.get(f"TCC_EA0_RDREQ_{s}_sum", 0.0) for s in ("32B", "64B", "128B"))
    rd = 32.0 * r32 + 64.0 * r64 + 128.0 * r128
    w64 = c.get("TCC_EA0_WRREQ_64B_sum", 0.0)
    wr = 64.0 * w64 + 32.0 * (c.get("TCC_EA0_WRREQ_sum", 0.0) - w64)
    return rd, wr, c.get("TCC_EA0_RDREQ_sum", 0.0) - (r32 + r64 + r128)


def pmc_bytes(read_dir: str, write_dir: str) -> dict:
    """HBM bytes per dispatch per kernel (means) from the two passes:
    {kernel: {"dispatches", "read_bytes", "write_bytes"}}; the copy probe's
    sizes apart."""
    acc = {}
    for name, grid, c in _pmc_dispatches(read_dir, write_dir):
        if name.startswith("copy_probe"):
            name = f"{name}[{grid}]"
        rd, wr, _ = pmc_request_bytes(c)
        a = acc.setdefault(name, [0, 0.0, 0.0])
        a[0] += 1
        a[1] += rd
        a[2] += wr
    return {n: {"dispatches": a[0], "read_bytes": a[1] / a[0], "write_bytes": a[2] / a[0]} for n, a in acc.items()}


def _call_of_kernel(name: str, route_call: str):
    if name.startswith("swiglu"):  # swiglu_kernel<U>, swiglu8_kernel
        return "swiglu"
    if name.startswith("combine_kernel"):
        return "combine"
    if name.startswith(("route_", "place_expand_kernel", "expand_")):
        return route_call
    return None


def traffic_report(read_dir: str, write_dir: str, cfg, pad_to=1, fp8_group=0, mxfp8=False, cmds=()) -> str:
    """Markdown summary of the two counter passes of a bench.py run: the copy
    probe's measured bytes against the 2 GiB it moves, then each call of
    the step (all the kernels it launches) against its algorithmic bytes,
    with the machine-readable block measured_traffic reads."""
    disp = _pmc_dispatches(read_dir, write_dir)
    route_call = ("route_expand_mxfp8" if mxfp8 else "route_expand_fp8" if fp8_group
                  else "route_expand" if pad_to == 1 else "route_expand_padded")
    ab = algorithmic_bytes(cfg, fp8_group)
    probe = [pmc_request_bytes(c) for n, g, c in disp if n.startswith("copy_probe") and g == COPY_PROBE_LANES]
    steps = sum(1 for n, _, _ in disp if n.startswith("swiglu"))
    per_kernel, per_call = {}, {}
    for n, _, c in disp:
        call = _call_of_kernel(n, route_call)
        if call is None:
            continue
        rd, wr, miss = pmc_request_bytes(c)
        k = per_kernel.setdefault((call, n), [0, 0.0, 0.0, 0.0])
        k[0] += 1
        k[1] += rd
        k[2] += wr
        k[3] += miss
        per_call[call] = per_call.get(call, 0.0) + rd + wr
    gib = float(1 << 30)
    lines = [f"Copy probe check (1 GiB read + 1 GiB write per dispatch, {len(probe)} dispatches): "
             + ", ".join(f"read {r / gib:.5f} GiB, write {w / gib:.5f} GiB" for r, w, _ in probe[:1])
             + (f"; unaccounted read requests {probe[0][2]:.0f}" if probe else ""), "",
             "| call | kernel | dispatches | read bytes | write bytes | HBM bytes per step | algorithmic bytes | ratio |",
             "|---|---|---|---|---|---|---|---|"]
    js = {"workload": cfg.name, "pad_to": pad_to, "fp8_group": fp8_group, "mxfp8": mxfp8, "steps": steps,
          "kernels": {}}
    for call in (route_call, "swiglu", "combine"):
        for (cl, n), k in sorted(per_kernel.items()):
            if cl == call:
                lines.append(f"| {call} | `{n}` | {k[0]} | {k[1] / k[0]:.0f} | {k[2] / k[0]:.0f} | "
                             f"{(k[1] + k[2]) / max(steps, 1):.0f} | | |")
        tot = per_call.get(call, 0.0) / max(steps, 1)
        lines.append(f"| **{call}** | (sum) | | | | {tot:.0f} | {ab[call]} | {tot / ab[call]:.4f} |")
        js["kernels"][call] = {"traffic_bytes": int(round(tot)), "source_digest": source_digest(call)}
    head = "\n".join(f"    {c}" for c in cmds)
    return ("Commands (rocprofv3 from /tmp with TMPDIR=/tmp; `<repo>` is the repository root):\n\n" + head + "\n\n"
            if cmds else "") + "\n".join(lines) + ("\n\nMachine-readable copy (bench.py reads `traffic_bytes` while "
                                                "the call's source digest matches):\n\n```json\n"
                                                + json.dumps(js, indent=1) + "\n```\n")


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="qwen3_30b_a3b")
    ap.add_argument("--sets", type=int, default=0,
                    help="input/output sets rotated across steps (0: sized so that the copies of x "
                         "exceed the Infinity Cache twice over)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--pad", type=int, default=1, help="pad expert segments to a multiple of this many rows")
    ap.add_argument("--fp8-group", type=int, default=0,
                    help="expand with FP8 E4M3 quantisation, one scale per this many columns (0: bf16 expand)")
    ap.add_argument("--mxfp8", action="store_true",
                    help="expand with MXFP8 quantisation (E4M3 codes, E8M0 scale per 32 columns) after the route")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", dest="graph", action="store_false",
                    help="skip the HIP-graph replay timing (ms_per_step_graph)")
    ap.add_argument("--events", choices=["nofence", "torch", "none"], default="nofence",
                    help="per-call HIP events inside the timed region (default: without the system fence)")
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of CPU work per CPU-baseline leg")
    ap.add_argument("--cpu-leg", choices=["single", "all"], help=argparse.SUPPRESS)
    ap.add_argument("--summarize-trace", metavar="CSV",
                    help="print per-kernel medians from a rocprofv3 kernel-trace CSV, skipping --warmup "
                         "dispatches of each kernel, and exit")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("READ_DIR", "WRITE_DIR"),
                    help="print HBM bytes per dispatch per kernel from two rocprofv3 --pmc output folders "
                         "(PMC_READ counters, then PMC_WRITE) as JSON, and exit")
    ap.add_argument("--traffic-report", nargs=2, metavar=("READ_DIR", "WRITE_DIR"),
                    help="print the per-call HBM traffic of a bench run with the same --config/--pad/--fp8-group/"
                         "--mxfp8 from its two rocprofv3 --pmc output folders (markdown), and exit")
    args = ap.parse_args(argv)

    if args.cpu_leg:
        print(json.dumps(_cpu_leg(args.config, args.seed, args.cpu_leg, args.cpu_budget)), flush=True)
        return 0
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace, args.warmup))
        return 0
    if args.summarize_pmc:
        print(json.dumps(pmc_bytes(*args.summarize_pmc), indent=1))
        return 0
    if args.traffic_report:
        from moe_glue_amd import inputs as I

        print(traffic_report(*args.traffic_report, I.CONFIGS[args.config], args.pad, args.fp8_group, args.mxfp8))
        return 0

    if args.gpus != 1:
        print(f"bench.py: the MoE glue path runs on one GPU only; --gpus {args.gpus} is not supported "
              "(no multi-GPU dispatch/combine is implemented)", file=sys.stderr)
        return 2

    import torch
    from moe_glue_amd import inputs as I

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    cfg = I.CONFIGS[args.config]
    inp = I.make_inputs(cfg, args.seed)
    nsets = args.sets if args.sets > 0 else default_sets(cfg, args.pad, args.fp8_group)
    if args.mxfp8 and args.fp8_group:
        print("bench.py: --mxfp8 and --fp8-group are two scale formats; choose one", file=sys.stderr)
        return 2
    sets = Sets(inp, nsets, dev, args.pad, args.fp8_group, args.mxfp8)
    achievable, _ = copy_probe_gbps(dev)
    floor_us = launch_floor_us(dev)

    for s in range(args.warmup):
        sets.step(s)
    torch.cuda.synchronize()

    names = sets.calls
    # Timed region 1: the path alone, K steps back to back -> value, ms_per_step.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        sets.step(s)
    host_s = time.perf_counter() - t0
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    # Timed region 2: the same K steps with a HIP event between calls on the
    # launch stream -> per-call device times (the markers cost a little, so
    # they stay out of region 1).
    use_events = args.events != "none"
    ev = None
    events_elapsed = None
    if use_events:
        if args.events == "torch":
            ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
        else:
            stream = torch.cuda.current_stream(dev).cuda_stream
            ev = [[HipEvent(stream) for _ in range(len(names) + 1)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for s in range(args.steps):
            sets.step(s, ev[s])
        torch.cuda.synchronize()
        events_elapsed = time.perf_counter() - t1

    # Timed region 3: the same steps replayed from a HIP graph (no per-call
    # host cost) -> ms_per_step_graph, reported beside the eager figure.
    graph_ms = graph_ms_per_step(sets, dev, args.steps) if args.graph else None

    ab = algorithmic_bytes(cfg, args.fp8_group)
    variant = variant_name(cfg.name, args.pad, args.fp8_group, args.mxfp8)
    kernels = {}
    mix_gbps = {}
    if use_events:
        for i, n in enumerate(names):
            ms = [ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(args.steps)]
            us = 1e3 * sum(ms) / len(ms)
            gbps = ab[n] / (us * 1e-6) / 1e9
            rd, wr = rw_bytes(cfg, args.fp8_group)[n]
            mix = mix_of(rd, wr)
            if mix not in mix_gbps:
                mix_gbps[mix] = mix_probe_gbps(dev, *mix)
            same = mix_probe_gbps(dev, *mix, nbytes=ab[n], reps=21)  # the same bytes, one plain launch
            kernels[n] = {"us": round(us, 3), "bytes": ab[n], "GBps": round(gbps, 1),
                          "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4),
                          "frac_of_achievable": round(gbps / achievable, 4),
                          "mix": {"reads": mix[0], "writes": mix[1], "probe_GBps": round(mix_gbps[mix], 1),
                                  "frac": round(gbps / mix_gbps[mix], 4), "same_bytes_GBps": round(same, 1),
                                  "frac_same_bytes": round(gbps / same, 4)},
                          "traffic": measured_traffic(n, variant)}
    # the roofline kernel: the longest call that is a single kernel (route and
    # route_expand launch several)
    single = [n for n in names if n not in ("route", "route_expand", "route_expand_padded", "route_expand_fp8",
                                            "route_expand_mxfp8")]
    dominant = max(single, key=lambda n: kernels[n]["us"]) if kernels else None
    roofline = None
    slowest = None
    if kernels:
        d = kernels[dominant]
        roofline = {"kernel": dominant, "bound": "hbm", "achieved": d["GBps"], "peak": HBM_PEAK_GBPS,
                    "unit": "GB/s", "frac": d["frac_of_peak"], "traffic": measured_traffic(dominant, variant)}
        # the call furthest below the copy probe, whatever its kernel count
        worst = min(names, key=lambda n: kernels[n]["frac_of_achievable"])
        w = kernels[worst]
        slowest = {"call": worst, "us": w["us"], "GBps": w["GBps"], "frac_of_peak": w["frac_of_peak"],
                   "frac_of_achievable": w["frac_of_achievable"]}

    ms_per_step = 1e3 * elapsed / args.steps
    rec = {
        "metric": METRIC,
        "value": round(cfg.T * args.steps / elapsed, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}", "T": cfg.T, "H": cfg.H, "E": cfg.E, "k": cfg.k, "I": cfg.I,
                   "input_sets": nsets, "seed": args.seed, "pad_to": args.pad, "fp8_group": args.fp8_group,
                   "mxfp8": args.mxfp8},
        "path_GBps": round(sum(ab[n] for n in names) / (elapsed / args.steps) / 1e9, 1),
        "achievable_copy_GBps": round(achievable, 1),
        "launch_floor_us": floor_us,
        "host_us_per_step": round(1e6 * host_s / args.steps, 2),
        "events": args.events,
        "ms_per_step_with_events": None if events_elapsed is None else round(1e3 * events_elapsed / args.steps, 4),
        "ms_per_step_graph": graph_ms,
        "kernels": kernels,
        "roofline": roofline,
        "slowest_call": slowest,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        del sets
        rec["cpu_baseline"] = cpu_baseline(cfg, args.seed, args.cpu_budget)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
