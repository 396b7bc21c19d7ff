"""Helpers for the GPU tests: move seeded host inputs to the device, run the
HIP path through the C ABI (the moe_glue_amd binding), bring results back."""
from __future__ import annotations

import numpy as np


def device():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return torch.device("cuda:0")


def to_dev(a: np.ndarray, dev):
    import torch

    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:  # raw bf16 bits
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(a).to(dev)


def to_host(t) -> np.ndarray:
    import torch

    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def route_host(r: dict) -> dict:
    return {k: to_host(v) for k, v in r.items() if k != "workspace"}


def run_path(inp: dict, dev, parts=("route", "expand", "swiglu", "combine"), fused: bool = False) -> dict:
    """The whole HIP path on one input dict from moe_glue_amd.inputs.  With
    `fused`, route and expand run as one moe_route_expand call (as the
    benchmark does)."""
    import torch
    import moe_glue_amd as mg

    cfg = inp["cfg"]
    out = {}
    logits = to_dev(inp["logits"], dev)
    bias = to_dev(inp["bias"], dev) if inp.get("bias") is not None else None
    if fused:  # route + expand in one call; x_expanded comes with the route outputs
        r = mg.route_expand(logits, cfg.k, to_dev(inp["x"], dev), bias)
    else:
        r = mg.route(logits, cfg.k, bias)
    out.update(route_host(r))
    # the row kernels trust dest_of_src; make sure it is a permutation before they run
    d = out["dest_of_src"]
    assert d.size == cfg.R and (d.size == 0 or (d.min() >= 0 and d.max() < cfg.R)), "dest_of_src out of range"
    assert np.array_equal(np.sort(d), np.arange(cfg.R)), "dest_of_src is not a permutation"
    if "expand" in parts and not fused:
        out["x_expanded"] = to_host(mg.expand_rows(to_dev(inp["x"], dev), r["dest_of_src"], cfg.k))
    if "swiglu" in parts:
        out["act"] = to_host(mg.swiglu(to_dev(inp["h"], dev)))
    if "combine" in parts:
        out["out"] = to_host(mg.combine(to_dev(inp["y"], dev), r["topk_weights"], r["dest_of_src"]))
    torch.cuda.synchronize(dev)
    return out
