"""moe_glue_amd: the memory-bound Mixture-of-Experts glue path on MI355X (gfx950).

Four calls, each a thin wrapper over the C ABI of the HIP library
(include/moe_glue.h):

    route(logits, k, bias=None)        softmax top-k, expert counts/offsets,
                                       permutation maps
    expand_rows(x, dest_of_src, k)     expandInputRows: token rows -> expert rows
    swiglu(h)                          doActivation: silu(gate) * up
    combine(y, topk_weights, dest_of_src)  weighted sum back to token order
    route_expand(logits, k, x, bias=None)  route + expand, one launch for T <= 64
    route_expand_noalloc(logits, k, x, out=...)  the same with the library's built-in
                                       workspace (allocates nothing given `out`)
    route_padded(logits, k, pad_to)    route with expert segments padded to pad_to rows
    expand_rows_fp8(x, dest, k, group) expand with FP8 E4M3 quantisation per column group
    expand_rows_mxfp8(x, dest, k)    expand with MXFP8 quantisation (E8M0 scale per 32 columns)
    route_expand_fp8 / route_expand_mxfp8  route + the quantising expand in one call

Tensors are torch CUDA (HIP) tensors; bf16 tensors use torch.bfloat16.  Work
is enqueued on torch's current stream and nothing synchronises.  Every call
accepts preallocated outputs (``out=`` / the route output dict) so a caller
can run the path without allocating.
"""
from __future__ import annotations

from ._binding import (E_MAX, EXPORTED, K_MAX, LIB_PATH, MoEGlueArgumentError, MoEGlueError, check,  # noqa: F401
                       load)

__all__ = ["route", "route_workspace_bytes", "alloc_route_outputs", "route_padded", "padded_rows", "expand_rows",
           "expand_rows_fp8", "expand_rows_mxfp8",
           "route_expand", "route_expand_noalloc", "noalloc_scratch_bytes", "route_expand_padded", "route_expand_fp8", "route_expand_mxfp8", "swiglu", "combine",
           "copy_probe", "mix_probe", "MoEGlueError", "MoEGlueArgumentError", "E_MAX", "K_MAX"]


def _torch():
    import torch

    return torch


def _stream(device) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t) -> int:
    return 0 if t is None else t.data_ptr()


def _need_gpu(name: str, t, dtype=None, ndim=None) -> None:
    if t is None:
        raise MoEGlueArgumentError(1, f"{name} is required")
    if not t.is_cuda:
        raise MoEGlueArgumentError(2, f"{name} must be a GPU tensor (got device {t.device})")
    if not t.is_contiguous():
        raise MoEGlueArgumentError(2, f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise MoEGlueArgumentError(2, f"{name} must be {dtype} (got {t.dtype})")
    if ndim is not None and t.dim() != ndim:
        raise MoEGlueArgumentError(2, f"{name} must have {ndim} dims (got shape {tuple(t.shape)})")


def _check_bias(bias, E: int) -> None:
    """bias: None, or fp32 [E] on the GPU (the kernels read bias[e] for every e < E)."""
    if bias is None:
        return
    torch = _torch()
    _need_gpu("bias", bias, torch.float32, 1)
    if bias.shape[0] != E:
        raise MoEGlueArgumentError(2, f"bias has {bias.shape[0]} entries, logits has E={E}")


def _check_vec(name: str, t, dtype, n: int, at_least: bool = False) -> None:
    """t: a GPU tensor of `dtype` with exactly n (or at least n) elements."""
    _need_gpu(name, t, dtype)
    if (t.numel() < n) if at_least else (t.numel() != n):
        raise MoEGlueArgumentError(2, f"{name} has {t.numel()} entries, expected {'at least ' if at_least else ''}{n}")


def _check_route_out(out: dict, T: int, E: int, k: int, rows: int) -> None:
    """Caller-supplied route outputs: ids/weights/dest_of_src [T*k], offsets
    [E+1], counts [E] (or absent), src_of_dest at least `rows` entries (the
    padded row bound for a padded layout).  The workspace size is checked by
    the library itself, which receives its byte count."""
    torch = _torch()
    _check_vec("topk_ids", out.get("topk_ids"), torch.int32, T * k)
    _check_vec("topk_weights", out.get("topk_weights"), torch.float32, T * k)
    _check_vec("expert_offsets", out.get("expert_offsets"), torch.int32, E + 1)
    if out.get("expert_counts") is not None:
        _check_vec("expert_counts", out["expert_counts"], torch.int32, E)
    _check_vec("dest_of_src", out.get("dest_of_src"), torch.int32, T * k)
    _check_vec("src_of_dest", out.get("src_of_dest"), torch.int32, rows, at_least=True)
    ws = out.get("workspace")
    if ws is not None:
        _need_gpu("workspace", ws)


def _check_rows_out(name: str, t, rows: int, width: int, dtype) -> None:
    """t: a 2-D GPU tensor of `dtype`, [>= rows, width]."""
    _need_gpu(name, t, dtype, 2)
    if t.shape[0] < rows or t.shape[1] != width:
        raise MoEGlueArgumentError(2, f"{name} is {list(t.shape)}, expected [>= {rows}, {width}]")


def route_workspace_bytes(T: int, E: int, k: int) -> int:
    return int(load().moe_route_workspace_bytes(T, E, k))


def alloc_route_outputs(T: int, E: int, k: int, device) -> dict:
    """Device buffers for route(): ids, weights, offsets, counts, maps, workspace."""
    torch = _torch()
    i32, f32 = torch.int32, torch.float32
    return {
        "topk_ids": torch.empty((T, k), dtype=i32, device=device),
        "topk_weights": torch.empty((T, k), dtype=f32, device=device),
        "expert_offsets": torch.empty((E + 1,), dtype=i32, device=device),
        "expert_counts": torch.empty((E,), dtype=i32, device=device),
        "dest_of_src": torch.empty((T * k,), dtype=i32, device=device),
        "src_of_dest": torch.empty((T * k,), dtype=i32, device=device),
        "workspace": torch.empty((max(16, route_workspace_bytes(T, E, k)),), dtype=torch.uint8, device=device),
    }


def route(logits, k: int, bias=None, out: dict | None = None) -> dict:
    """Softmax top-k routing and dispatch bookkeeping; see moe_route in include/moe_glue.h."""
    torch = _torch()
    _need_gpu("logits", logits, torch.float32, 2)
    T, E = logits.shape
    _check_bias(bias, E)
    if out is None:
        out = alloc_route_outputs(T, E, k, logits.device)
    _check_route_out(out, T, E, k, T * k)
    ws = out["workspace"]
    lib = load()
    st = lib.moe_route(_ptr(logits), _ptr(bias), T, E, k, _ptr(out["topk_ids"]), _ptr(out["topk_weights"]),
                       _ptr(out["expert_offsets"]), _ptr(out.get("expert_counts")), _ptr(out["dest_of_src"]),
                       _ptr(out["src_of_dest"]), _ptr(ws), ws.numel() if ws is not None else 0,
                       _stream(logits.device))
    check(st, "moe_route")
    return out


def padded_rows(T: int, E: int, k: int, pad_to: int) -> int:
    """Upper bound on the rows of the padded layout: T*k + E*(pad_to-1)."""
    return int(load().moe_route_padded_rows(T, E, k, pad_to))


def route_padded(logits, k: int, pad_to: int, bias=None, out: dict | None = None) -> dict:
    """route() with each expert's segment padded to a multiple of pad_to rows;
    src_of_dest has padded_rows() entries (-1 on padding rows, valid up to
    expert_offsets[E]).  See moe_route_padded in include/moe_glue.h."""
    torch = _torch()
    _need_gpu("logits", logits, torch.float32, 2)
    T, E = logits.shape
    _check_bias(bias, E)
    if out is None:
        out = alloc_route_outputs(T, E, k, logits.device)
        out["src_of_dest"] = torch.empty((max(1, padded_rows(T, E, k, pad_to)),), dtype=torch.int32,
                                         device=logits.device)
    _check_route_out(out, T, E, k, padded_rows(T, E, k, pad_to))
    ws = out["workspace"]
    st = load().moe_route_padded(_ptr(logits), _ptr(bias), T, E, k, pad_to, _ptr(out["topk_ids"]),
                                 _ptr(out["topk_weights"]), _ptr(out["expert_offsets"]),
                                 _ptr(out.get("expert_counts")), _ptr(out["dest_of_src"]), _ptr(out["src_of_dest"]),
                                 _ptr(ws), ws.numel() if ws is not None else 0, _stream(logits.device))
    check(st, "moe_route_padded")
    return out


def route_expand_padded(logits, k: int, pad_to: int, x, bias=None, out: dict | None = None) -> dict:
    """route_padded() and expand_rows() in one call; see moe_route_expand_padded
    in include/moe_glue.h.  x_expanded has padded_rows() rows (padding rows
    are not written)."""
    torch = _torch()
    _need_gpu("logits", logits, torch.float32, 2)
    _need_gpu("x", x, torch.bfloat16, 2)
    T, E = logits.shape
    if x.shape[0] != T:
        raise MoEGlueArgumentError(2, f"x has {x.shape[0]} rows, logits has T={T}")
    H = x.shape[1]
    _check_bias(bias, E)
    P = max(1, padded_rows(T, E, k, pad_to))
    if out is None:
        out = alloc_route_outputs(T, E, k, logits.device)
        out["src_of_dest"] = torch.empty((P,), dtype=torch.int32, device=logits.device)
    if out.get("x_expanded") is None:
        out["x_expanded"] = torch.empty((P, H), dtype=torch.bfloat16, device=x.device)
    _check_route_out(out, T, E, k, padded_rows(T, E, k, pad_to))
    _check_rows_out("x_expanded", out["x_expanded"], padded_rows(T, E, k, pad_to), H, torch.bfloat16)
    ws = out["workspace"]
    st = load().moe_route_expand_padded(_ptr(logits), _ptr(bias), T, E, k, pad_to, _ptr(x), H, _ptr(out["topk_ids"]),
                                        _ptr(out["topk_weights"]), _ptr(out["expert_offsets"]),
                                        _ptr(out.get("expert_counts")), _ptr(out["dest_of_src"]),
                                        _ptr(out["src_of_dest"]), _ptr(out["x_expanded"]), _ptr(ws),
                                        ws.numel() if ws is not None else 0, _stream(logits.device))
    check(st, "moe_route_expand_padded")
    return out


def route_expand_fp8(logits, k: int, x, group: int, pad_to: int = 1, bias=None, out: dict | None = None) -> dict:
    """route_padded() (route() for pad_to = 1) and expand_rows_fp8() in one
    call; see moe_route_expand_fp8 in include/moe_glue.h.  Returns the route
    dict plus "x_expanded" (uint8 E4M3 codes [rows, H]) and "scales" (fp32
    [rows, H/group]); padding rows are not written."""
    torch = _torch()
    _need_gpu("logits", logits, torch.float32, 2)
    _need_gpu("x", x, torch.bfloat16, 2)
    T, E = logits.shape
    if x.shape[0] != T:
        raise MoEGlueArgumentError(2, f"x has {x.shape[0]} rows, logits has T={T}")
    H = x.shape[1]
    _check_bias(bias, E)
    P = max(1, padded_rows(T, E, k, pad_to)) if pad_to > 1 else max(1, T * k)
    if out is None:
        out = alloc_route_outputs(T, E, k, logits.device)
        out["src_of_dest"] = torch.empty((P,), dtype=torch.int32, device=logits.device)
    if out.get("x_expanded") is None:
        out["x_expanded"] = torch.empty((P, H), dtype=torch.uint8, device=x.device)
    if out.get("scales") is None:
        out["scales"] = torch.empty((P, max(1, H // group)), dtype=torch.float32, device=x.device)
    rows = padded_rows(T, E, k, pad_to) if pad_to > 1 else T * k
    _check_route_out(out, T, E, k, rows)
    _check_rows_out("x_expanded", out["x_expanded"], rows, H, torch.uint8)
    _check_rows_out("scales", out["scales"], rows, H // group if group > 0 and H % group == 0 else -1,
                    torch.float32)
    ws = out["workspace"]
    st = load().moe_route_expand_fp8(_ptr(logits), _ptr(bias), T, E, k, pad_to, _ptr(x), H, group,
                                     _ptr(out["topk_ids"]), _ptr(out["topk_weights"]), _ptr(out["expert_offsets"]),
                                     _ptr(out.get("expert_counts")), _ptr(out["dest_of_src"]),
                                     _ptr(out["src_of_dest"]), _ptr(out["x_expanded"]), _ptr(out["scales"]),
                                     _ptr(ws), ws.numel() if ws is not None else 0, _stream(logits.device))
    check(st, "moe_route_expand_fp8")
    return out


def route_expand_mxfp8(logits, k: int, x, pad_to: int = 1, bias=None, out: dict | None = None) -> dict:
    """route_padded() (route() for pad_to = 1) and expand_rows_mxfp8() in one
    call; see moe_route_expand_mxfp8 in include/moe_glue.h.  Returns the route
    dict plus "x_expanded" (uint8 E4M3 codes [rows, H]) and "scales" (uint8
    E8M0 bytes [rows, H/32]); padding rows are not written."""
    torch = _torch()
    _need_gpu("logits", logits, torch.float32, 2)
    _need_gpu("x", x, torch.bfloat16, 2)
    T, E = logits.shape
    if x.shape[0] != T:
        raise MoEGlueArgumentError(2, f"x has {x.shape[0]} rows, logits has T={T}")
    H = x.shape[1]
    _check_bias(bias, E)
    P = max(1, padded_rows(T, E, k, pad_to)) if pad_to > 1 else max(1, T * k)
    if out is None:
        out = alloc_route_outputs(T, E, k, logits.device)
        out["src_of_dest"] = torch.empty((P,), dtype=torch.int32, device=logits.device)
    if out.get("x_expanded") is None:
        out["x_expanded"] = torch.empty((P, H), dtype=torch.uint8, device=x.device)
    if out.get("scales") is None:
        out["scales"] = torch.empty((P, max(1, H // 32)), dtype=torch.uint8, device=x.device)
    rows = padded_rows(T, E, k, pad_to) if pad_to > 1 else T * k
    _check_route_out(out, T, E, k, rows)
    _check_rows_out("x_expanded", out["x_expanded"], rows, H, torch.uint8)
    _check_rows_out("scales", out["scales"], rows, H // 32 if H % 32 == 0 else -1, torch.uint8)
    ws = out["workspace"]
    st = load().moe_route_expand_mxfp8(_ptr(logits), _ptr(bias), T, E, k, pad_to, _ptr(x), H,
                                       _ptr(out["topk_ids"]), _ptr(out["topk_weights"]), _ptr(out["expert_offsets"]),
                                       _ptr(out.get("expert_counts")), _ptr(out["dest_of_src"]),
                                       _ptr(out["src_of_dest"]), _ptr(out["x_expanded"]), _ptr(out["scales"]),
                                       _ptr(ws), ws.numel() if ws is not None else 0, _stream(logits.device))
    check(st, "moe_route_expand_mxfp8")
    return out


def expand_rows(x, dest_of_src, k: int, out=None):
    """x_expanded[dest_of_src[t*k+j]] = x[t]; see moe_expand_rows in include/moe_glue.h."""
    torch = _torch()
    _need_gpu("x", x, torch.bfloat16, 2)
    _need_gpu("dest_of_src", dest_of_src, torch.int32)
    T, H = x.shape
    if dest_of_src.numel() != T * k:
        raise MoEGlueArgumentError(2, f"dest_of_src has {dest_of_src.numel()} entries, expected T*k={T * k}")
    if out is None:
        out = torch.empty((T * k, H), dtype=torch.bfloat16, device=x.device)
    else:
        _need_gpu("out", out, torch.bfloat16, 2)
        if out.shape[0] < T * k or out.shape[1] != H:
            raise MoEGlueArgumentError(2, f"out must be [>= {T * k}, {H}] (more rows for a padded layout)")
    st = load().moe_expand_rows(_ptr(x), _ptr(dest_of_src), T, H, k, _ptr(out), _stream(x.device))
    check(st, "moe_expand_rows")
    return out


def expand_rows_fp8(x, dest_of_src, k: int, group: int, rows: int | None = None, out=None, scales=None):
    """FP8 (E4M3) quantising expand; returns (codes uint8 [rows, H], scales fp32
    [rows, H/group]).  See moe_expand_rows_fp8 in include/moe_glue.h."""
    torch = _torch()
    _need_gpu("x", x, torch.bfloat16, 2)
    _need_gpu("dest_of_src", dest_of_src, torch.int32)
    T, H = x.shape
    if dest_of_src.numel() != T * k:
        raise MoEGlueArgumentError(2, f"dest_of_src has {dest_of_src.numel()} entries, expected T*k={T * k}")
    n = T * k if rows is None else rows
    if n < T * k:
        raise MoEGlueArgumentError(2, f"rows={n} is below T*k={T * k}")
    if out is None:
        out = torch.empty((n, H), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((n, max(1, H // group)), dtype=torch.float32, device=x.device)
    _check_rows_out("out", out, n, H, torch.uint8)
    _check_rows_out("scales", scales, n, H // group if group > 0 and H % group == 0 else -1, torch.float32)
    st = load().moe_expand_rows_fp8(_ptr(x), _ptr(dest_of_src), T, H, k, group, _ptr(out), _ptr(scales),
                                    _stream(x.device))
    check(st, "moe_expand_rows_fp8")
    return out, scales


def expand_rows_mxfp8(x, dest_of_src, k: int, rows: int | None = None, out=None, scales=None):
    """MXFP8 quantising expand; returns (codes uint8 [rows, H], E8M0 scale bytes
    uint8 [rows, H/32]).  See moe_expand_rows_mxfp8 in include/moe_glue.h."""
    torch = _torch()
    _need_gpu("x", x, torch.bfloat16, 2)
    _need_gpu("dest_of_src", dest_of_src, torch.int32)
    T, H = x.shape
    if dest_of_src.numel() != T * k:
        raise MoEGlueArgumentError(2, f"dest_of_src has {dest_of_src.numel()} entries, expected T*k={T * k}")
    n = T * k if rows is None else rows
    if n < T * k:
        raise MoEGlueArgumentError(2, f"rows={n} is below T*k={T * k}")
    if out is None:
        out = torch.empty((n, H), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((n, max(1, H // 32)), dtype=torch.uint8, device=x.device)
    _check_rows_out("out", out, n, H, torch.uint8)
    _check_rows_out("scales", scales, n, H // 32 if H % 32 == 0 else -1, torch.uint8)
    st = load().moe_expand_rows_mxfp8(_ptr(x), _ptr(dest_of_src), T, H, k, _ptr(out), _ptr(scales),
                                      _stream(x.device))
    check(st, "moe_expand_rows_mxfp8")
    return out, scales


def route_expand(logits, k: int, x, bias=None, out: dict | None = None) -> dict:
    """route() and expand_rows() in one call (one launch for T <= 64); see
    moe_route_expand in include/moe_glue.h.  Returns route()'s dict plus
    "x_expanded"."""
    torch = _torch()
    _need_gpu("logits", logits, torch.float32, 2)
    _need_gpu("x", x, torch.bfloat16, 2)
    T, E = logits.shape
    if x.shape[0] != T:
        raise MoEGlueArgumentError(2, f"x has {x.shape[0]} rows, logits has T={T}")
    H = x.shape[1]
    _check_bias(bias, E)
    if out is None:
        out = alloc_route_outputs(T, E, k, logits.device)
    if out.get("x_expanded") is None:
        out["x_expanded"] = torch.empty((T * k, H), dtype=torch.bfloat16, device=x.device)
    _check_route_out(out, T, E, k, T * k)
    _check_rows_out("x_expanded", out["x_expanded"], T * k, H, torch.bfloat16)
    ws = out["workspace"]
    st = load().moe_route_expand(_ptr(logits), _ptr(bias), T, E, k, _ptr(x), H, _ptr(out["topk_ids"]),
                                 _ptr(out["topk_weights"]), _ptr(out["expert_offsets"]),
                                 _ptr(out.get("expert_counts")), _ptr(out["dest_of_src"]), _ptr(out["src_of_dest"]),
                                 _ptr(out["x_expanded"]), _ptr(ws), ws.numel() if ws is not None else 0,
                                 _stream(logits.device))
    check(st, "moe_route_expand")
    return out


def noalloc_scratch_bytes() -> int:
    """Bytes of the library's built-in scratch behind route_expand_noalloc()."""
    return int(load().moe_noalloc_scratch_bytes())


def route_expand_noalloc(logits, k: int, x, bias=None, out: dict | None = None) -> dict:
    """route_expand() with the library's built-in device scratch as the route
    workspace; see moe_route_expand_noalloc in include/moe_glue.h.  With `out`
    (the route dict without "workspace", plus "x_expanded") nothing is
    allocated.  Calls that can overlap on one GPU share the scratch and race."""
    torch = _torch()
    _need_gpu("logits", logits, torch.float32, 2)
    _need_gpu("x", x, torch.bfloat16, 2)
    T, E = logits.shape
    if x.shape[0] != T:
        raise MoEGlueArgumentError(2, f"x has {x.shape[0]} rows, logits has T={T}")
    H = x.shape[1]
    _check_bias(bias, E)
    if out is None:
        out = alloc_route_outputs(T, E, k, logits.device)
        del out["workspace"]
        out["x_expanded"] = torch.empty((T * k, H), dtype=torch.bfloat16, device=x.device)
    _check_route_out(out, T, E, k, T * k)
    _check_rows_out("x_expanded", out.get("x_expanded"), T * k, H, torch.bfloat16)
    st = load().moe_route_expand_noalloc(_ptr(logits), _ptr(bias), T, E, k, _ptr(x), H, _ptr(out["topk_ids"]),
                                         _ptr(out["topk_weights"]), _ptr(out["expert_offsets"]),
                                         _ptr(out.get("expert_counts")), _ptr(out["dest_of_src"]),
                                         _ptr(out["src_of_dest"]), _ptr(out["x_expanded"]), _stream(logits.device))
    check(st, "moe_route_expand_noalloc")
    return out


def swiglu(h, out=None):
    """act = silu(h[:, :I]) * h[:, I:]; see moe_swiglu in include/moe_glue.h."""
    torch = _torch()
    _need_gpu("h", h, torch.bfloat16, 2)
    R, I2 = h.shape
    if I2 % 2:
        raise MoEGlueArgumentError(2, f"h has an odd width {I2}; expected [R, 2I]")
    I = I2 // 2
    if out is None:
        out = torch.empty((R, I), dtype=torch.bfloat16, device=h.device)
    else:
        _need_gpu("out", out, torch.bfloat16, 2)
        if tuple(out.shape) != (R, I):
            raise MoEGlueArgumentError(2, f"out must be [{R}, {I}]")
    st = load().moe_swiglu(_ptr(h), R, I, _ptr(out), _stream(h.device))
    check(st, "moe_swiglu")
    return out


def combine(y, topk_weights, dest_of_src, out=None):
    """out[t] = sum_j w[t,j] * y[dest_of_src[t*k+j]]; see moe_combine in include/moe_glue.h."""
    torch = _torch()
    _need_gpu("y", y, torch.bfloat16, 2)
    _need_gpu("topk_weights", topk_weights, torch.float32, 2)
    _need_gpu("dest_of_src", dest_of_src, torch.int32)
    T, k = topk_weights.shape
    R, H = y.shape
    if R < T * k or dest_of_src.numel() != T * k:
        raise MoEGlueArgumentError(2, f"y has {R} rows and dest_of_src {dest_of_src.numel()}; expected T*k={T * k} "
                                      "entries and at least as many rows")
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=y.device)
    else:
        _need_gpu("out", out, torch.bfloat16, 2)
        if tuple(out.shape) != (T, H):
            raise MoEGlueArgumentError(2, f"out must be [{T}, {H}]")
    st = load().moe_combine(_ptr(y), _ptr(topk_weights), _ptr(dest_of_src), T, H, k, _ptr(out), _stream(y.device))
    check(st, "moe_combine")
    return out


def copy_probe(src, dst) -> None:
    """Plain 16-byte-per-lane copy of src's bytes into dst (bandwidth measuring stick)."""
    _need_gpu("src", src)
    _need_gpu("dst", dst)
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise MoEGlueArgumentError(2, "dst is smaller than src")
    check(load().moe_copy_probe(_ptr(src), _ptr(dst), nbytes, _stream(src.device)), "moe_copy_probe")


def mix_probe(src, dst, cycles: int, reads: int, writes: int, vectors_per_lane: int = 1, threads: int = 256) -> None:
    """Streaming probe: `cycles` cycles of `reads` reading and `writes`
    writing waves, vectors_per_lane KiB each (the bandwidth of that
    read:write mix)."""
    kib = 1024 * vectors_per_lane
    if reads > 0:
        _need_gpu("src", src)
        if src.numel() * src.element_size() < cycles * reads * kib:
            raise MoEGlueArgumentError(1, "src is smaller than cycles * reads * vectors_per_lane KiB")
    _need_gpu("dst", dst)
    if dst.numel() * dst.element_size() < max(cycles * writes * kib, 1024):
        raise MoEGlueArgumentError(2, "dst is smaller than cycles * writes * vectors_per_lane KiB (1 KiB at least)")
    check(load().moe_mix_probe(_ptr(src) if reads > 0 else None, _ptr(dst), cycles, reads, writes, vectors_per_lane,
                               threads, _stream(dst.device)), "moe_mix_probe")
