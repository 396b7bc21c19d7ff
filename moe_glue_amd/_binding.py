"""ctypes binding of libmoe_glue.so (the C ABI in include/moe_glue.h).

Argument marshalling only: every step of the MoE glue path runs in the HIP
kernels behind the C ABI.  PyTorch supplies device memory and the current
stream.  There is no fallback: if the library is missing, or a tensor is not
on a GPU, the call raises.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_lib", "libmoe_glue.so")

# moe_status codes
MOE_OK, MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_ALIGN, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(7)
E_MAX = 512
K_MAX = 16
PAD_MAX = 4096

EXPORTED = ("moe_route_workspace_bytes", "moe_route", "moe_route_padded_rows", "moe_route_padded",
            "moe_expand_rows", "moe_expand_rows_fp8", "moe_expand_rows_mxfp8", "moe_route_expand", "moe_route_expand_padded",
            "moe_route_expand_fp8", "moe_route_expand_mxfp8", "moe_noalloc_scratch_bytes", "moe_route_expand_noalloc",
            "moe_swiglu", "moe_combine", "moe_copy_probe", "moe_mix_probe",
            "moe_status_string", "moe_last_error")
# include/moe_glue_testing.h
TESTING_EXPORTED = ("moe_testing_force",)
ROUTE_VARIANTS = {"auto": 0, "single": 1, "two": 2, "three": 3}
EXPAND_ORDERS = {"auto": 0, "token": 1, "fused": 2, "grouped": 3, "placed": 4}

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32


class MoEGlueError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class MoEGlueArgumentError(MoEGlueError, ValueError):
    pass


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (no GPU work happens at load time)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"moe_glue HIP library not built: {path} is missing "
                           "(run python -m moe_glue_amd.build or __graft_entry__.build())")
    # PyTorch ships its own HIP runtime under the same soname; load it first so
    # that the library binds to that one runtime (the one that owns the device
    # memory and streams handed in) rather than pulling in a second copy.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    lib.moe_route_workspace_bytes.restype = ctypes.c_size_t
    lib.moe_route_workspace_bytes.argtypes = [_i32, _i32, _i32]
    lib.moe_route.restype = ctypes.c_int
    lib.moe_route.argtypes = [_vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
    lib.moe_route_padded_rows.restype = ctypes.c_size_t
    lib.moe_route_padded_rows.argtypes = [_i32, _i32, _i32, _i32]
    lib.moe_route_padded.restype = ctypes.c_int
    lib.moe_route_padded.argtypes = [_vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                     ctypes.c_size_t, _vp]
    lib.moe_expand_rows.restype = ctypes.c_int
    lib.moe_expand_rows.argtypes = [_vp, _vp, _i32, _i32, _i32, _vp, _vp]
    lib.moe_expand_rows_fp8.restype = ctypes.c_int
    lib.moe_expand_rows_fp8.argtypes = [_vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp]
    lib.moe_expand_rows_mxfp8.restype = ctypes.c_int
    lib.moe_expand_rows_mxfp8.argtypes = [_vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp]
    lib.moe_route_expand.restype = ctypes.c_int
    lib.moe_route_expand.argtypes = [_vp, _vp, _i32, _i32, _i32, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                     ctypes.c_size_t, _vp]
    lib.moe_route_expand_padded.restype = ctypes.c_int
    lib.moe_route_expand_padded.argtypes = [_vp, _vp, _i32, _i32, _i32, _i32, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp,
                                            _vp, _vp, ctypes.c_size_t, _vp]
    lib.moe_route_expand_fp8.restype = ctypes.c_int
    lib.moe_route_expand_fp8.argtypes = [_vp, _vp, _i32, _i32, _i32, _i32, _vp, _i32, _i32, _vp, _vp, _vp, _vp, _vp,
                                         _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
    lib.moe_route_expand_mxfp8.restype = ctypes.c_int
    lib.moe_route_expand_mxfp8.argtypes = [_vp, _vp, _i32, _i32, _i32, _i32, _vp, _i32, _vp, _vp, _vp, _vp, _vp,
                                           _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
    lib.moe_noalloc_scratch_bytes.restype = ctypes.c_size_t
    lib.moe_noalloc_scratch_bytes.argtypes = []
    lib.moe_route_expand_noalloc.restype = ctypes.c_int
    lib.moe_route_expand_noalloc.argtypes = [_vp, _vp, _i32, _i32, _i32, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp,
                                             _vp, _vp]
    lib.moe_swiglu.restype = ctypes.c_int
    lib.moe_swiglu.argtypes = [_vp, _i32, _i32, _vp, _vp]
    lib.moe_combine.restype = ctypes.c_int
    lib.moe_combine.argtypes = [_vp, _vp, _vp, _i32, _i32, _i32, _vp, _vp]
    lib.moe_copy_probe.restype = ctypes.c_int
    lib.moe_copy_probe.argtypes = [_vp, _vp, ctypes.c_size_t, _vp]
    lib.moe_mix_probe.restype = ctypes.c_int
    lib.moe_mix_probe.argtypes = [_vp, _vp, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32, _i32, _i32, _vp]
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_status_string.argtypes = [ctypes.c_int]
    lib.moe_last_error.restype = ctypes.c_char_p
    lib.moe_last_error.argtypes = []
    lib.moe_testing_force.restype = ctypes.c_int
    lib.moe_testing_force.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    _lib = lib
    return lib


def check(status: int, fn: str) -> None:
    if status == MOE_OK:
        return
    lib = load()
    name = lib.moe_status_string(status).decode()
    detail = lib.moe_last_error().decode()
    cls = MoEGlueError if status == MOE_ERR_HIP else MoEGlueArgumentError
    raise cls(status, f"{fn}: {name}: {detail}")


def testing_force(route: str = "auto", order: str = "auto", workgroups_per_group: int = 0) -> None:
    """Test and measurement hook (include/moe_glue_testing.h): force the route
    variant and the expand order process-wide; "auto" everywhere restores the
    library's own choice."""
    rc = load().moe_testing_force(ROUTE_VARIANTS[route], EXPAND_ORDERS[order], int(workgroups_per_group))
    if rc != 0:
        raise ValueError(f"moe_testing_force rejected ({route}, {order}, {workgroups_per_group})")
