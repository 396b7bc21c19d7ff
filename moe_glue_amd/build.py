"""Build the HIP library moe_glue_amd/_lib/libmoe_glue.so for gfx950 with hipcc.

Usage: python -m moe_glue_amd.build [--isa]   (--isa also keeps the gfx950
assembly of every kernel file under _build/isa/ for inspection).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBDIR = os.path.join(PKG, "_lib")
LIB = os.path.join(LIBDIR, "libmoe_glue.so")
BUILD = os.path.join(ROOT, "_build")

SOURCES = ["api.cpp", "route.hip", "dispatch.hip", "expand.hip", "quant.hip", "swiglu.hip", "combine.hip",
           "probe.hip", "noalloc.hip", "place_expand.hip"]
HEADERS = ["device_common.h", "kernels.h", "route_common.h", "fp8_common.h", "place_copy.h"]
ARCH = "gfx950"

# -packed-fp32-ops off: hipcc would otherwise form v_pk_{add,mul,fma}_f32 from
# scalar or float2 code; none is wanted here.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _compile(src: str, obj: str, isa_dir: str | None) -> None:
    cmd = [hipcc(), *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if isa_dir:
        cmd += ["-save-temps=obj"]
    proc = subprocess.run(cmd, capture_output=True, text=True, cwd=isa_dir or BUILD)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{proc.stderr}")
    noise = "is not a recognized feature for this target"
    warn = "\n".join(ln for ln in proc.stderr.splitlines() if ln.strip() and noise not in ln)
    if warn:
        print(f"[{src}]\n{warn}", file=sys.stderr)


def build(isa: bool = False, verbose: bool = True) -> str:
    os.makedirs(LIBDIR, exist_ok=True)
    objdir = os.path.join(BUILD, "obj")
    os.makedirs(objdir, exist_ok=True)
    isa_dir = os.path.join(BUILD, "isa") if isa else None
    if isa_dir:
        os.makedirs(isa_dir, exist_ok=True)
    objs = [os.path.join(objdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        list(ex.map(lambda so: _compile(so[0], so[1], isa_dir), zip(SOURCES, objs)))
    tmp = LIB + ".tmp"
    subprocess.run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], check=True)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    files = [os.path.join(CSRC, f) for f in SOURCES + HEADERS] + [os.path.join(INCLUDE, "moe_glue.h"), os.path.join(INCLUDE, "moe_glue_testing.h")]
    return any(os.path.getmtime(f) > t for f in files)


if __name__ == "__main__":
    build(isa="--isa" in sys.argv)
