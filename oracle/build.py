"""Build the CPU oracle (plain C, gcc) into oracle/libmoe_oracle.so.

TEST INFRASTRUCTURE ONLY: the oracle is loaded by the test suite, the package
smoke check and the benchmark's CPU-baseline leg, never by the HIP library.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_oracle.c")
LIB = os.path.join(HERE, "libmoe_oracle.so")

# -ffp-contract=off: no fused multiply-adds, so every fp64 operation rounds as written.
CFLAGS = ["-std=c11", "-O2", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra"]


def build(src: str = SRC, out: str = LIB, extra_flags=()) -> str:
    cmd = ["gcc", *CFLAGS, *extra_flags, "-I", HERE, src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def is_stale(lib: str = LIB) -> bool:
    if not os.path.exists(lib):
        return True
    t = os.path.getmtime(lib)
    return any(os.path.getmtime(os.path.join(HERE, f)) > t for f in ("moe_oracle.c", "moe_oracle.h"))


if __name__ == "__main__":
    print(build(*sys.argv[1:2]))
