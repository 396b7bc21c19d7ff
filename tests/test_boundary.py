"""The C-ABI library on the CPU: it loads, exports every declared entry point,
and rejects bad arguments with the documented status BEFORE any HIP call (so
these run without a GPU).  Also checks the host-side helpers."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_glue.h")


@pytest.fixture(scope="module")
def lib():
    from moe_glue_amd import build as mbuild
    from moe_glue_amd import _binding

    if mbuild.is_stale():
        mbuild.build(verbose=False)
    return _binding.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_\w+)\s*\(", text)))


def test_header_declares_the_four_calls():
    names = declared_functions()
    for n in ("moe_route", "moe_expand_rows", "moe_swiglu", "moe_combine", "moe_route_workspace_bytes",
              "moe_status_string", "moe_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in include/moe_glue.h but not exported"


def test_binding_names_match_header():
    from moe_glue_amd import _binding

    assert set(_binding.EXPORTED) == set(declared_functions())


FAKE = 0x10000  # a 16-byte-aligned non-NULL address: never dereferenced, since validation fails first


def status(lib, rc):
    return lib.moe_status_string(rc).decode()


def test_route_argument_errors(lib):
    ws = 1 << 20
    args = lambda T, E, k, ids=FAKE, off=FAKE, wsp=FAKE, logits=FAKE: (
        logits, None, T, E, k, ids, FAKE, off, None, FAKE, FAKE, wsp, ws, None)
    assert status(lib, lib.moe_route(*args(-1, 8, 2))) == "MOE_ERR_SHAPE"
    assert status(lib, lib.moe_route(*args(4, 0, 1))) == "MOE_ERR_SHAPE"
    assert status(lib, lib.moe_route(*args(4, 8, 0))) == "MOE_ERR_SHAPE"
    assert status(lib, lib.moe_route(*args(4, 8, 9))) == "MOE_ERR_SHAPE"
    assert status(lib, lib.moe_route(*args(4, 513, 2))) == "MOE_ERR_UNSUPPORTED"
    assert status(lib, lib.moe_route(*args(4, 64, 17))) == "MOE_ERR_UNSUPPORTED"
    assert status(lib, lib.moe_route(*args(2 ** 24, 512, 8))) == "MOE_ERR_UNSUPPORTED"
    assert status(lib, lib.moe_route(*args(4, 8, 2, ids=None))) == "MOE_ERR_NULL"
    assert status(lib, lib.moe_route(*args(4, 8, 2, off=None))) == "MOE_ERR_NULL"
    assert status(lib, lib.moe_route(*args(4, 8, 2, logits=FAKE + 2))) == "MOE_ERR_ALIGN"


def test_route_workspace_errors(lib, monkeypatch):
    monkeypatch.setenv("MOE_GLUE_ROUTE_VARIANT", "three")
    T, E, k = 4096, 128, 8
    need = lib.moe_route_workspace_bytes(T, E, k)
    hist = (4096 // 16 + 1) * 128 * 4  # 16-token histogram rows + one row of totals
    assert need == hist + T * k * 8  # + the row list of moe_route_expand (two int32 per row)
    base = (FAKE, None, T, E, k, FAKE, FAKE, FAKE, None, FAKE, FAKE)
    assert status(lib, lib.moe_route(*base, None, need, None)) == "MOE_ERR_WORKSPACE"
    assert status(lib, lib.moe_route(*base, FAKE, hist - 1, None)) == "MOE_ERR_WORKSPACE"
    assert status(lib, lib.moe_route(*base, FAKE + 4, need, None)) == "MOE_ERR_WORKSPACE"
    assert b"workspace" in lib.moe_last_error()
    # moe_route_expand also needs the row list
    xargs = (FAKE, None, T, E, k, FAKE, 2048, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE)
    assert status(lib, lib.moe_route_expand(*xargs, FAKE, need - 1, None)) == "MOE_ERR_WORKSPACE"


def test_route_workspace_size_rules(lib):
    # histogram rows (+ totals), rounded up to 16 bytes, then T*k row-list entries of 8 bytes
    assert lib.moe_route_workspace_bytes(0, 8, 2) > 0
    assert lib.moe_route_workspace_bytes(1, 5, 2) == 2 * 8 * 4 + 2 * 8  # one row + totals, experts padded to 8
    assert lib.moe_route_workspace_bytes(65, 8, 2) == (3 + 1) * 8 * 4 + 65 * 2 * 8  # 32 tokens per row at E=8
    assert lib.moe_route_workspace_bytes(33, 512, 16) == (3 + 1) * 512 * 4 + 33 * 16 * 8
    assert lib.moe_route_workspace_bytes(20, 5, 3) == 16 * (-(-2 * 8 * 4 // 16)) + 20 * 3 * 8
    assert lib.moe_route_workspace_bytes(4, 8, 9) == 0  # invalid


@pytest.mark.parametrize("fn", ["expand", "combine"])
def test_row_kernels_argument_errors(lib, fn):
    def call(x=FAKE, d=FAKE, T=4, H=256, k=2, o=FAKE):
        if fn == "expand":
            return status(lib, lib.moe_expand_rows(x, d, T, H, k, o, None))
        return status(lib, lib.moe_combine(x, FAKE, d, T, H, k, o, None))

    assert call(T=-1) == "MOE_ERR_SHAPE"
    assert call(H=0) == "MOE_ERR_SHAPE"
    assert call(k=0) == "MOE_ERR_SHAPE"
    assert call(k=17) == "MOE_ERR_SHAPE"
    assert call(H=100) == "MOE_ERR_ALIGN"  # 200-byte rows are not a multiple of 16 bytes
    assert call(x=FAKE + 8) == "MOE_ERR_ALIGN"
    assert call(o=FAKE + 2) == "MOE_ERR_ALIGN"
    assert call(x=None) == "MOE_ERR_NULL"
    assert call(d=None) == "MOE_ERR_NULL"
    assert call(T=2 ** 30, H=16) == "MOE_ERR_UNSUPPORTED"
    # T = 0 is a no-op that needs no pointers and makes no HIP call
    assert call(x=None, d=None, o=None, T=0) == "MOE_OK"


def test_swiglu_argument_errors(lib):
    assert status(lib, lib.moe_swiglu(FAKE, -1, 768, FAKE, None)) == "MOE_ERR_SHAPE"
    assert status(lib, lib.moe_swiglu(FAKE, 4, 0, FAKE, None)) == "MOE_ERR_SHAPE"
    assert status(lib, lib.moe_swiglu(FAKE, 4, 12, FAKE, None)) == "MOE_ERR_ALIGN"
    assert status(lib, lib.moe_swiglu(FAKE + 4, 4, 768, FAKE, None)) == "MOE_ERR_ALIGN"
    assert status(lib, lib.moe_swiglu(None, 4, 768, FAKE, None)) == "MOE_ERR_NULL"
    assert status(lib, lib.moe_swiglu(FAKE, 2 ** 28, 64, FAKE, None)) == "MOE_ERR_UNSUPPORTED"
    assert status(lib, lib.moe_swiglu(None, 0, 768, None, None)) == "MOE_OK"


def test_copy_probe_argument_errors(lib):
    assert status(lib, lib.moe_copy_probe(None, FAKE, 32, None)) == "MOE_ERR_NULL"
    assert status(lib, lib.moe_copy_probe(FAKE, FAKE, 24, None)) == "MOE_ERR_ALIGN"
    assert status(lib, lib.moe_copy_probe(None, None, 0, None)) == "MOE_OK"


def test_status_strings(lib):
    names = [lib.moe_status_string(i).decode() for i in range(7)]
    assert names == ["MOE_OK", "MOE_ERR_NULL", "MOE_ERR_SHAPE", "MOE_ERR_ALIGN", "MOE_ERR_UNSUPPORTED",
                     "MOE_ERR_WORKSPACE", "MOE_ERR_HIP"]


def test_python_binding_maps_errors_to_value_error(lib):
    from moe_glue_amd import _binding

    rc = lib.moe_swiglu(FAKE, 4, 12, FAKE, None)
    with pytest.raises(ValueError, match="MOE_ERR_ALIGN"):
        _binding.check(rc, "moe_swiglu")


def test_python_binding_rejects_cpu_tensors():
    import torch
    import moe_glue_amd as mg

    with pytest.raises(ValueError, match="GPU tensor"):
        mg.swiglu(torch.zeros((4, 16), dtype=torch.bfloat16))


def test_fastdiv_host(tmp_path):
    """The multiply-shift division of the streaming kernels, on the host."""
    exe = tmp_path / "fastdiv_check"
    src = os.path.join(ROOT, "tests", "host", "fastdiv_check.cpp")
    inc = os.path.join(ROOT, "moe_glue_amd", "csrc")
    subprocess.run(["hipcc", "-O2", "-std=c++17", "-x", "hip", "--offload-arch=gfx950", "-I", inc, src, "-o",
                    str(exe)], check=True, capture_output=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0 and out.stdout.startswith("ok"), out.stdout + out.stderr


def test_row_groups_host(tmp_path):
    """The token-group arithmetic of the grouped expand and a model of the
    row-list positions, on the host (tests/host/row_groups_check.cpp)."""
    exe = tmp_path / "row_groups_check"
    src = os.path.join(ROOT, "tests", "host", "row_groups_check.cpp")
    csrc = os.path.join(ROOT, "moe_glue_amd", "csrc")
    subprocess.run(["hipcc", "-O2", "-std=c++17", "-x", "hip", "--offload-arch=gfx950", "-Xclang", "-target-feature",
                    "-Xclang", "-packed-fp32-ops", "-I", csrc, "-I", os.path.join(ROOT, "include"), src,
                    os.path.join(csrc, "route.hip"), "-o", str(exe)], check=True, capture_output=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0 and out.stdout.startswith("ok"), out.stdout + out.stderr


def test_place_copy_slices_host(tmp_path):
    """The slices of the place step's token-order copy cover every (token,
    column) of a unit once, and keep FP8 scale groups whole, on the host
    (tests/host/place_copy_check.cpp)."""
    exe = tmp_path / "place_copy_check"
    src = os.path.join(ROOT, "tests", "host", "place_copy_check.cpp")
    csrc = os.path.join(ROOT, "moe_glue_amd", "csrc")
    subprocess.run(["hipcc", "-O2", "-std=c++17", "-x", "hip", "--offload-arch=gfx950", "-I", csrc, src, "-o",
                    str(exe)], check=True, capture_output=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0 and out.stdout.startswith("ok"), out.stdout + out.stderr


def test_route_expand_argument_errors(lib):
    def call(T=4, E=8, k=2, x=FAKE, H=256, ids=FAKE, xe=FAKE, ws=None, wsb=0):
        return status(lib, lib.moe_route_expand(FAKE, None, T, E, k, x, H, ids, FAKE, FAKE, None, FAKE, FAKE, xe,
                                                ws, wsb, None))

    assert call(k=9) == "MOE_ERR_SHAPE"
    assert call(E=600) == "MOE_ERR_UNSUPPORTED"
    assert call(ids=None) == "MOE_ERR_NULL"
    assert call(x=None) == "MOE_ERR_NULL"
    assert call(xe=None) == "MOE_ERR_NULL"
    assert call(H=12) == "MOE_ERR_ALIGN"
    assert call(x=FAKE + 8) == "MOE_ERR_ALIGN"
    # above the one-launch size the route workspace is required
    assert call(T=65) == "MOE_ERR_WORKSPACE"
    assert call(T=4096, E=128, k=8, ws=FAKE, wsb=16) == "MOE_ERR_WORKSPACE"


def test_route_padded_argument_errors(lib):
    def call(T=4, E=8, k=2, pad=16):
        return status(lib, lib.moe_route_padded(FAKE, None, T, E, k, pad, FAKE, FAKE, FAKE, None, FAKE, FAKE,
                                                FAKE, 1 << 20, None))

    assert call(pad=0) == "MOE_ERR_SHAPE"
    assert call(pad=-3) == "MOE_ERR_SHAPE"
    assert call(pad=4097) == "MOE_ERR_UNSUPPORTED"
    assert call(T=2 ** 22, E=512, k=16, pad=4096) == "MOE_ERR_UNSUPPORTED"
    assert call(k=9) == "MOE_ERR_SHAPE"
    assert lib.moe_route_padded_rows(4096, 128, 8, 128) == 4096 * 8 + 128 * 127
    assert lib.moe_route_padded_rows(10, 4, 2, 1) == 20
    assert lib.moe_route_padded_rows(10, 4, 2, 0) == 0


def test_route_expand_padded_argument_errors(lib):
    def call(T=4, E=8, k=2, pad=16, x=FAKE, H=256, xe=FAKE, ws=None, wsb=0):
        return status(lib, lib.moe_route_expand_padded(FAKE, None, T, E, k, pad, x, H, FAKE, FAKE, FAKE, None, FAKE,
                                                       FAKE, xe, ws, wsb, None))

    assert call(pad=0) == "MOE_ERR_SHAPE"
    assert call(pad=4097) == "MOE_ERR_UNSUPPORTED"
    assert call(k=9) == "MOE_ERR_SHAPE"
    assert call(x=None) == "MOE_ERR_NULL"
    assert call(H=12) == "MOE_ERR_ALIGN"
    assert call(T=65) == "MOE_ERR_WORKSPACE"
    need = lib.moe_route_workspace_bytes(4096, 128, 8)
    assert call(T=4096, E=128, k=8, H=2048, ws=FAKE, wsb=need - 1) == "MOE_ERR_WORKSPACE"
    assert b"moe_route_expand_padded" in lib.moe_last_error()


def test_expand_fp8_argument_errors(lib):
    def call(x=FAKE, d=FAKE, T=4, H=256, k=2, group=128, q=FAKE, sc=FAKE):
        return status(lib, lib.moe_expand_rows_fp8(x, d, T, H, k, group, q, sc, None))

    assert call(group=12) == "MOE_ERR_UNSUPPORTED"
    assert call(group=4) == "MOE_ERR_UNSUPPORTED"
    assert call(group=1024) == "MOE_ERR_UNSUPPORTED"
    assert call(H=192, group=128) == "MOE_ERR_SHAPE"
    assert call(H=100) == "MOE_ERR_ALIGN"
    assert call(sc=None) == "MOE_ERR_NULL"
    assert call(q=None) == "MOE_ERR_NULL"
    assert call(q=FAKE + 4) == "MOE_ERR_ALIGN"
    assert call(x=FAKE + 8) == "MOE_ERR_ALIGN"
    assert call(sc=FAKE + 2) == "MOE_ERR_ALIGN"
    assert call(T=0, x=None, d=None, q=None, sc=None) == "MOE_OK"


def test_expand_mxfp8_argument_errors(lib):
    def call(x=FAKE, d=FAKE, T=4, H=256, k=2, q=FAKE, sc=FAKE):
        return status(lib, lib.moe_expand_rows_mxfp8(x, d, T, H, k, q, sc, None))

    assert call(H=48) == "MOE_ERR_SHAPE"       # 16-byte rows, but not whole 32-column blocks
    assert call(H=100) == "MOE_ERR_ALIGN"
    assert call(k=0) == "MOE_ERR_SHAPE"
    assert call(k=17) == "MOE_ERR_SHAPE"
    assert call(sc=None) == "MOE_ERR_NULL"
    assert call(q=None) == "MOE_ERR_NULL"
    assert call(d=None) == "MOE_ERR_NULL"
    assert call(q=FAKE + 4) == "MOE_ERR_ALIGN"
    assert call(x=FAKE + 8) == "MOE_ERR_ALIGN"
    assert call(T=-1) == "MOE_ERR_SHAPE"
    assert call(T=0, x=None, d=None, q=None, sc=None) == "MOE_OK"


def test_route_expand_mxfp8_argument_errors(lib):
    def call(T=4, E=8, k=2, pad=1, x=FAKE, H=256, q=FAKE, sc=FAKE, ws=None, wsb=0):
        return status(lib, lib.moe_route_expand_mxfp8(FAKE, None, T, E, k, pad, x, H, FAKE, FAKE, FAKE, None,
                                                      FAKE, FAKE, q, sc, ws, wsb, None))

    assert call(pad=0) == "MOE_ERR_SHAPE"
    assert call(k=9) == "MOE_ERR_SHAPE"
    assert call(H=48) == "MOE_ERR_SHAPE"
    assert call(H=100) == "MOE_ERR_ALIGN"
    assert call(x=None) == "MOE_ERR_NULL"
    assert call(sc=None) == "MOE_ERR_NULL"
    assert call(q=FAKE + 4) == "MOE_ERR_ALIGN"
    assert call(T=65) == "MOE_ERR_WORKSPACE"
    need = lib.moe_route_workspace_bytes(4096, 128, 8)
    assert call(T=4096, E=128, k=8, H=2048, ws=FAKE, wsb=need - 1) == "MOE_ERR_WORKSPACE"
    assert b"moe_route_expand_mxfp8" in lib.moe_last_error()


def test_route_expand_fp8_argument_errors(lib):
    def call(T=4, E=8, k=2, pad=1, x=FAKE, H=256, group=128, q=FAKE, sc=FAKE, ws=None, wsb=0):
        return status(lib, lib.moe_route_expand_fp8(FAKE, None, T, E, k, pad, x, H, group, FAKE, FAKE, FAKE, None,
                                                    FAKE, FAKE, q, sc, ws, wsb, None))

    assert call(pad=0) == "MOE_ERR_SHAPE"
    assert call(k=9) == "MOE_ERR_SHAPE"
    assert call(group=12) == "MOE_ERR_UNSUPPORTED"
    assert call(group=1024) == "MOE_ERR_UNSUPPORTED"
    assert call(H=192, group=128) == "MOE_ERR_SHAPE"
    assert call(H=100) == "MOE_ERR_ALIGN"
    assert call(x=None) == "MOE_ERR_NULL"
    assert call(sc=None) == "MOE_ERR_NULL"
    assert call(q=FAKE + 4) == "MOE_ERR_ALIGN"
    assert call(T=65) == "MOE_ERR_WORKSPACE"
    need = lib.moe_route_workspace_bytes(4096, 128, 8)
    assert call(T=4096, E=128, k=8, H=2048, ws=FAKE, wsb=need - 1) == "MOE_ERR_WORKSPACE"
    assert b"moe_route_expand_fp8" in lib.moe_last_error()
