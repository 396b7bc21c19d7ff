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
TESTING_HEADER = os.path.join(ROOT, "include", "moe_glue_testing.h")


@pytest.fixture(scope="module")
def lib():
    from moe_glue_amd import build as mbuild
    from moe_glue_amd import _binding

    if mbuild.is_stale():
        mbuild.build(verbose=False)
    return _binding.load()


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_\w+)\s*\(", text)))


def test_include_holds_only_the_two_headers():
    assert sorted(os.listdir(os.path.join(ROOT, "include"))) == ["moe_glue.h", "moe_glue_testing.h"]


def test_header_declares_the_four_calls():
    names = declared_functions()
    for n in ("moe_route", "moe_expand_rows", "moe_swiglu", "moe_combine", "moe_route_workspace_bytes",
              "moe_status_string", "moe_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for header in (HEADER, TESTING_HEADER):
        for name in declared_functions(header):
            assert hasattr(lib, name), f"{name} declared in {os.path.basename(header)} but not exported"


def test_binding_names_match_header():
    from moe_glue_amd import _binding

    assert set(_binding.EXPORTED) == set(declared_functions())
    assert set(_binding.TESTING_EXPORTED) == set(declared_functions(TESTING_HEADER))


def test_testing_hook_rejects_out_of_range_values(lib):
    assert lib.moe_testing_force(4, 0, 0) == -1
    assert lib.moe_testing_force(0, 5, 0) == -1
    assert lib.moe_testing_force(0, 0, -1) == -1
    assert lib.moe_testing_force(0, 0, 0) == 0


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


def test_route_workspace_errors(lib, force):
    force.route("three")
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


def test_mix_probe_argument_errors(lib):
    assert status(lib, lib.moe_mix_probe(None, FAKE, 64, 1, 1, 1, 256, None)) == "MOE_ERR_NULL"
    assert status(lib, lib.moe_mix_probe(FAKE, None, 64, 1, 1, 1, 256, None)) == "MOE_ERR_NULL"
    assert status(lib, lib.moe_mix_probe(FAKE + 4, FAKE, 64, 1, 1, 1, 256, None)) == "MOE_ERR_ALIGN"
    assert status(lib, lib.moe_mix_probe(FAKE, FAKE, 64, 65, 1, 1, 256, None)) == "MOE_ERR_SHAPE"
    assert status(lib, lib.moe_mix_probe(FAKE, FAKE, (1 << 23) + 1, 1, 1, 1, 256, None)) == "MOE_ERR_SHAPE"
    assert status(lib, lib.moe_mix_probe(FAKE, FAKE, 64, 1, 1, 3, 256, None)) == "MOE_ERR_SHAPE"
    assert status(lib, lib.moe_mix_probe(FAKE, FAKE, 64, 1, 1, 1, 128, None)) == "MOE_ERR_SHAPE"
    assert status(lib, lib.moe_mix_probe(None, None, 0, 1, 1, 1, 256, None)) == "MOE_OK"
    assert status(lib, lib.moe_mix_probe(None, None, 64, 0, 0, 1, 256, None)) == "MOE_OK"


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


def test_place_expand_indexing_host(tmp_path):
    """The placing destination-order expand's index arithmetic for random
    routings and forced workgroups per group: every index in bounds, every
    destination placed and copied once, at the stable counting-sort position
    (tests/host/place_expand_check.cpp)."""
    exe = tmp_path / "place_expand_check"
    src = os.path.join(ROOT, "tests", "host", "place_expand_check.cpp")
    csrc = os.path.join(ROOT, "moe_glue_amd", "csrc")
    subprocess.run(["hipcc", "-O2", "-std=c++17", "-x", "hip", "--offload-arch=gfx950", "-Xclang", "-target-feature",
                    "-Xclang", "-packed-fp32-ops", "-I", csrc, "-I", os.path.join(ROOT, "include"), src,
                    os.path.join(csrc, "route.hip"), os.path.join(csrc, "place_expand.hip"), "-o", str(exe)],
                   check=True, capture_output=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
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


class FakeGpu:
    """Stands in for a contiguous GPU tensor of a given shape and dtype, so the
    binding's checks can run on the CPU.  Its data pointer is never wanted: a
    check that fails raises before any pointer is read, and data_ptr() raises
    to make sure no call with a fake address reaches the library."""

    def __init__(self, shape, dtype):
        import torch

        self._t = torch.empty(shape, dtype=dtype)
        self.dtype = dtype
        self.shape = self._t.shape
        self.is_cuda = True
        self.device = torch.device("cuda", 0)

    def is_contiguous(self):
        return True

    def dim(self):
        return self._t.dim()

    def numel(self):
        return self._t.numel()

    def element_size(self):
        return self._t.element_size()

    def data_ptr(self):
        raise AssertionError("the binding reached a library call with a fake tensor")


def fake_route_out(T, E, k, src_rows=None, counts=True):
    import torch

    out = {"topk_ids": FakeGpu((T, k), torch.int32), "topk_weights": FakeGpu((T, k), torch.float32),
           "expert_offsets": FakeGpu((E + 1,), torch.int32),
           "expert_counts": FakeGpu((E,), torch.int32) if counts else None,
           "dest_of_src": FakeGpu((T * k,), torch.int32),
           "src_of_dest": FakeGpu((T * k if src_rows is None else src_rows,), torch.int32),
           "workspace": FakeGpu((1 << 16,), torch.uint8)}
    return out


@pytest.mark.parametrize("call", ["route", "route_padded", "route_expand", "route_expand_padded", "route_expand_fp8",
                                  "route_expand_mxfp8"])
def test_binding_rejects_bias_of_wrong_length(lib, call):
    """Every route wrapper checks that bias has E entries before any launch
    (the kernels read bias[e] for every e < E)."""
    import torch
    import moe_glue_amd as mg

    T, E, k, H = 70, 16, 4, 64
    logits = FakeGpu((T, E), torch.float32)
    x = FakeGpu((T, H), torch.bfloat16)
    rows = mg.padded_rows(T, E, k, 8)
    for bad in (E - 1, E + 1):
        bias = FakeGpu((bad,), torch.float32)
        out = fake_route_out(T, E, k, rows)
        out["x_expanded"] = FakeGpu((rows, H), torch.uint8 if call.endswith("fp8") else torch.bfloat16)
        out["scales"] = FakeGpu((rows, H // 32), torch.uint8 if call.endswith("mxfp8") else torch.float32)
        with pytest.raises(ValueError, match="bias has"):
            if call == "route":
                mg.route(logits, k, bias, out=out)
            elif call == "route_padded":
                mg.route_padded(logits, k, 8, bias, out=out)
            elif call == "route_expand":
                mg.route_expand(logits, k, x, bias, out=out)
            elif call == "route_expand_padded":
                mg.route_expand_padded(logits, k, 8, x, bias, out=out)
            elif call == "route_expand_fp8":
                mg.route_expand_fp8(logits, k, x, 32, 8, bias, out=out)
            else:
                mg.route_expand_mxfp8(logits, k, x, 8, bias, out=out)


def test_binding_rejects_short_route_outputs(lib):
    """Caller-supplied route outputs are size-checked: an unpadded src_of_dest
    handed to a padded route, short id/weight/map arrays, short offsets."""
    import torch
    import moe_glue_amd as mg

    T, E, k = 70, 16, 4
    logits = FakeGpu((T, E), torch.float32)
    with pytest.raises(ValueError, match="src_of_dest"):
        mg.route_padded(logits, k, 8, out=fake_route_out(T, E, k))  # T*k entries, padded rows needed
    for key, shape, dtype in (("topk_ids", (T * k - 1,), torch.int32), ("topk_weights", (T, k - 1), torch.float32),
                              ("expert_offsets", (E,), torch.int32), ("expert_counts", (E - 1,), torch.int32),
                              ("dest_of_src", (T * k + 1,), torch.int32), ("src_of_dest", (T * k - 1,), torch.int32),
                              ("topk_ids", (T, k), torch.int64)):
        out = fake_route_out(T, E, k)
        out[key] = FakeGpu(shape, dtype)
        with pytest.raises(ValueError, match=key):
            mg.route(logits, k, out=out)


def test_binding_rejects_short_expanded_rows(lib):
    """x_expanded (and scales) of the combined calls must hold every expanded row."""
    import torch
    import moe_glue_amd as mg

    T, E, k, H = 70, 16, 4, 64
    logits = FakeGpu((T, E), torch.float32)
    x = FakeGpu((T, H), torch.bfloat16)
    out = fake_route_out(T, E, k)
    out["x_expanded"] = FakeGpu((T * k - 1, H), torch.bfloat16)
    with pytest.raises(ValueError, match="x_expanded"):
        mg.route_expand(logits, k, x, out=out)
    out = fake_route_out(T, E, k)
    out["x_expanded"] = FakeGpu((T * k, H), torch.uint8)
    out["scales"] = FakeGpu((T * k, H // 16 + 1), torch.float32)
    with pytest.raises(ValueError, match="scales"):
        mg.route_expand_fp8(logits, k, x, 16, out=out)
    out = fake_route_out(T, E, k)
    out["x_expanded"] = FakeGpu((T * k, H), torch.uint8)
    out["scales"] = FakeGpu((T * k - 1, H // 32), torch.uint8)
    with pytest.raises(ValueError, match="scales"):
        mg.route_expand_mxfp8(logits, k, x, out=out)


@pytest.mark.parametrize("fmt", ["fp8", "mxfp8"])
def test_binding_quantising_expand_checks_sizes(lib, fmt):
    """expand_rows_fp8 / _mxfp8: dest_of_src must have T*k entries, the code
    rows and scales must hold every expanded row, with the right widths."""
    import torch
    import moe_glue_amd as mg

    T, H, k, group = 10, 64, 3, 32
    x = FakeGpu((T, H), torch.bfloat16)
    sdt = torch.float32 if fmt == "fp8" else torch.uint8

    def call(dest, out=None, scales=None, rows=None):
        if fmt == "fp8":
            return mg.expand_rows_fp8(x, dest, k, group, rows=rows, out=out, scales=scales)
        return mg.expand_rows_mxfp8(x, dest, k, rows=rows, out=out, scales=scales)

    good = FakeGpu((T * k,), torch.int32)
    with pytest.raises(ValueError, match="dest_of_src"):
        call(FakeGpu((T * k - 1,), torch.int32), FakeGpu((T * k, H), torch.uint8), FakeGpu((T * k, H // 32), sdt))
    with pytest.raises(ValueError, match="out"):
        call(good, FakeGpu((T * k - 1, H), torch.uint8), FakeGpu((T * k, H // 32), sdt))
    with pytest.raises(ValueError, match="out"):
        call(good, FakeGpu((T * k, H + 8), torch.uint8), FakeGpu((T * k, H // 32), sdt))
    with pytest.raises(ValueError, match="scales"):
        call(good, FakeGpu((T * k, H), torch.uint8), FakeGpu((T * k - 1, H // 32), sdt))
    with pytest.raises(ValueError, match="scales"):
        call(good, FakeGpu((T * k, H), torch.uint8), FakeGpu((T * k, H // 32 + 1), sdt))
    with pytest.raises(ValueError, match="rows"):
        call(good, FakeGpu((T * k, H), torch.uint8), FakeGpu((T * k, H // 32), sdt), rows=T * k - 1)


def test_route_expand_noalloc_argument_errors(lib):
    """moe_route_expand_noalloc checks its arguments, then the scratch limit,
    before its first HIP call (the scratch address lookup)."""
    def call(T=4, E=8, k=2, x=FAKE, H=256, ids=FAKE, xe=FAKE):
        return status(lib, lib.moe_route_expand_noalloc(FAKE, None, T, E, k, x, H, ids, FAKE, FAKE, None, FAKE,
                                                        FAKE, xe, None))

    cap = lib.moe_noalloc_scratch_bytes()
    assert cap == 4 << 20
    assert call(k=9) == "MOE_ERR_SHAPE"
    assert call(ids=None) == "MOE_ERR_NULL"
    assert call(x=None) == "MOE_ERR_NULL"
    assert call(H=12) == "MOE_ERR_ALIGN"
    assert lib.moe_route_workspace_bytes(65536, 128, 8) > cap
    assert call(T=65536, E=128, k=8, H=64) == "MOE_ERR_UNSUPPORTED"
    assert b"scratch" in lib.moe_last_error()
    assert lib.moe_route_workspace_bytes(4096, 128, 8) <= cap  # the Qwen3-30B-A3B-shaped batch fits
    assert lib.moe_route_workspace_bytes(8192, 256, 8) <= cap  # and the DeepSeek-V3-shaped one
