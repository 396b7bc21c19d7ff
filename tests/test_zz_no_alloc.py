"""moe_route_expand_noalloc (the route + expand call whose workspace is the
library's built-in device scratch) against moe_route_expand with a caller
workspace, through the C ABI on an MI355X.  Every output is compared bit for
bit (the same kernels run on the same inputs; ids, maps and copies are
integer or bit work, the weights come from the same instructions).

Calls run back to back on one stream, each one smaller than the one before,
so each call finds the scratch holding what the previous, larger call left:
the placing destination-order expand (its chunk claims and count rows in the
scratch), the three-launch route (a histogram matrix too large for the
two-launch form), the two-launch route with the copy in its place launch,
then the one-launch dispatch (T <= 64)."""
import sys

import numpy as np
import pytest

import gpu_util as G
from moe_glue_amd import inputs

pytestmark = pytest.mark.gpu

# (T, E, k, H), largest first
SHAPES = [(4096, 128, 8, 2048), (5000, 512, 4, 64), (3000, 64, 6, 1024), (700, 128, 8, 512), (300, 16, 4, 64),
          (48, 128, 8, 2048), (5, 8, 2, 256)]


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _outputs(T, E, k, H, dev, fill):
    import torch

    i32, f32 = torch.int32, torch.float32
    d = {
        "topk_ids": torch.full((T, k), fill, dtype=i32, device=dev),
        "topk_weights": torch.full((T, k), float(fill), dtype=f32, device=dev),
        "expert_offsets": torch.full((E + 1,), fill, dtype=i32, device=dev),
        "expert_counts": torch.full((E,), fill, dtype=i32, device=dev),
        "dest_of_src": torch.full((T * k,), fill, dtype=i32, device=dev),
        "src_of_dest": torch.full((T * k,), fill, dtype=i32, device=dev),
        "x_expanded": torch.full((T * k, H), fill, dtype=torch.int16, device=dev).view(torch.bfloat16),
    }
    return d


def _args(d):
    p = lambda key: d[key].data_ptr()  # noqa: E731
    return (p("topk_ids"), p("topk_weights"), p("expert_offsets"), p("expert_counts"), p("dest_of_src"),
            p("src_of_dest"), p("x_expanded"))


def _host(d):
    return {key: G.to_host(v) for key, v in d.items()}


@pytest.mark.parametrize("seed", [0, 1])
def test_noalloc_matches_route_expand_on_shrinking_calls(seed):
    import torch
    import moe_glue_amd as mg

    dev = G.device()
    lib = mg.load()
    stream = torch.cuda.current_stream(dev).cuda_stream
    cap = lib.moe_noalloc_scratch_bytes()
    for (T, E, k, H) in SHAPES:
        need = lib.moe_route_workspace_bytes(T, E, k)
        assert 0 < need <= cap, (T, E, k, need, cap)
        cfg = inputs.Config("noalloc", T=T, H=H, E=E, k=k, I=8)
        inp = inputs.make_inputs(cfg, seed, parts=("x", "logits"))
        logits = G.to_dev(inp["logits"], dev)
        x = G.to_dev(inp["x"], dev)
        _log(f"[noalloc] T={T} E={E} k={k} H={H} seed={seed} workspace={need} B")
        ref = _outputs(T, E, k, H, dev, -7)
        ws = torch.randint(0, 256, (need,), dtype=torch.uint8, device=dev)  # caller workspace, garbage-filled
        got = _outputs(T, E, k, H, dev, -9)
        rc = lib.moe_route_expand(logits.data_ptr(), None, T, E, k, x.data_ptr(), H, *_args(ref)[:6],
                                  ref["x_expanded"].data_ptr(), ws.data_ptr(), need, stream)
        assert rc == 0, lib.moe_last_error().decode()
        rc = lib.moe_route_expand_noalloc(logits.data_ptr(), None, T, E, k, x.data_ptr(), H, *_args(got)[:6],
                                          got["x_expanded"].data_ptr(), stream)
        assert rc == 0, lib.moe_last_error().decode()
        torch.cuda.synchronize(dev)
        r, g = _host(ref), _host(got)
        for key in r:
            assert np.array_equal(r[key].view(np.uint8), g[key].view(np.uint8)), f"T={T} E={E}: {key} differs"


def test_noalloc_rejects_batches_beyond_the_scratch():
    import moe_glue_amd as mg

    lib = mg.load()
    cap = lib.moe_noalloc_scratch_bytes()
    T, E, k = 65536, 128, 8  # ~6 MiB of workspace
    assert lib.moe_route_workspace_bytes(T, E, k) > cap
    with pytest.raises(ValueError, match="scratch"):
        mg.route_expand_noalloc(G.to_dev(np.zeros((T, E), np.float32), G.device()), k,
                                G.to_dev(np.zeros((T, 64), np.uint16), G.device()))
