"""dg_route_noalloc (routing with its scratch in a static device array, for
callers that cannot allocate) against dg_test_route (the same kernels with
the context's workspace), bit for bit, on two calls in a row, the second
with fewer rows; sizes beyond the static array are refused on the host."""
import ctypes

import numpy as np
import pytest
import torch

from block_discrete_diffusion_dg_amd import binding as B
from block_discrete_diffusion_dg_amd import synth
from tests.gpu_util import make_engine, say

pytestmark = pytest.mark.gpu


def _logits(rows, E, seed):
    z = synth.hashed_normal((rows, E), synth.tensor_seed(seed, 0, "z"), 1.0, dtype=torch.float32).clone()
    z[0, 5] = z[0, 3] = 9.0  # an exact tie at the top
    z[1, :] = 0.25           # a row of equal logits
    return z.cuda()


def _noalloc(lib, z, k):
    rows, E = z.shape
    dev = z.device
    out = dict(idx=torch.full((rows, k), -1, dtype=torch.int32, device=dev),
               w=torch.full((rows, k), -1.0, dtype=torch.float32, device=dev),
               cnt=torch.full((E,), -1, dtype=torch.int32, device=dev),
               off=torch.full((E + 1,), -1, dtype=torch.int32, device=dev),
               perm=torch.full((rows * k,), -1, dtype=torch.int32, device=dev),
               slot=torch.full((rows, k), -1, dtype=torch.int32, device=dev))
    st = lib.dg_route_noalloc(torch.cuda.current_stream().cuda_stream, z.data_ptr(), rows, E, k,
                              *[out[n].data_ptr() for n in ("idx", "w", "cnt", "off", "perm", "slot")])
    assert st == B.DG_OK, st
    return out


def test_route_noalloc_matches_the_workspace_path():
    model = synth.FULL
    lib = B.load()
    E, k = model.n_experts, model.top_k
    rows_big = B.ROUTE_NOALLOC_MAX_ROWS
    import dataclasses
    eng, _ = make_engine(dataclasses.replace(model, n_layers=0), max_ctx=4 * model.canvas, max_rows=rows_big)
    for rows, seed in [(rows_big, 1), (37, 2)]:  # the second call is smaller: stale scratch must not matter
        say(f"[noalloc] rows={rows}")
        z = _logits(rows, E, seed)
        got = _noalloc(lib, z, k)
        want = eng.test_route(z)
        torch.cuda.synchronize()
        for n in ("idx", "w", "cnt", "off", "perm", "slot"):
            assert torch.equal(got[n].cpu(), want[n].cpu()), (rows, n)
    # refused on the host, nothing launched
    z = _logits(4, E, 3)
    dummy = z.data_ptr()
    s = torch.cuda.current_stream().cuda_stream
    assert lib.dg_route_noalloc(s, dummy, rows_big + 1, E, k, *[dummy] * 6) == B.DG_ECAPACITY
    assert lib.dg_route_noalloc(s, dummy, 4, 129, k, *[dummy] * 6) == B.DG_EINVAL
    assert lib.dg_route_noalloc(s, None, 4, E, k, *[dummy] * 6) == B.DG_EINVAL
