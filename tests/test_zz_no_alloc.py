"""velox_sparse_attn_noalloc (the entry point for callers that cannot allocate,
whose unit schedule lives in the library's fixed device array) against
velox_sparse_attn with a caller workspace, through the C ABI: outputs and LSE
bitwise equal, on two calls in a row, the second smaller than the first."""

import ctypes

import numpy as np
import pytest
import torch

import geometry_routed_block_amd as velox
from geometry_routed_block_amd import _lib
import synth
from gpu_common import say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _inputs(wl, N):
    q, k, v = synth.make_qkv(wl, device=DEV)
    q = q[:, : N * 128].contiguous()
    kbar = velox.block_mean(k[:, : wl.M * 128])
    p = velox.route_scores(q, kbar, wl.M)
    coord = np.concatenate([wl.coords[: wl.M], wl.coords[wl.M: wl.M + N]])
    ids, lens = velox.route_select(p, torch.from_numpy(wl.g[:N]).to(DEV),
                                   torch.from_numpy(wl.rho[:N]).to(DEV),
                                   torch.from_numpy(np.ascontiguousarray(coord, np.int32)).to(DEV),
                                   wl.params)
    return q, k, v, ids, lens


def _call(name, q, k, v, ids, lens, M, ws=None):
    lib = _lib.load()
    H, NT, d = q.shape
    o = torch.full_like(q, 7.0)
    lse = torch.full((H, NT), 7.0, dtype=torch.float32, device=q.device)
    args = [q.data_ptr(), k.data_ptr(), v.data_ptr(), _lib.VELOX_BF16, q.stride(0), k.stride(0), H,
            NT // 128, M, d, ctypes.c_float(1.0 / d ** 0.5), ids.data_ptr(), lens.data_ptr(),
            ids.shape[-1], 1, o.data_ptr(), lse.data_ptr()]
    if ws is not None:
        args.append(ws.data_ptr())
    args.append(torch.cuda.current_stream().cuda_stream)
    _lib.check(getattr(lib, name)(*args))
    torch.cuda.synchronize()
    return o, lse


def test_noalloc_matches_the_workspace_call_on_two_calls():
    for wl, N in ((synth.chunk48(), 36), (synth.wan13(), 35)):
        say(f"no-allocation attention: {wl.name}, H={wl.H}, N={N}, M={wl.M}")
        q, k, v, ids, lens = _inputs(wl, N)
        ws = velox.attn_workspace(q, ids.shape[-1])
        o_ref, l_ref = _call("velox_sparse_attn", q, k, v, ids, lens, wl.M, ws)
        o, l = _call("velox_sparse_attn_noalloc", q, k, v, ids, lens, wl.M)
        assert torch.equal(o, o_ref), f"{wl.name}: outputs differ"
        assert torch.equal(l, l_ref), f"{wl.name}: LSE differs"
        del q, k, v
        torch.cuda.empty_cache()
