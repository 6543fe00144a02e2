"""The routed step captured in a HIP graph: importance, routes and sparse
attention (and the split-row variant) recorded once and replayed. Every replay,
with eager work and synchronisations in between, must reproduce the eager
results bit for bit, also after the inputs change in place."""

import numpy as np
import pytest
import torch

import geometry_routed_block_amd as velox
import synth
from gpu_common import say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.mark.parametrize("n_split", [1, 3])
def test_step_replays_match_eager(n_split):
    wl = synth.wan13()
    say(f"graph capture of the routed step, n_split={n_split}")
    q, k, v = synth.make_qkv(wl, device=DEV)
    kbar = velox.block_mean(k[:, : wl.M * 128])
    g = torch.from_numpy(wl.g).to(DEV)
    rho = torch.from_numpy(wl.rho).to(DEV)
    coord = torch.from_numpy(np.ascontiguousarray(wl.coords, np.int32)).to(DEV)
    L = velox.route_bound(wl.params, wl.M)
    p = torch.empty(wl.H, wl.N, wl.M, device=DEV)
    ids = torch.empty(wl.H, wl.N, L, dtype=torch.int32, device=DEV)
    lens = torch.empty(wl.H, wl.N, dtype=torch.int32, device=DEV)
    o = torch.empty_like(q)
    lse = torch.empty(wl.H, wl.N * 128, device=DEV)
    ws = velox.split_workspace(q, n_split) if n_split > 1 else None

    def step():
        velox.route_scores(q, kbar, wl.M, out=p)
        velox.route_select(p, g, rho, coord, wl.params, L=L, route_ids=ids, route_len=lens)
        velox.sparse_attn(q, k, v, ids, lens, wl.M, out=o, lse=lse, n_split=n_split, workspace=ws)

    def eager_copy():
        step()
        torch.cuda.synchronize()
        return [t.clone() for t in (p, ids, lens, o, lse)]

    ref = eager_copy()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):       # warm-up on the capture stream
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (p, o, lse):
            t.fill_(-7.0)
        ids.fill_(-7)
        lens.fill_(-7)
        graph.replay()
        torch.cuda.synchronize()
        _ = (q.float() * 2).sum().item()          # eager work between replays
        for a, b in zip((p, ids, lens, o, lse), ref):
            assert torch.equal(a, b), f"replay {rep} differs"
    # new inputs in place: the replay follows them
    q.mul_(0.5)
    ref2 = eager_copy()
    graph.replay()
    torch.cuda.synchronize()
    for a, b in zip((p, ids, lens, o, lse), ref2):
        assert torch.equal(a, b)
    assert not torch.equal(ref2[0], ref[0])
