"""Reference-frame safeguards and the route input report on the GPU.

[digest] Method steps, step 4 (eq. 14) and [onedev] "What differs": the
reference-frame blocks are added as safeguards outside the budget, next to the
26-neighbourhood. Routes are compared bit for bit with the oracle fed the same
fp32 importances, for reference ids inside the reservation, among the
budget-selected blocks, duplicated and out of range (ignored), with the
neighbour safeguards on; eagerly and replayed from a captured HIP graph whose
reference ids live in a caller-owned device tensor.

The input report: rows whose p or g break the fixed-point preconditions of the
mass cut are counted in a device status word."""

import numpy as np
import pytest
import torch

import geometry_routed_block_amd as velox
import oracle
import synth
from gpu_common import check_routes_exact, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _route_inputs(wl, device=DEV):
    q, k, v = synth.make_qkv(wl, device="cpu" if wl.M < 1000 else DEV)
    q, k = q.to(DEV), k.to(DEV)
    kbar = velox.block_mean(k[:, : wl.M * 128])
    p = velox.route_scores(q, kbar, wl.M)
    g = torch.from_numpy(wl.g).to(DEV)
    rho = torch.from_numpy(wl.rho).to(DEV)
    coord = torch.from_numpy(np.ascontiguousarray(wl.coords, np.int32)).to(DEV)
    return p, g, rho, coord


@pytest.mark.parametrize("wlname", ["tiny", "chunk48"])
def test_ref_ids_bit_exact(wlname):
    wl = synth.tiny() if wlname == "tiny" else synth.chunk48()
    M = wl.M
    p, g, rho, coord = _route_inputs(wl)
    # ids inside the reservation (last history ids), a low id the budget may
    # select anyway, a duplicate, and out-of-range ids (negative, == M, > M)
    ref = [M - 1, M - 2, 0, 3, 3, M // 2, -1, M, M + 7]
    if wlname == "chunk48":
        ref += [17, 400, 999, 1200, 1200]
    prm = wl.params.replace(ref_ids=tuple(ref), neigh26=1)
    say(f"ref ids on {wlname}: {ref}")
    ids, lens = velox.route_select(p, g, rho, coord, prm)
    torch.cuda.synchronize()
    routes = check_routes_exact(wl.__class__(**{**wl.__dict__, "params": prm}), p, ids, lens)
    valid = {r for r in ref if 0 <= r < M}
    for h in range(wl.H):
        for i in range(wl.N):
            assert valid <= set(routes[h][i])
    # the same call with the ids in a caller-owned device tensor
    ref_t = torch.tensor(ref, dtype=torch.int32, device=DEV)
    ids2, lens2 = velox.route_select(p, g, rho, coord, prm.replace(ref_ids=()), ref_ids=ref_t)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids2) and torch.equal(lens, lens2)


def test_ref_ids_with_small_reservation_tiny():
    """n_prev smaller than a chunk: neighbours and reference ids both add
    blocks the budget did not take, with L at its bound."""
    wl = synth.tiny()
    for n_prev in (0, 2):
        prm = wl.params.replace(n_prev=n_prev, ref_ids=(1, 5, 9, 9, 15, 16, -4), neigh26=1,
                                K_cov=3, K_unc=4)
        p, g, rho, coord = _route_inputs(wl)
        L = velox.route_bound(prm, wl.M)
        ids, lens = velox.route_select(p, g, rho, coord, prm, L=L)
        torch.cuda.synchronize()
        check_routes_exact(wl.__class__(**{**wl.__dict__, "params": prm}), p, ids, lens)


def test_ref_ids_graph_replay_follows_the_device_tensor():
    wl = synth.wan13()
    p, g, rho, coord = _route_inputs(wl)
    prm = wl.params.replace(neigh26=0)
    ref_t = torch.tensor([5, 77, 142, 200, -1], dtype=torch.int32, device=DEV)
    L = velox.route_bound(prm, wl.M) + ref_t.numel()
    ids = torch.empty(wl.H, wl.N, L, dtype=torch.int32, device=DEV)
    lens = torch.empty(wl.H, wl.N, dtype=torch.int32, device=DEV)

    def step():
        velox.route_select(p, g, rho, coord, prm, L=L, route_ids=ids, route_len=lens, ref_ids=ref_t)

    def expect(ref_list):
        prm_r = prm.replace(ref_ids=tuple(ref_list))
        return check_routes_exact(wl.__class__(**{**wl.__dict__, "params": prm_r}), p, ids, lens)

    step()
    torch.cuda.synchronize()
    expect([5, 77, 142, 200, -1])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep, new in enumerate(([5, 77, 142, 200, -1], [0, 1, 2, 3, 4], [140, 141, 142, 141, 9000])):
        ref_t.copy_(torch.tensor(new, dtype=torch.int32))
        ids.fill_(-7)
        lens.fill_(-7)
        graph.replay()
        torch.cuda.synchronize()
        _ = (p * 2).sum().item()          # eager work between replays
        expect(new)
        say(f"replay {rep} with ref ids {new}: routes exact")


def test_input_report_flags_bad_rows():
    H, N, M = 2, 4, 50
    rng = np.random.default_rng(7)
    p = rng.random((H, N, M)).astype(np.float32)
    p /= p.sum(axis=2, keepdims=True)
    g = rng.random((N, M)).astype(np.float32)
    g[1] = 1.0                                   # covered row 1: every block at full overlap
    rho = np.array([0.3, 0.95, 0.3, 0.3], np.float32)
    prm = synth.RouteParams(lam=14.0, theta_cov=0.5, theta_unc=0.8, K_cov=20, K_unc=30)
    p[0, 1] *= np.float32(1.2)                   # sum 1.2: Z = 15 * 1.2 * 2^60 >= 2^64 under the cut
    p[1, 2, 7] = -1e-3                           # negative importance
    g[3, 11] = 1.5                               # overlap above 1 (rows 3 of both heads)
    status = torch.full((2,), -5, dtype=torch.int32, device=DEV)
    pd, gd, rd = (torch.from_numpy(x).to(DEV) for x in (p, g, rho))
    ids, lens = velox.route_select(pd, gd, rd, None, prm, status=status)
    torch.cuda.synchronize()
    assert status.cpu().tolist() == [4, 1]       # rows 0*4+1, 0*4+3, 1*4+2, 1*4+3
    ids_np, lens_np = ids.cpu().numpy(), lens.cpu().numpy()
    for h in range(H):
        for i in range(N):
            r = ids_np[h, i, : lens_np[h, i]]
            assert (np.diff(r) > 0).all() and (r >= 0).all() and (r < M).all()
            if (h * N + i) not in (1, 3, 6, 7):
                assert r.tolist() == oracle.route_row(p[h, i], g[i], rho[i], prm, M, None, i)
    # NaN importance, and a clean call that resets the report
    p2 = p.copy()
    p2[0, 0, 3] = np.nan
    velox.route_select(torch.from_numpy(p2).to(DEV), gd, rd, None, prm, status=status)
    torch.cuda.synchronize()
    assert status.cpu().tolist()[0] == 5 and status.cpu().tolist()[1] == 0
    ok = rng.random((H, N, M)).astype(np.float32)
    ok /= ok.sum(axis=2, keepdims=True)
    g_ok = np.clip(g, 0, 1)
    velox.route_select(torch.from_numpy(ok).to(DEV), torch.from_numpy(g_ok).to(DEV), rd, None, prm,
                       status=status)
    torch.cuda.synchronize()
    assert status.cpu().tolist() == [0, H * N]
