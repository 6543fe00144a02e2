"""GPU parity of route materialisation on crafted importances: exact ties
(routes decided by block index alone), zero weights, caps that take every
candidate, caps above the radix-select limit (the sort fallback), and
26-neighbour safeguards on a history long enough that the kernel tests the
neighbours in its late loop. Routes are compared bit for bit with the
oracle."""

import numpy as np
import pytest
import torch

import geometry_routed_block_amd as velox
import oracle
from synth import RouteParams
from gpu_common import say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _rows(kind, H, N, M, rng):
    p = np.empty((H, N, M), np.float32)
    for h in range(H):
        for i in range(N):
            if kind == "uniform":                      # every weight equal
                row = np.full(M, 1.0 / M)
            elif kind == "zeros":                      # most weights exactly zero
                row = np.zeros(M)
                hot = rng.choice(M, 40, replace=False)
                row[hot] = rng.random(40)
            elif kind == "plateaus":                   # a few distinct values, many ties
                row = rng.integers(1, 5, M).astype(np.float64)
            else:                                      # continuous
                row = rng.lognormal(0.0, 2.0, M)
            p[h, i] = (row / row.sum()).astype(np.float32)
    return p


def _check(p, g, rho, prm, coords=None):
    H, N, M = p.shape
    ids, lens = velox.route_select(torch.from_numpy(p).to(DEV), torch.from_numpy(g).to(DEV),
                                   torch.from_numpy(rho).to(DEV),
                                   None if coords is None else torch.from_numpy(coords).to(DEV), prm)
    torch.cuda.synchronize()
    ids, lens = ids.cpu().numpy(), lens.cpu().numpy()
    for h in range(H):
        for i in range(N):
            ref = oracle.route_row(p[h, i], g[i], rho[i], prm, M, coords, i)
            got = ids[h, i, : lens[h, i]].tolist()
            assert got == ref, f"route mismatch at head {h} block {i}"
            assert np.all(ids[h, i, lens[h, i]:] == -1)


@pytest.mark.parametrize("kind", ["uniform", "zeros", "plateaus", "continuous"])
@pytest.mark.parametrize("M,K_cov,K_unc,theta", [(700, 40, 90, 0.6), (1300, 1100, 1250, 0.97),
                                                 (301, 400, 400, 0.999)])
def test_select_ties_zeros_and_caps(kind, M, K_cov, K_unc, theta):
    say(f"select {kind} M={M} K=({K_cov},{K_unc}) theta={theta}")
    rng = np.random.default_rng(M + len(kind))
    H, N = 2, 6
    p = _rows(kind, H, N, M, rng)
    g = rng.random((N, M)).astype(np.float32) * 0.4
    rho = np.array([0.95, 0.2, 1.0, 0.0, 0.91, 0.5], np.float32)
    prm = RouteParams(K_cov=K_cov, K_unc=K_unc, theta_cov=theta, theta_unc=theta, n_prev=5)
    _check(p, g, rho, prm)


def test_select_without_reservation_takes_everything():
    rng = np.random.default_rng(5)
    H, N, M = 1, 4, 257
    p = _rows("plateaus", H, N, M, rng)
    g = np.zeros((N, M), np.float32)
    rho = np.zeros(N, np.float32)
    prm = RouteParams(K_cov=M, K_unc=M, theta_unc=1.0, n_prev=0)
    _check(p, g, rho, prm)


def test_route_check_accepts_routes_and_flags_each_fault():
    rng = np.random.default_rng(9)
    H, N, M = 2, 6, 300
    p = _rows("continuous", H, N, M, rng)
    g = rng.random((N, M)).astype(np.float32) * 0.4
    rho = np.array([0.95, 0.2, 1.0, 0.0, 0.91, 0.5], np.float32)
    ids, lens = velox.route_select(torch.from_numpy(p).to(DEV), torch.from_numpy(g).to(DEV),
                                   torch.from_numpy(rho).to(DEV), None,
                                   RouteParams(K_cov=40, K_unc=60, theta_unc=0.8, n_prev=3))
    assert velox.check_routes(ids, lens, M) == (0, -1)
    L = ids.shape[-1]
    faults = {3: lambda r, n: r.__setitem__(1, r[0]),            # duplicate id
              5: lambda r, n: r.__setitem__(slice(0, 2), r[[1, 0]]),   # descending pair
              7: lambda r, n: r.__setitem__(n - 1, M),           # id past the history
              8: lambda r, n: r.__setitem__(0, -3)}              # negative id
    ids_np, lens_np = ids.cpu().numpy().reshape(H * N, L), lens.cpu().numpy().reshape(H * N)
    for row, f in faults.items():
        assert lens_np[row] >= 2
        f(ids_np[row], lens_np[row])
    lens_np[10] = L + 1                                          # longer than the buffer
    lens_np[11] = -1
    bad, first = velox.check_routes(torch.from_numpy(ids_np).to(DEV), torch.from_numpy(lens_np).to(DEV), M)
    assert (bad, first) == (6, 3)


def test_select_neighbours_on_a_long_history():
    # 9000 history blocks (a 30 x 15 x 20 block grid, frame-major) and query
    # blocks one frame later: more than 32 candidate rows per thread, where the
    # kernel fills the neighbour bits in its late loop instead of during the
    # weight pass
    rng = np.random.default_rng(21)
    H, N, T, Y, X = 1, 4, 30, 15, 20
    M = T * Y * X
    hist = np.stack(np.meshgrid(np.arange(T), np.arange(Y), np.arange(X), indexing="ij"), -1).reshape(-1, 3)
    query = np.array([[T, 0, 0], [T, 7, 9], [T, 14, 19], [T + 1, 3, 3]])   # corner, middle, corner, two frames on
    coords = np.ascontiguousarray(np.concatenate([hist, query]).astype(np.int32))
    say(f"select with neighbours, M={M}")
    p = _rows("continuous", H, N, M, rng)
    g = rng.random((N, M)).astype(np.float32) * 0.4
    rho = np.array([0.95, 0.2, 1.0, 0.5], np.float32)
    prm = RouteParams(K_cov=60, K_unc=90, theta_unc=0.7, n_prev=X, neigh26=1)   # reserves one grid row
    _check(p, g, rho, prm, coords)
