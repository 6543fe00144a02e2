"""GPU parity of the comparison routers (route modes, head-shared importance
and shared-route attention) against the oracle."""

import numpy as np
import pytest
import torch

import geometry_routed_block_amd as velox
import oracle
import synth
from gpu_common import P_RTOL, check_attention_rows, check_routes_exact, say, to_np

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _gpu_inputs(wl):
    q, k, v = synth.make_qkv(wl, device=DEV)
    kbar = velox.block_mean(k[:, : wl.M * 128])
    g = torch.from_numpy(wl.g).to(DEV)
    rho = torch.from_numpy(wl.rho).to(DEV)
    coord = torch.from_numpy(np.ascontiguousarray(wl.coords, np.int32)).to(DEV)
    return q, k, v, kbar, g, rho, coord


@pytest.mark.parametrize("mode", [1, 2])
def test_route_modes_bit_exact_at_chunk48(mode):
    wl = synth.chunk48()
    wl.H = 4
    wl.params = wl.params.replace(mode=mode, theta_cov=0.5)
    say(f"route mode {mode} chunk48 H=4")
    q, k, v, kbar, g, rho, coord = _gpu_inputs(wl)
    p = velox.route_scores(q, kbar, wl.M)
    ids, lens = velox.route_select(p, g, rho, coord, wl.params)
    torch.cuda.synchronize()
    check_routes_exact(wl, p, ids, lens)


def test_shared_importance_routes_and_attention():
    wl = synth.wan13()
    wl.H = 6
    say("head-shared routes wan13 H=6")
    q, k, v, kbar, g, rho, coord = _gpu_inputs(wl)
    p1 = velox.route_scores_shared(q, kbar, wl.M)                    # [1][N][M]
    ids, lens = velox.route_select(p1, g, rho, coord, wl.params)     # [1][N][L]
    o, lse = velox.sparse_attn(q, k, v, ids[0], lens[0], wl.M, want_lse=True)
    # the same routes replicated per head through the per-head entry point
    o_rep, lse_rep = velox.sparse_attn(q, k, v, ids.expand(wl.H, -1, -1).contiguous(),
                                       lens.expand(wl.H, -1).contiguous(), wl.M, want_lse=True)
    torch.cuda.synchronize()
    qn, kn = to_np(q), to_np(k)
    qb = np.stack([oracle.block_means(qn[h:h + 1])[0] for h in range(wl.H)])
    kb = np.stack([oracle.block_means(kn[h:h + 1, : wl.M * 128])[0] for h in range(wl.H)])
    ref = oracle.importance_shared(qb, kb, wl.scale)
    np.testing.assert_allclose(p1[0].cpu().numpy(), ref, rtol=P_RTOL, atol=1e-30)
    routes = check_routes_exact(wl, p1, ids, lens)                   # one head
    assert torch.equal(o, o_rep) and torch.equal(lse, lse_rep)
    shared = [routes[0] for _ in range(wl.H)]
    rows = [(h, i) for h in range(wl.H) for i in (0, 7, 35)]
    check_attention_rows(wl, qn, kn, to_np(v), o, lse, shared, rows)
