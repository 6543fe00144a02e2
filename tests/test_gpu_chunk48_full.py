"""GPU parity at the benchmarked chunk-48 shape (40 heads, d 128, bf16, 36
query blocks, 1692 history blocks), in the launch configuration bench.py
times: every route bit-exact, importance of every head, attention of all
1440 (head, query block) rows and dense attention of one whole head against
the oracle. Host memory stays bounded: the oracle works one head at a time."""

import numpy as np
import pytest
import torch

import geometry_routed_block_amd as velox
import oracle
import synth
from gpu_common import (LSE_ATOL, O_ATOL, P_RTOL, check_routes_exact, run_path, say, to_np)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def c48():
    wl = synth.chunk48()
    say("chunk48: generating inputs on the GPU")
    q, k, v = synth.make_qkv(wl, device=DEV)
    r = run_path(wl, q, k, v)
    return wl, q, k, v, r


def _head(x, h, rows=None):
    return to_np(x[h:h + 1] if rows is None else x[h:h + 1, :rows])


def test_chunk48_routes_and_importance_every_head(c48):
    wl, q, k, v, r = c48
    say("chunk48: all 1440 routes")
    check_routes_exact(wl, r["p"], r["ids"], r["lens"])
    lens = r["lens"].cpu().numpy()
    cov = wl.rho >= np.float32(wl.params.eta_cov)
    assert (lens[:, cov] == wl.params.K_cov).all() and (lens[:, ~cov] == wl.params.K_unc).all()
    for h in range(wl.H):
        qb = oracle.block_means(_head(q, h))
        kb = oracle.block_means(_head(k, h, wl.M * 128))
        np.testing.assert_allclose(r["kbar"][h].cpu().numpy(), kb[0], rtol=1e-5, atol=1e-6)
        np.testing.assert_allclose(r["p"][h].cpu().numpy(), oracle.importance(qb, kb, wl.scale)[0],
                                   rtol=P_RTOL, atol=1e-30)
    say("chunk48: importance of 40 heads ok")


@pytest.mark.parametrize("heads", [range(0, 20), range(20, 40)], ids=["heads0-19", "heads20-39"])
def test_chunk48_attention_every_row(c48, heads):
    wl, q, k, v, r = c48
    ids, lens = r["ids"].cpu().numpy(), r["lens"].cpu().numpy()
    o_all, lse_all = r["o"], r["lse"]
    tol, ltol = O_ATOL["bf16"], LSE_ATOL["bf16"]
    worst = 0.0
    for h in heads:
        qn, kn, vn = _head(q, h), _head(k, h), _head(v, h)
        o_h = to_np(o_all[h]).astype(np.float64)
        lse_h = lse_all[h].cpu().numpy()
        for i in range(wl.N):
            route = ids[h, i, : lens[h, i]].tolist()
            ref_o, ref_l = oracle.sparse_attention_block(qn, kn, vn, wl.scale, 0, i, route, wl.M, wl.N)
            err = np.abs(o_h[i * 128:(i + 1) * 128] - ref_o).max()
            lerr = np.abs(lse_h[i * 128:(i + 1) * 128] - ref_l).max()
            assert err <= tol, f"O error {err:.3g} at head {h} block {i}"
            assert lerr <= ltol, f"LSE error {lerr:.3g} at head {h} block {i}"
            worst = max(worst, err)
        say(f"chunk48: head {h}: 36 rows ok (worst |dO| so far {worst:.2e})")


def test_chunk48_dense_one_whole_head(c48):
    wl, q, k, v, r = c48
    h = 23
    o_d, lse_d = velox.dense_attn(q, k, v, wl.M, want_lse=True)
    torch.cuda.synchronize()
    qn, kn, vn = _head(q, h), _head(k, h), _head(v, h)
    o_h = to_np(o_d[h]).astype(np.float64)
    lse_h = lse_d[h].cpu().numpy()
    for i in range(wl.N):
        ref_o, ref_l = oracle.dense_attention_block(qn, kn, vn, wl.scale, 0, i, wl.M, wl.N)
        assert np.abs(o_h[i * 128:(i + 1) * 128] - ref_o).max() <= O_ATOL["bf16"], i
        assert np.abs(lse_h[i * 128:(i + 1) * 128] - ref_l).max() <= LSE_ATOL["bf16"], i
    say("chunk48: dense head 23 ok")
