"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs. Routes bit-exact; importance within 1e-5 relative;
attention within 2e-2 (bf16) / 1e-4 (fp32) absolute."""

import numpy as np
import pytest
import torch

import geometry_routed_block_amd as velox
import oracle
import synth
from gpu_common import (LSE_ATOL, O_ATOL, P_RTOL, check_attention_rows, check_routes_exact,
                        routes_from_gpu, run_path, sample_rows, say, to_np)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _inputs(wl, device_gen="cpu"):
    q, k, v = synth.make_qkv(wl, device=device_gen)
    return q.to(DEV), k.to(DEV), v.to(DEV), to_np(q), to_np(k), to_np(v)


def _check_p(wl, q_np, k_np, kbar, p, heads=None):
    heads = range(wl.H) if heads is None else heads
    for h in heads:
        qb = oracle.block_means(q_np[h:h + 1])
        kb = oracle.block_means(k_np[h:h + 1, : wl.M * 128])
        np.testing.assert_allclose(kbar[h].cpu().numpy(), kb[0], rtol=1e-5, atol=1e-6)
        ref = oracle.importance(qb, kb, wl.scale)[0]
        np.testing.assert_allclose(p[h].cpu().numpy(), ref, rtol=P_RTOL, atol=1e-30)


@pytest.mark.parametrize("theta,n_prev", [(0.9, 4), (0.5, 0), (1.0, 4), (0.5, 2)])
def test_tiny_full_path(theta, n_prev):
    wl = synth.tiny()
    wl.params = wl.params.replace(theta_unc=theta, n_prev=n_prev)
    say(f"tiny theta={theta} n_prev={n_prev}")
    q, k, v, qn, kn, vn = _inputs(wl)
    r = run_path(wl, q, k, v)
    _check_p(wl, qn, kn, r["kbar"], r["p"])
    routes = check_routes_exact(wl, r["p"], r["ids"], r["lens"])
    rows = [(h, i) for h in range(wl.H) for i in range(wl.N)]
    check_attention_rows(wl, qn, kn, vn, r["o"], r["lse"], routes, rows)


def test_tiny_dense():
    wl = synth.tiny()
    q, k, v, qn, kn, vn = _inputs(wl)
    o, lse = velox.dense_attn(q, k, v, wl.M, want_lse=True)
    rows = [(h, i) for h in range(wl.H) for i in range(wl.N)]
    check_attention_rows(wl, qn, kn, vn, o, lse, None, rows, dense=True)


def test_wan13_full_path():
    wl = synth.wan13()
    say("wan13 full path")
    q, k, v, qn, kn, vn = _inputs(wl)
    r = run_path(wl, q, k, v)
    _check_p(wl, qn, kn, r["kbar"], r["p"])
    routes = check_routes_exact(wl, r["p"], r["ids"], r["lens"])
    lens = r["lens"].cpu().numpy()
    cov = wl.rho >= np.float32(0.9)
    assert np.all(lens[:, cov] <= wl.params.K_cov) and np.all(lens[:, ~cov] <= wl.params.K_unc)
    check_attention_rows(wl, qn, kn, vn, r["o"], r["lse"], routes, sample_rows(wl, 24, 5))
    o_d, lse_d = velox.dense_attn(q, k, v, wl.M, want_lse=True)
    check_attention_rows(wl, qn, kn, vn, o_d, lse_d, None, sample_rows(wl, 6, 6), dense=True)


@pytest.mark.parametrize("frac", [0.0, 0.5, 1.0])
def test_chunk48_coverage_sweep(frac):
    """Coverage sweep at the chunk-48 shape: every route bit-exact, and
    attention on sampled rows of covered and uncovered blocks."""
    wl = synth.sweep(frac)
    say(f"sweep coverage {frac}")
    q, k, v = synth.make_qkv(wl, device=DEV)
    r = run_path(wl, q, k, v)
    routes = check_routes_exact(wl, r["p"], r["ids"], r["lens"])
    lens = r["lens"].cpu().numpy()
    cov = wl.rho >= np.float32(wl.params.eta_cov)
    assert cov.mean() == pytest.approx(frac, abs=1 / wl.N)
    assert (lens[:, cov] <= wl.params.K_cov).all() and (lens[:, ~cov] <= wl.params.K_unc).all()
    assert lens.min() >= wl.params.n_prev
    rows = sample_rows(wl, 10, 40 + int(frac * 10))
    heads = sorted({h for h, _ in rows})
    sub = synth.Workload(**{**wl.__dict__, "H": len(heads)})
    qn, kn, vn = to_np(q[heads]), to_np(k[heads]), to_np(v[heads])
    sub_rows = [(heads.index(h), i) for h, i in rows]
    check_attention_rows(sub, qn, kn, vn, r["o"][heads], r["lse"][heads],
                         [routes[h] for h in heads], sub_rows)


def test_sparse_with_every_tile_equals_dense_bitwise():
    wl = synth.wan13()
    q, k, v, *_ = _inputs(wl)
    ids = torch.arange(wl.M, dtype=torch.int32, device=DEV).repeat(wl.H, wl.N, 1).contiguous()
    lens = torch.full((wl.H, wl.N), wl.M, dtype=torch.int32, device=DEV)
    o_s, l_s = velox.sparse_attn(q, k, v, ids, lens, wl.M, want_lse=True)
    o_d, l_d = velox.dense_attn(q, k, v, wl.M, want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o_s, o_d) and torch.equal(l_s, l_d)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_unit_values_give_unit_output(dtype):
    wl = synth.wan13() if dtype == "bf16" else synth.tiny()
    q, k, v, *_ = _inputs(wl)
    v = torch.ones_like(v)
    r = run_path(wl, q, k, v)
    err = (r["o"].float() - 1.0).abs().max().item()
    assert err <= (O_ATOL[dtype] if dtype == "bf16" else 1e-6), err


def test_deterministic_reruns():
    wl = synth.wan13()
    q, k, v, *_ = _inputs(wl)
    a = run_path(wl, q, k, v)
    b = run_path(wl, q, k, v)
    for key in ("kbar", "p", "ids", "lens", "o", "lse"):
        assert torch.equal(a[key], b[key]), key


def test_empty_history_attends_current_chunk_only():
    wl = synth.tiny()
    wl.M = 0
    wl.g = np.zeros((wl.N, 0), np.float32)
    wl.params = wl.params.replace(n_prev=0)
    wl.coords = wl.coords[16:]
    q, k, v, qn, kn, vn = _inputs(wl)
    k = k[:, 16 * 128:].contiguous()
    v = v[:, 16 * 128:].contiguous()
    kn, vn = kn[:, 16 * 128:], vn[:, 16 * 128:]
    r = run_path(wl, q, k, v)
    assert r["lens"].cpu().numpy().max() == 0
    assert (r["ids"].cpu().numpy() == -1).all()
    routes = [[[] for _ in range(wl.N)] for _ in range(wl.H)]
    rows = [(h, i) for h in range(wl.H) for i in range(wl.N)]
    check_attention_rows(wl, qn, kn, vn, r["o"], r["lse"], routes, rows)


def test_without_current_chunk_and_empty_rows():
    wl = synth.tiny()
    q, k, v, qn, kn, vn = _inputs(wl)
    r = run_path(wl, q, k, v, include_current=False)
    routes = routes_from_gpu(r["ids"], r["lens"])
    rows = [(h, i) for h in range(wl.H) for i in range(wl.N)]
    check_attention_rows(wl, qn, kn, vn, r["o"], r["lse"], routes, rows, include_current=False)
    # rows with no tile at all: o = 0, lse = -inf
    lens0 = torch.zeros_like(r["lens"])
    o, lse = velox.sparse_attn(q, k, v, r["ids"], lens0, wl.M, include_current=False,
                               want_lse=True)
    assert torch.all(o == 0) and torch.all(torch.isinf(lse)) and torch.all(lse < 0)


def test_reservation_larger_than_cap():
    wl = synth.tiny()
    wl.params = wl.params.replace(K_cov=2, K_unc=3, n_prev=5)
    q, k, v, qn, kn, vn = _inputs(wl)
    r = run_path(wl, q, k, v)
    routes = check_routes_exact(wl, r["p"], r["ids"], r["lens"])
    for h in range(wl.H):
        for i in range(wl.N):
            assert set(range(11, 16)) <= set(routes[h][i])


def test_long_cap_and_mass_cut_ragged():
    """M not a multiple of any kernel tile, K close to M, several thresholds."""
    wl = synth.wan13()
    for theta in (0.3, 0.6, 0.95):
        wl.params = wl.params.replace(K_cov=140, K_unc=143, theta_cov=theta, theta_unc=theta,
                                      n_prev=7, neigh26=1)
        q, k, v, *_ = _inputs(wl) if theta == 0.3 else (q, k, v)
        r = run_path(wl, q, k, v)
        check_routes_exact(wl, r["p"], r["ids"], r["lens"])


@pytest.mark.parametrize("d,dtype", [(64, "bf16"), (128, "f32")])
def test_other_head_dims(d, dtype):
    wl = synth.tiny()
    wl.d, wl.dtype = d, dtype
    q, k, v, qn, kn, vn = _inputs(wl)
    r = run_path(wl, q, k, v)
    _check_p(wl, qn, kn, r["kbar"], r["p"])
    routes = check_routes_exact(wl, r["p"], r["ids"], r["lens"])
    rows = [(h, i) for h in range(wl.H) for i in range(wl.N)]
    check_attention_rows(wl, qn, kn, vn, r["o"], r["lse"], routes, rows)
