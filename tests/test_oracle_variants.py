"""Pins of the comparison routers in the oracle: the matched model-only route,
hard geometric top-K and the head-shared importance. CPU only."""

import numpy as np
import pytest
from scipy.special import softmax

import oracle
import synth


def _rows(seed, M=60, N=6):
    rng = np.random.default_rng(seed)
    p = rng.dirichlet(np.ones(M), size=N).astype(np.float32)
    g = (rng.uniform(size=(N, M)) * (rng.uniform(size=(N, M)) < 0.4)).astype(np.float32)
    rho = np.array([0.95, 0.3, 0.92, 0.5, 0.99, 0.1], np.float32)[:N]
    return p, g, rho


BASE = synth.RouteParams(K_cov=12, K_unc=20, n_prev=4, theta_unc=0.5)


@pytest.mark.parametrize("seed", range(5))
def test_model_only_equals_fusion_with_zero_lambda(seed):
    p, g, rho = _rows(seed)
    for i in range(p.shape[0]):
        a = oracle.route_row(p[i], g[i], rho[i], BASE.replace(mode=1), p.shape[1])
        b = oracle.route_row(p[i], g[i], rho[i], BASE.replace(lam=0.0), p.shape[1])
        assert a == b


@pytest.mark.parametrize("seed", range(5))
def test_model_only_ignores_geometry_and_keeps_budgets(seed):
    p, g, rho = _rows(seed)
    prm = BASE.replace(mode=1)
    for i in range(p.shape[0]):
        a = oracle.route_row(p[i], g[i], rho[i], prm, p.shape[1])
        b = oracle.route_row(p[i], np.zeros_like(g[i]), rho[i], prm, p.shape[1])
        assert a == b
        covered = rho[i] >= prm.eta_cov
        assert len(a) == (prm.K_cov if covered else len(a))    # covered rows: full top-K_cov
        assert len(a) <= (prm.K_cov if covered else prm.K_unc)


@pytest.mark.parametrize("seed", range(5))
def test_geometry_only_ranks_covered_rows_by_overlap(seed):
    p, g, rho = _rows(seed)
    prm = BASE.replace(mode=2, theta_cov=0.3)        # a mass cut is ignored in this mode
    M = p.shape[1]
    for i in range(p.shape[0]):
        r = oracle.route_row(p[i], g[i], rho[i], prm, M)
        if rho[i] >= prm.eta_cov:
            # independent of p; equal to the model-only route of a row whose
            # importances are the overlaps themselves
            assert r == oracle.route_row(p[(i + 1) % p.shape[0]], g[i], rho[i], prm, M)
            assert r == oracle.route_row(g[i], g[i], rho[i], BASE.replace(mode=1, theta_cov=1.0), M)
            assert len(r) == prm.K_cov
            # every selected non-reserved block has overlap >= every dropped one
            sel = set(r) - set(range(M - prm.n_prev, M))
            rest = set(range(M - prm.n_prev)) - sel
            assert min(g[i][list(sel)]) >= max(g[i][list(rest)])
        else:   # uncovered rows keep the model route
            assert r == oracle.route_row(p[i], g[i], rho[i], BASE, M)


def test_shared_importance_reduces_to_per_head_and_to_concatenation():
    rng = np.random.default_rng(4)
    H, N, M, d = 3, 5, 40, 16
    qb = rng.normal(size=(H, N, d))
    kb = rng.normal(size=(H, M, d))
    s = 0.25
    # one head: the per-head importance
    assert np.allclose(oracle.importance_shared(qb[:1], kb[:1], s), oracle.importance(qb[:1], kb[:1], s)[0])
    # identical heads: the per-head importance
    rep_q, rep_k = np.repeat(qb[:1], H, 0), np.repeat(kb[:1], H, 0)
    assert np.allclose(oracle.importance_shared(rep_q, rep_k, s), oracle.importance(qb[:1], kb[:1], s)[0])
    # head-mean of inner products = inner product of head-concatenated means / H
    qcat = qb.transpose(1, 0, 2).reshape(N, H * d)
    kcat = kb.transpose(1, 0, 2).reshape(M, H * d)
    ref = softmax(s * (qcat @ kcat.T) / H, axis=1)
    assert np.allclose(oracle.importance_shared(qb, kb, s), ref, rtol=1e-12, atol=1e-15)
    assert np.allclose(oracle.importance_shared(qb, kb, s).sum(1), 1.0)
