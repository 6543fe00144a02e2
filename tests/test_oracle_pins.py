"""Pins of the CPU oracle against things other than itself: closed forms,
library routines, hand-worked values from the pages' formulas, brute force on
tiny inputs and a statistic the pages print. CPU only."""

import json
import os
from fractions import Fraction
from itertools import combinations

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import synth
from synth import RouteParams

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- block means

def test_block_mean_constant_block():
    x = np.zeros((1, 256, 4))
    x[0, :128] = [1.0, -2.0, 0.5, 3.0]
    x[0, 128:] = 7.0
    m = oracle.block_means(x)
    assert np.array_equal(m[0, 0], [1.0, -2.0, 0.5, 3.0])
    assert np.array_equal(m[0, 1], [7.0] * 4)


def test_block_mean_explicit_loop():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((2, 384, 5))
    m = oracle.block_means(x)
    for h in range(2):
        for b in range(3):
            for c in range(5):
                s = 0.0
                for t in range(128):
                    s += x[h, b * 128 + t, c]
                assert m[h, b, c] == pytest.approx(s / 128, abs=1e-13)


def test_importance_logit_is_mean_of_tile_logits():
    """q̄·k̄ equals the mean of the 128x128 tile of q_a·k_b (bilinearity)."""
    rng = np.random.default_rng(4)
    q = rng.standard_normal((1, 128, 16))
    k = rng.standard_normal((1, 256, 16))
    qb, kb = oracle.block_means(q), oracle.block_means(k)
    for r in range(2):
        tile = q[0] @ k[0, r * 128:(r + 1) * 128].T
        assert qb[0, 0] @ kb[0, r] == pytest.approx(tile.mean(), abs=1e-12)


# ---------------------------------------------------------------- importance

def test_importance_matches_scipy_softmax_on_explicit_logits():
    rng = np.random.default_rng(5)
    qb = rng.standard_normal((2, 3, 8))
    kb = rng.standard_normal((2, 7, 8))
    scale = 0.37
    p = oracle.importance(qb, kb, scale)
    for h in range(2):
        for i in range(3):
            logits = [scale * sum(qb[h, i, c] * kb[h, r, c] for c in range(8)) for r in range(7)]
            np.testing.assert_allclose(p[h, i], scipy.special.softmax(logits), rtol=1e-13)


def test_importance_invariants():
    rng = np.random.default_rng(6)
    qb = rng.standard_normal((2, 4, 16))
    kb = rng.standard_normal((2, 9, 16))
    p = oracle.importance(qb, kb, 0.25)
    np.testing.assert_allclose(p.sum(-1), 1.0, rtol=1e-14)
    # zero query mean -> uniform
    pu = oracle.importance(np.zeros_like(qb), kb, 0.25)
    np.testing.assert_allclose(pu, 1.0 / 9, rtol=1e-14)
    # a single history block gets all the mass
    assert np.all(oracle.importance(qb, kb[:, :1], 0.25) == 1.0)
    # a common shift u of every key mean adds q̄·u to a whole row: p unchanged
    u = rng.standard_normal(16)
    np.testing.assert_allclose(oracle.importance(qb, kb + u, 0.25), p, rtol=1e-12)
    # empty history
    assert oracle.importance(qb, kb[:, :0], 0.25).shape == (2, 4, 0)


# ---------------------------------------------------------------- fusion

def test_fusion_worked_example():
    gd = _load("fusion_worked.json")
    prm = RouteParams(**gd["params"])
    gh = oracle.ghat(np.array(gd["g"], np.float32), prm.tau, prm.g_ref)
    np.testing.assert_allclose(gh, gd["ghat"], rtol=1e-6)
    w, cov = oracle.fused_weights(np.array(gd["p"], np.float32), np.array(gd["g"], np.float32),
                                  gd["rho_covered"], prm)
    assert cov
    np.testing.assert_allclose(w, gd["w_covered"], rtol=1e-6)
    np.testing.assert_allclose(w / w.astype(np.float64).sum(), gd["p_tilde"], rtol=1e-6)
    np.testing.assert_allclose(w / np.array(gd["p"], np.float32), gd["multiplier"], rtol=1e-6)
    w2, cov2 = oracle.fused_weights(np.array(gd["p"], np.float32), np.array(gd["g"], np.float32),
                                    gd["rho_uncovered"], prm)
    assert not cov2
    assert np.array_equal(w2, np.array(gd["w_uncovered"], np.float32))


def test_ghat_threshold_and_saturation():
    tau, gref = np.float32(0.1), np.float32(0.2)
    g = np.array([0.0, np.float32(0.1), np.nextafter(np.float32(0.1), np.float32(1)),
                  np.float32(0.2), 0.5, 1.0], np.float32)
    gh = oracle.ghat(g, tau, gref)
    assert gh[0] == 0 and gh[1] == 0           # strict: g == tau is not above tau
    assert 0.5 <= gh[2] < 0.5001               # just above tau: ~tau / g_ref
    assert gh[3] == 1 and gh[4] == 1 and gh[5] == 1


def test_multiplier_set_and_max_three():
    """u in {1} ∪ [1 + λτ/g_ref, 1 + λ] = {1} ∪ [2, 3] for the pages' values."""
    rng = np.random.default_rng(7)
    prm = RouteParams()
    g = rng.uniform(0, 1, 20000).astype(np.float32)
    g[:50] = np.nextafter(np.float32(0.1), np.float32(1))
    p = np.ones(20000, np.float32)
    w, cov = oracle.fused_weights(p, g, 0.95, prm)
    assert cov
    u = w / p
    assert u.max() == 3.0
    assert np.all((u == 1.0) | ((u >= 2.0) & (u <= 3.0)))
    assert np.all((u == 1.0) == (g <= np.float32(0.1)))


def test_fusion_lambda_zero_and_low_overlap_is_identity():
    rng = np.random.default_rng(8)
    p = rng.dirichlet(np.ones(30)).astype(np.float32)
    g = rng.uniform(0, 1, 30).astype(np.float32)
    w, _ = oracle.fused_weights(p, g, 0.95, RouteParams(lam=0.0))
    assert np.array_equal(w, p)
    w, _ = oracle.fused_weights(p, g * np.float32(0.1), 0.95, RouteParams())
    assert np.array_equal(w, p)


def test_fixed_mass_is_exact_floor():
    rng = np.random.default_rng(9)
    w = np.concatenate([rng.uniform(0, 3, 1000), [0.0, 3.0, 1e-40, 2.0 ** -60, 2.0 ** -61]]).astype(np.float32)
    W = oracle.fixed_mass(w)
    for x, X in zip(w, W):
        exact = Fraction(float(x)) * 2 ** 60
        assert X == int(exact) and X <= exact < X + 1


# ---------------------------------------------------------------- routes

def _route_case(p, g, rho, prm, M, coords=None, i=0):
    return oracle.route_row(np.asarray(p, np.float32), np.asarray(g, np.float32), rho, prm, M,
                            coords, i)


def test_route_worked_examples():
    gd = _load("route_worked.json")
    for case in gd["cases"]:
        kw = {k: case[k] for k in ("K_cov", "K_unc", "theta_cov", "theta_unc", "n_prev") if k in case}
        prm = RouteParams(**kw)
        got = _route_case(gd["p"], gd["g"], case["rho"], prm, 4)
        assert got == case["expect"], case["why"]


def test_route_mass_threshold_reached_exactly():
    gd = _load("route_threshold_exact.json")
    for case in gd["cases"]:
        kw = {k: case[k] for k in ("K_cov", "K_unc", "theta_cov", "theta_unc", "n_prev") if k in case}
        got = _route_case(gd["p"], gd["g"], case["rho"], RouteParams(**kw), 3)
        assert got == case["expect"], case["why"]


def _rank_key(w, r):
    return (-Fraction(float(w[r])), r)


@pytest.mark.parametrize("seed", range(40))
def test_route_brute_force_tiny(seed):
    """Selected set = the best-ranked candidates, of the minimal count that the
    mass threshold (exact rational arithmetic) or the cap allows; found by
    enumerating every subset of the candidates."""
    rng = np.random.default_rng(100 + seed)
    M = int(rng.integers(1, 9))
    n_prev = int(rng.integers(0, min(M, 3) + 1))
    covered = bool(rng.integers(0, 2))
    theta = float(rng.choice([0.3, 0.5, 0.8, 0.95, 1.0]))
    K = int(rng.integers(1, M + 3))
    prm = RouteParams(K_cov=K, K_unc=K, theta_cov=theta, theta_unc=theta, n_prev=n_prev,
                      lam=float(rng.choice([0.0, 2.0, 5.0])))
    logits = rng.standard_normal(M) * 2
    p = np.exp(logits) / np.exp(logits).sum()
    if seed % 5 == 0:
        p[: M // 2] = p[0]                      # force ties
    p = p.astype(np.float32)
    g = (rng.uniform(0, 1, M) * (rng.uniform(size=M) < 0.6)).astype(np.float32)
    rho = 0.95 if covered else 0.2
    got = _route_case(p, g, rho, prm, M)

    w, _ = oracle.fused_weights(p, g, rho, prm)
    reserved = set(range(M - n_prev, M))
    cand = [r for r in range(M) if r not in reserved]
    Z = sum(Fraction(float(x)) for x in w)
    th = Fraction(float(np.float32(theta)))

    def mass(S):
        return sum(Fraction(float(w[r])) for r in S)

    # The best subset of each size c, by brute force over all subsets: the one
    # subset whose every member outranks every non-member.
    best = {}
    for c in range(len(cand) + 1):
        found = [S for S in combinations(cand, c)
                 if all(_rank_key(w, a) < _rank_key(w, b)
                        for a in S for b in cand if b not in S)]
        assert len(found) == 1
        best[c] = found[0]
    limit = max(0, min(K - n_prev, len(cand)))
    c_star = limit
    if theta < 1.0:
        for c in range(limit + 1):
            if mass(reserved) + mass(best[c]) >= th * Z:
                c_star = c
                break
    expect = sorted(reserved | set(best[c_star]))
    # Fixed-point mass agrees with exact rationals unless a prefix sits within
    # 2^-50 of the threshold; such a seed is skipped.
    near = any(abs(float((mass(reserved) + mass(best[c])) - th * Z)) < 2 ** -50
               for c in range(limit + 1)) if theta < 1.0 else False
    if not near:
        assert got == expect
    # Every selected candidate outranks every unselected one (by exhaustion).
    sel = [r for r in got if r not in reserved]
    uns = [r for r in cand if r not in got]
    for a in sel:
        for b in uns:
            assert _rank_key(w, a) < _rank_key(w, b)
    assert reserved <= set(got)


def test_route_all_when_budget_covers_history():
    rng = np.random.default_rng(11)
    M = 37
    p = rng.dirichlet(np.ones(M)).astype(np.float32)
    g = rng.uniform(0, 1, M).astype(np.float32)
    prm = RouteParams(K_cov=M, K_unc=M + 5, theta_cov=1.0, theta_unc=1.0)
    assert _route_case(p, g, 0.95, prm, M) == list(range(M))
    assert _route_case(p, g, 0.10, prm, M) == list(range(M))


def test_uncovered_route_ignores_geometry():
    rng = np.random.default_rng(12)
    M = 300
    p = rng.dirichlet(np.ones(M)).astype(np.float32)
    prm = RouteParams(n_prev=20)
    base = _route_case(p, np.zeros(M, np.float32), 0.5, prm, M)
    for _ in range(5):
        g = rng.uniform(0, 1, M).astype(np.float32)
        assert _route_case(p, g, 0.5, prm, M) == base


def test_lambda_zero_covered_equals_model_route():
    rng = np.random.default_rng(13)
    M = 200
    p = rng.dirichlet(np.ones(M) * 0.3).astype(np.float32)
    g = rng.uniform(0, 1, M).astype(np.float32)
    prm = RouteParams(lam=0.0, K_cov=60, K_unc=60, theta_cov=0.7, theta_unc=0.7)
    assert _route_case(p, g, 0.95, prm, M) == _route_case(p, g, 0.2, prm, M)


def test_fused_ranking_only_reorders_toward_higher_ghat():
    """If a precedes b in the model ranking but follows it in the fused one,
    then ĝ_b > ĝ_a, or the fused weights tie exactly (broken by id)."""
    rng = np.random.default_rng(14)
    prm = RouteParams()
    for _ in range(20):
        M = 120
        p = rng.dirichlet(np.ones(M)).astype(np.float32)
        g = (rng.uniform(0, 1, M) * (rng.uniform(size=M) < 0.4)).astype(np.float32)
        w, cov = oracle.fused_weights(p, g, 0.99, prm)
        assert cov
        gh = oracle.ghat(g, prm.tau, prm.g_ref)
        model = sorted(range(M), key=lambda r: (-float(p[r]), r))
        fused = sorted(range(M), key=lambda r: (-float(w[r]), r))
        pos = {r: n for n, r in enumerate(fused)}
        for x in range(M):
            for y in range(x + 1, M):
                a, b = model[x], model[y]
                if pos[a] > pos[b]:
                    assert gh[b] > gh[a] or w[a] == w[b]


def test_reservation_always_present_and_route_bounded():
    w = synth.tiny()
    rng = np.random.default_rng(15)
    for _ in range(10):
        p = rng.dirichlet(np.ones(w.M), size=(2, w.N)).astype(np.float32)
        R = oracle.routes(p, w.g, w.rho, w.params, w.M, w.coords)
        for h in range(2):
            for i in range(w.N):
                r = R[h][i]
                assert set(range(w.M - w.params.n_prev, w.M)) <= set(r)
                assert len(r) <= max(w.params.K_cov, w.params.K_unc) + 26
                assert r == sorted(set(r)) and all(0 <= x < w.M for x in r)


def test_random_expectation_50_of_143():
    """I.i.d. importances, no reservation: any fixed block lands in the top-50
    with probability 50/143; a position-biased selection would fail this."""
    gd = _load("random_expectation.json")
    M, K = gd["M"], gd["K"]
    assert round(K / M, 3) == gd["printed"]
    rng = np.random.default_rng(16)
    prm = RouteParams(K_unc=K, theta_unc=1.0)
    counts = np.zeros(M)
    trials = 400
    for _ in range(trials):
        p = rng.dirichlet(np.ones(M)).astype(np.float32)
        for r in _route_case(p, np.zeros(M, np.float32), 0.0, prm, M):
            counts[r] += 1
    rate = counts / trials
    assert abs(rate.mean() - gd["expected_rate"]) < 1e-12     # exactly K per row
    # first, middle and last thirds of the id range are all near 50/143
    for part in np.array_split(rate, 3):
        assert abs(part.mean() - gd["expected_rate"]) < 0.02


# ---------------------------------------------------------------- safeguards

def test_safeguard_neighbours_hand_enumerated():
    # 3x3x3 block grid: the centre cell (1,1,1) is the query block; the 26
    # others are history blocks 0..25 in lexicographic (t,h,w) order.
    cells = [(t, h, w) for t in range(3) for h in range(3) for w in range(3) if (t, h, w) != (1, 1, 1)]
    far = [(5, 0, 0), (1, 1, 3), (3, 1, 1)]          # distance 4, 2, 2: never neighbours
    coords = np.array(cells + far + [(1, 1, 1)], np.int32)
    M = len(cells) + len(far)
    p = np.full(M, 1.0 / M, np.float32)
    prm = RouteParams(K_unc=1, theta_unc=1.0, neigh26=1)
    got = _route_case(p, np.zeros(M, np.float32), 0.0, prm, M, coords, 0)
    # top-1 by (weight, id) is block 0 (all weights equal); plus all 26 neighbours
    assert got == list(range(26))


def test_safeguards_on_tiny_grid_without_reservation():
    w = synth.tiny()
    prm = w.params.replace(n_prev=0, K_cov=1, K_unc=1, theta_unc=1.0)
    p = np.zeros(w.M, np.float32)
    p[0] = 1.0                                         # top-1 is block 0
    # The current chunk sits at t=4 on a 2x2 grid: every t=3 block (ids 12..15)
    # is within Chebyshev distance 1 of every query block; t<=2 blocks are not.
    for i in range(w.N):
        got = _route_case(p, w.g[i], w.rho[i], prm, w.M, w.coords, i)
        assert got == [0, 12, 13, 14, 15]
    assert {int(c[0]) for c in w.coords[12:16]} == {3}
    assert {int(c[0]) for c in w.coords[16:]} == {4}


def test_ref_ids_added_outside_budget():
    M = 10
    p = np.linspace(1, 2, M).astype(np.float32)
    prm = RouteParams(K_unc=2, theta_unc=1.0, ref_ids=(0, 3))
    assert _route_case(p / p.sum(), np.zeros(M, np.float32), 0.0, prm, M) == [0, 3, 8, 9]


def test_empty_history():
    assert _route_case(np.zeros(0), np.zeros(0), 0.95, RouteParams(), 0) == []


# ---------------------------------------------------------------- attention

def _rand_qkv(seed, H=2, N=2, T=6, d=16):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((H, N * 128, d)), rng.standard_normal((H, T * 128, d)),
            rng.standard_normal((H, T * 128, d)))


def test_dense_matches_torch_sdpa_float64():
    q, k, v = _rand_qkv(20)
    scale = 0.25
    M, N = 4, 2
    for h in range(2):
        for i in range(N):
            o, lse = oracle.dense_attention_block(q, k, v, scale, h, i, M, N)
            Q = torch.from_numpy(q[h, i * 128:(i + 1) * 128])[None, None]
            K = torch.from_numpy(k[h, :(M + N) * 128])[None, None]
            V = torch.from_numpy(v[h, :(M + N) * 128])[None, None]
            ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=scale)[0, 0]
            np.testing.assert_allclose(o, ref.numpy(), rtol=1e-10, atol=1e-12)
            lref = torch.logsumexp(scale * (Q[0, 0] @ K[0, 0].T), dim=-1)
            np.testing.assert_allclose(lse, lref.numpy(), rtol=1e-12)


def test_single_tile_is_textbook_attention():
    q, k, v = _rand_qkv(21)
    o, _ = oracle.attention_block(q, k, v, 0.3, 1, 1, [3])
    Q, K, V = q[1, 128:256], k[1, 384:512], v[1, 384:512]
    s = 0.3 * Q @ K.T
    P = np.exp(s) / np.exp(s).sum(1, keepdims=True)
    np.testing.assert_allclose(o, P @ V, rtol=1e-10)


def test_route_all_equals_dense_and_order_free():
    q, k, v = _rand_qkv(22)
    M, N = 4, 2
    o1, l1 = oracle.sparse_attention_block(q, k, v, 0.2, 0, 1, list(range(M)), M, N)
    o2, l2 = oracle.dense_attention_block(q, k, v, 0.2, 0, 1, M, N)
    np.testing.assert_allclose(o1, o2, rtol=1e-13)
    o3, l3 = oracle.attention_block(q, k, v, 0.2, 0, 1, [5, 2, 0, 4])
    o4, l4 = oracle.attention_block(q, k, v, 0.2, 0, 1, [0, 2, 4, 5])
    np.testing.assert_allclose(o3, o4, rtol=1e-12)
    np.testing.assert_allclose(l3, l4, rtol=1e-13)


def test_unit_values_give_unit_output():
    q, k, _ = _rand_qkv(23)
    v = np.ones_like(k)
    o, _ = oracle.sparse_attention_block(q, k, v, 0.5, 1, 0, [1, 3], 4, 2)
    np.testing.assert_allclose(o, 1.0, rtol=1e-14)


def test_sparse_without_current_chunk():
    q, k, v = _rand_qkv(24)
    o, _ = oracle.sparse_attention_block(q, k, v, 0.5, 0, 0, [2], 4, 2, include_current=False)
    o2, _ = oracle.attention_block(q, k, v, 0.5, 0, 0, [2])
    np.testing.assert_array_equal(o, o2)
