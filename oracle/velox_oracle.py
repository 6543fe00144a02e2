"""CPU oracle for routed block-sparse history attention (Velox).

TEST INFRASTRUCTURE ONLY. This module is the plain, slow, obviously-correct
statement of what the routed-attention path computes. Only the test suite, the
smoke check and the benchmark's CPU-baseline leg may import it; the library
never calls it and shares no code with it.

Pages cited (all describe "Velox: Spatial Memory Makes World Models Efficient"):
- [digest]   paper digest on paper.rainbus.top (Chinese): sections Prerequisites,
             Motivation, Core method, Method steps.
- [project]  project page "Velox: Spatial Memory Makes Long-context World Models
             Efficient" (velox-world.com/velox): 02 · Method (fusion formula and
             its legend, "Covered and uncovered blocks", "Why the route is a
             block"), 03 · Results (Figure 3 caption).
- [onedev]   Korean summary on onedev.kr: "How it works", "What differs",
             "How to use".

Precision: importance and attention in float64 on inputs widened exactly from
their stored type. The route is decided in IEEE float32 (round to nearest, no
fused multiply-add, no denormal flush) plus exact integer mass accounting,
because a route is a discrete decision that both sides must take from the same
float32 importances.

Readings where the pages are silent (each is listed, with its reason, in the
design notes of the repository):
- importance logit scale is 1/sqrt(d) (the mean query-key inner product of a
  tile, scaled as attention scales it);
- covered rows take the fused top-K_cov with no mass cut unless theta_cov < 1;
  uncovered rows take the minimal mass prefix reaching theta_unc, capped at K_unc;
- the reserved previous-chunk blocks count toward both the cap and the mass;
- ties in weight go to the smaller block id;
- cumulative mass is counted in fixed point: floor(w * 2^60) per block, with the
  cut test  m * 2^24 >= floor(theta * 2^24) * Z  taken in exact integers;
- safeguard neighbours are history blocks at Chebyshev distance exactly 1 from
  the query block in the caller's (t, h, w) block grid; the current chunk always
  attends to itself, densely, after its routed history tiles.
Parity for every function here is pinned by tests against closed forms,
library routines, hand-worked values or brute force.
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np

BLOCK = 128                 # b_tok: tokens per block = attention tile
MASS_BITS = 60              # fixed-point scale of per-block mass
THETA_BITS = 24             # fixed-point scale of the mass threshold


# --------------------------------------------------------------------------
# Block means and block importance  ([digest] Method steps, step 4, eq. 9;
# [onedev] "What differs": importance = softmax of the mean query . mean key)
# --------------------------------------------------------------------------

def block_means(x: np.ndarray, block: int = BLOCK) -> np.ndarray:
    """Mean over each block of `block` consecutive tokens.

    x: [H][T][d] (any float dtype, T a multiple of `block`) -> float64 [H][T/block][d].
    """
    H, T, d = x.shape
    assert T % block == 0
    return x.astype(np.float64).reshape(H, T // block, block, d).mean(axis=2)


def importance(qbar: np.ndarray, kbar: np.ndarray, scale: float) -> np.ndarray:
    """p[h][i][r] = softmax over history r of scale * (qbar[h][i] . kbar[h][r]).

    qbar [H][N][d], kbar [H][M][d] (float64) -> p [H][N][M] float64.
    """
    logits = scale * np.einsum("hnd,hmd->hnm", qbar, kbar)
    if logits.shape[-1] == 0:
        return logits
    logits = logits - logits.max(axis=-1, keepdims=True)
    e = np.exp(logits)
    return e / e.sum(axis=-1, keepdims=True)


# --------------------------------------------------------------------------
# Soft geometric fusion  ([project] 02 · Method, fusion formula:
#   p~ proportional to p * (1 + lambda * ghat),  ghat = 1[g > tau] * min(g / g_ref, 1);
#   coverage gate rho_i >= eta_cov: [digest] Core method, [onedev] "What differs")
# --------------------------------------------------------------------------

def ghat(g: np.ndarray, tau, g_ref) -> np.ndarray:
    """Normalised overlap in float32: 0 unless g > tau, else min(g / g_ref, 1)."""
    g = np.asarray(g, dtype=np.float32)
    tau = np.float32(tau)
    g_ref = np.float32(g_ref)
    ratio = np.minimum(g / g_ref, np.float32(1.0))          # correctly rounded fp32 divide
    return np.where(g > tau, ratio, np.float32(0.0)).astype(np.float32)


def importance_shared(qbar_heads, kbar_heads, scale: float) -> np.ndarray:
    """Head-shared importance [N][M]: softmax over r of the mean over heads of
    scale * qbar_h . kbar_h (float64). The pages index p by layer only ([digest]
    Method steps, step 4); this is its reading for a multi-head layer."""
    qb = np.asarray(qbar_heads, dtype=np.float64)
    kb = np.asarray(kbar_heads, dtype=np.float64)
    logits = scale * np.einsum("hnd,hmd->nm", qb, kb) / qb.shape[0]
    logits -= logits.max(axis=1, keepdims=True)
    e = np.exp(logits)
    return e / e.sum(axis=1, keepdims=True)


MODE_FUSED, MODE_MODEL_ONLY, MODE_GEOMETRY_ONLY = 0, 1, 2


def fused_weights(p_row: np.ndarray, g_row: np.ndarray, rho_i, prm):
    """Unnormalised route weights w of one query block, in float32.

    Covered row (rho_i >= eta_cov): w = p * (1 + lambda * ghat), each product and
    sum rounded to float32. Uncovered row: w = p (the model's own distribution,
    untouched by geometry). Returns (w, covered).
    Comparison routers ([project] 03 · Results: a matched model-only
    block-sparse route; [digest] Prerequisites: soft fusion against hard
    geometric top-K): mode 1 keeps w = p on covered rows too (same budgets),
    mode 2 ranks covered rows by the overlap itself, w = g.
    Normalising w by its sum does not change the ranking, and the mass cut works
    on ratios, so the division of the formula is never materialised.
    """
    p_row = np.asarray(p_row, dtype=np.float32)
    covered = bool(np.float32(rho_i) >= np.float32(prm.eta_cov))
    if not covered:
        return p_row.copy(), False
    mode = int(getattr(prm, "mode", 0))
    if mode == MODE_MODEL_ONLY:
        return p_row.copy(), True
    if mode == MODE_GEOMETRY_ONLY:
        return np.asarray(g_row, dtype=np.float32).copy(), True
    gh = ghat(g_row, prm.tau, prm.g_ref)
    u = np.float32(1.0) + np.float32(prm.lam) * gh            # two float32 roundings
    return (p_row * u).astype(np.float32), True


def fixed_mass(w: np.ndarray) -> list[int]:
    """floor(w * 2^60) for each float32 weight, as exact Python integers."""
    return [int(Fraction(float(x)) * (1 << MASS_BITS)) for x in np.asarray(w, np.float32)]


# --------------------------------------------------------------------------
# Route materialisation  ([digest] Core method and Method steps, step 4;
# [project] 02 · Method, "Covered and uncovered blocks"; [onedev] "What differs":
# previous chunk reserved inside the budget, neighbours and reference blocks
# added outside it as deterministic safeguards)
# --------------------------------------------------------------------------

def route_row(p_row, g_row, rho_i, prm, M: int, coords=None, query_block: int = 0):
    """Ascending history block ids routed to one query block (one head).

    p_row: float32 [M] importances; g_row: float32 [M] overlaps; rho_i: coverage.
    coords: int [(M+N), 3] block-grid coordinates, needed when prm.neigh26.
    """
    if M == 0:
        return []
    w, covered = fused_weights(p_row, g_row, rho_i, prm)
    W = fixed_mass(w)
    Z = sum(W)
    n_prev = min(int(prm.n_prev), M)
    reserved = list(range(M - n_prev, M))
    route = list(reserved)
    mass = sum(W[r] for r in reserved)
    K = int(prm.K_cov if covered else prm.K_unc)
    theta = np.float32(prm.theta_cov if covered else prm.theta_unc)
    cut = bool(theta < np.float32(1.0))
    if covered and int(getattr(prm, "mode", 0)) == MODE_GEOMETRY_ONLY:
        cut = False            # overlaps are not a distribution: plain top-K_cov
    theta_q = int(Fraction(float(theta)) * (1 << THETA_BITS)) if cut else 0
    reserved_set = set(reserved)
    # Rank the other blocks by weight, heaviest first; equal weights by id.
    candidates = sorted((r for r in range(M) if r not in reserved_set),
                        key=lambda r: (-float(w[r]), r))
    for r in candidates:
        if len(route) >= K:
            break
        if cut and mass * (1 << THETA_BITS) >= theta_q * Z:
            break
        route.append(r)
        mass += W[r]
    chosen = set(route)
    if prm.neigh26:
        qt, qh, qw = (int(c) for c in coords[M + query_block])
        for r in range(M):
            t, h, ww = (int(c) for c in coords[r])
            if max(abs(t - qt), abs(h - qh), abs(ww - qw)) == 1:
                chosen.add(r)
    for r in prm.ref_ids:
        if 0 <= int(r) < M:
            chosen.add(int(r))
    return sorted(chosen)


def routes(p, g, rho, prm, M: int, coords=None):
    """Routes for every (head, query block): list over h of list over i."""
    H, N = p.shape[0], p.shape[1]
    return [[route_row(p[h, i], g[i], rho[i], prm, M, coords, i) for i in range(N)]
            for h in range(H)]


# --------------------------------------------------------------------------
# Attention over a set of tiles  ([digest] Core method, eq. 15: indexed
# block-sparse attention computes only the selected tiles; Prerequisites:
# dense FlashAttention visits all N x M_c tile pairs)
# --------------------------------------------------------------------------

def attention_block(q, k, v, scale: float, h: int, i: int, tiles, block: int = BLOCK):
    """Softmax attention of query block i of head h over the listed key tiles.

    q [H][N*block][d], k and v [H][T][d] (float arrays, widened to float64).
    Returns (o [block][d] float64, lse [block] float64, natural log).
    """
    tiles = list(tiles)
    Q = np.asarray(q[h, i * block:(i + 1) * block], dtype=np.float64)
    idx = np.concatenate([np.arange(t * block, (t + 1) * block) for t in tiles])
    K = np.asarray(k[h, idx], dtype=np.float64)
    V = np.asarray(v[h, idx], dtype=np.float64)
    s = scale * (Q @ K.T)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    o = (e @ V) / l
    return o, (m + np.log(l))[:, 0]


def sparse_attention_block(q, k, v, scale, h, i, route, M: int, N: int,
                           include_current: bool = True):
    """Routed history tiles, then (if include_current) the current chunk's tiles."""
    tiles = list(route) + (list(range(M, M + N)) if include_current else [])
    return attention_block(q, k, v, scale, h, i, tiles)


def dense_attention_block(q, k, v, scale, h, i, M: int, N: int):
    """All history tiles and all current-chunk tiles."""
    return attention_block(q, k, v, scale, h, i, range(M + N))
