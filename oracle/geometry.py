"""CPU oracle for the geometry scorer: slab overlaps g and coverage rho.

TEST INFRASTRUCTURE ONLY (imported by the tests, the smoke check and the
benchmark's CPU-baseline leg; the library never calls it and shares no code
with it).

What the pages fix:
- [digest] Prerequisites, "frustum slab and OBB overlap": a block is a token
  rectangle plus a percentile depth interval, approximated by a camera-facing
  oriented box; two blocks correspond by the ratio of intersection volume.
- [digest] Method steps, step 3, and [onedev] "How it works": the overlap
  g_{i,r} is an IoU of world-space OBBs whose intersection is approximated on a
  grid (eq. 7); coverage rho_i is the fraction of query-block tokens whose
  warped depth lands inside a valid history slab, and a block trusts geometry
  when rho_i >= eta_cov = 0.9 (eq. 8).
- [project] 02 · Method, "What the router sees": g is the overlap (IoU)
  between the query block's slab and a history block's slab, in world space.

Readings where the pages are silent (listed in the design notes):
- the grid is the n^3 lattice of cell centres of the query box A:
  local offsets e_j * ((2 k_j + 1) / n - 1), k_j = 0 .. n-1; the intersection
  volume is vol(A) * (lattice points inside B) / n^3 and the IoU is
  I / (vol(A) + vol(B) - I);
- a slab is valid iff its three half-extents are > 0; an invalid history slab
  overlaps nothing and covers nothing, an invalid query slab gives a zero row;
- "inside a slab" for a token is the point-in-OBB test of its world point (the
  slab's OBB approximation, the same primitive as the overlap); a token without
  depth (NaN point) is never covered.

Precision: every decision (point inside or not) and every output is computed
in IEEE float32, one rounding per operation, in the order written below, so
that a GPU implementation taking the same decisions matches exactly.
Operation order:
  world point   p_x = c_x + ((R00 u0 + R01 u1) + R02 u2)   (same for y, z)
  local coord   l_j = (R0j d0 + R1j d1) + R2j d2,  d = p - c_B
  inside        |l_j| <= e_j for j = 0, 1, 2
  volume        ((8 e0) e1) e2
  IoU           f = count / n^3;  I = vol_A f;  U = (vol_A + vol_B) - I;  g = I / U
                (g = 0 when count = 0)
OBB record layout (float32 [16]): centre (3), half-extents (3), axes R
row-major (9: axis j is column j), unused (1).
"""

from __future__ import annotations

import numpy as np

f32 = np.float32


def obb_fields(rec):
    """(centre [3], half-extents [3], R [3][3]) of one float32 record."""
    rec = np.asarray(rec, dtype=f32)
    return rec[0:3], rec[3:6], rec[6:15].reshape(3, 3)


def obb_valid(rec) -> bool:
    _, e, _ = obb_fields(rec)
    return bool(e[0] > 0 and e[1] > 0 and e[2] > 0)


def obb_volume(rec) -> np.float32:
    _, e, _ = obb_fields(rec)
    return f32(f32(f32(f32(8.0) * e[0]) * e[1]) * e[2])


def lattice_points(rec, n: int) -> np.ndarray:
    """World positions [n^3, 3] (float32) of box A's cell-centre lattice.

    Index order: k0 (along axis 0) slowest, then k1, then k2.
    """
    c, e, R = obb_fields(rec)
    t = np.array([f32(f32(2 * k + 1) / f32(n)) - f32(1.0) for k in range(n)], dtype=f32)
    k0, k1, k2 = np.meshgrid(np.arange(n), np.arange(n), np.arange(n), indexing="ij")
    u0 = (e[0] * t[k0.ravel()]).astype(f32)
    u1 = (e[1] * t[k1.ravel()]).astype(f32)
    u2 = (e[2] * t[k2.ravel()]).astype(f32)
    pts = np.empty((u0.size, 3), dtype=f32)
    for r in range(3):
        acc = (R[r, 0] * u0).astype(f32)
        acc = (acc + (R[r, 1] * u1).astype(f32)).astype(f32)
        acc = (acc + (R[r, 2] * u2).astype(f32)).astype(f32)
        pts[:, r] = (c[r] + acc).astype(f32)
    return pts


def inside_obb(pts, rec) -> np.ndarray:
    """Boolean mask: which float32 points [P, 3] lie inside box B (closed)."""
    c, e, R = obb_fields(rec)
    pts = np.asarray(pts, dtype=f32).reshape(-1, 3)
    d = (pts - c).astype(f32)
    ok = np.ones(pts.shape[0], dtype=bool)
    for j in range(3):
        l = (R[0, j] * d[:, 0]).astype(f32)
        l = (l + (R[1, j] * d[:, 1]).astype(f32)).astype(f32)
        l = (l + (R[2, j] * d[:, 2]).astype(f32)).astype(f32)
        ok &= np.abs(l) <= e[j]
    return ok


def overlap_pair(a, b, n: int = 8) -> np.float32:
    """g for one query box a and one history box b (eq. 7 reading above)."""
    if not (obb_valid(a) and obb_valid(b)):
        return f32(0.0)
    count = int(inside_obb(lattice_points(a, n), b).sum())
    if count == 0:
        return f32(0.0)
    va, vb = obb_volume(a), obb_volume(b)
    frac = f32(f32(count) / f32(n * n * n))
    inter = f32(va * frac)
    union = f32(f32(va + vb) - inter)
    return f32(inter / union)


def slab_overlap(q_obb, h_obb, n: int = 8) -> np.ndarray:
    """g [N][M] float32 for query boxes [N,16] against history boxes [M,16].

    Element for element the arithmetic of overlap_pair; the inside test runs
    for all history boxes of a row at once (numpy broadcasting).
    """
    q_obb = np.asarray(q_obb, dtype=f32)
    h_obb = np.asarray(h_obb, dtype=f32)
    N, M = q_obb.shape[0], h_obb.shape[0]
    g = np.zeros((N, M), dtype=f32)
    if M == 0:
        return g
    hc, he, hR = h_obb[:, 0:3], h_obb[:, 3:6], h_obb[:, 6:15].reshape(M, 3, 3)
    hvalid = (he > 0).all(axis=1)
    hvol = np.array([obb_volume(rec) for rec in h_obb], dtype=f32)
    for i in range(N):
        if not obb_valid(q_obb[i]):
            continue
        pts = lattice_points(q_obb[i], n)                               # [P,3]
        d = (pts[None, :, :] - hc[:, None, :]).astype(f32)              # [M,P,3]
        ok = np.ones(d.shape[:2], dtype=bool)
        for j in range(3):
            l = (hR[:, 0, j, None] * d[:, :, 0]).astype(f32)
            l = (l + (hR[:, 1, j, None] * d[:, :, 1]).astype(f32)).astype(f32)
            l = (l + (hR[:, 2, j, None] * d[:, :, 2]).astype(f32)).astype(f32)
            ok &= np.abs(l) <= he[:, j, None]
        count = ok.sum(axis=1)
        va = obb_volume(q_obb[i])
        for r in range(M):
            if not hvalid[r] or count[r] == 0:
                continue
            frac = f32(f32(int(count[r])) / f32(n * n * n))
            inter = f32(va * frac)
            g[i, r] = f32(inter / f32(f32(va + hvol[r]) - inter))
    return g


def token_covered(q_pts, h_obb) -> np.ndarray:
    """[N][T] booleans: token point inside at least one valid history box (eq. 8)."""
    q_pts = np.asarray(q_pts, dtype=f32)
    N, T = q_pts.shape[0], q_pts.shape[1]
    flat = q_pts.reshape(-1, 3)
    cov = np.zeros(flat.shape[0], dtype=bool)
    for rec in np.asarray(h_obb, dtype=f32):
        if obb_valid(rec):
            cov |= inside_obb(flat, rec)
    return cov.reshape(N, T)


def slab_coverage(q_pts, h_obb) -> np.ndarray:
    """rho [N] float32: covered tokens / tokens per block (exact in float32)."""
    cov = token_covered(q_pts, h_obb)
    return (cov.sum(axis=1).astype(np.float64) / cov.shape[1]).astype(f32)
