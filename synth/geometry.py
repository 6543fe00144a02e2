"""Synthetic frustum slabs and their world-space OBB overlaps.

Produces the routing inputs g[i][r] (overlap of current query block i with
history block r, in [0, 1]) and the coverage rho[i]. These are *inputs* of the
routed-attention path; upstream they come from streaming reconstruction, which
is not part of this library. Nothing here is routing or attention arithmetic.

What the pages fix, and what this generator takes from them:
- Paper digest ("Velox: Spatial Memory Makes World Models Efficient"),
  Prerequisites, "frustum slab and OBB overlap": a historical KV block is
  summarised by its token rectangle and a percentile depth interval, approximated
  by a camera-facing OBB; two blocks correspond by intersection-volume ratio.
- Same digest, Method steps, step 1 and 3: the depth interval is the 10/90
  percentile of the block's depths; the overlap uses a grid approximation of
  the intersection.
- Velox project page, 02 · Method, "What the router sees": top overlaps of a
  query block with its best history blocks are around 0.4-0.7 (a magnitude
  check for this generator, not a value it must reproduce).
Coverage rho_i (fraction of a query block's tokens whose warped depth falls in
a valid history slab) needs the multiwarp depth stage, which is out of scope;
rho is therefore assigned directly to reach a target covered fraction.
"""

from __future__ import annotations

import numpy as np

TOKEN_H, TOKEN_W = 29, 52      # latent token grid of an 832 x 464 clip
FOCAL = 26.0                   # tokens; about 90 degrees of horizontal FOV
LATTICE = 8                    # points per OBB axis for the intersection estimate


def camera_pose(chunk: int, period: float = 24.0, radius: float = 3.0):
    """World-from-camera rotation (columns right, up, forward) and centre.

    A smooth loop: the camera circles the origin every `period` chunks, looking
    mostly inward, so late chunks revisit places seen by early ones.
    """
    ang = 2.0 * np.pi * chunk / period
    centre = np.array([radius * np.cos(ang), 0.0, radius * np.sin(ang)])
    inward = -centre / np.linalg.norm(centre)
    tangent = np.array([-np.sin(ang), 0.0, np.cos(ang)])
    fwd = inward + 0.6 * tangent
    fwd /= np.linalg.norm(fwd)
    up0 = np.array([0.0, 1.0, 0.0])
    right = np.cross(up0, fwd)
    right /= np.linalg.norm(right)
    up = np.cross(fwd, right)
    return np.stack([right, up, fwd], axis=1), centre


def block_rectangles(blocks_h: int, blocks_w: int):
    """Token rectangles (u0, u1, v0, v1) of a blocks_h x blocks_w cell grid."""
    ue = np.linspace(0.0, TOKEN_W, blocks_w + 1)
    ve = np.linspace(0.0, TOKEN_H, blocks_h + 1)
    rects = np.zeros((blocks_h, blocks_w, 4))
    for bh in range(blocks_h):
        for bw in range(blocks_w):
            rects[bh, bw] = (ue[bw], ue[bw + 1], ve[bh], ve[bh + 1])
    return rects


def slab_obbs(coords: np.ndarray, chunk_of_block: np.ndarray, blocks_h: int,
              blocks_w: int, rng: np.random.Generator):
    """Camera-facing OBBs (centre [n,3], axes [n,3,3], half-extents [n,3]).

    Per block: depth samples ~ lognormal(mu=1.5, sigma=0.5), interval
    [Q10, Q90]; the box sits on the ray through the rectangle centre at the
    interval's mid-depth, its axes are the camera axes, its lateral extents are
    the rectangle's extents at mid-depth and its depth extent the interval.
    """
    rects = block_rectangles(blocks_h, blocks_w)
    n = coords.shape[0]
    centre = np.zeros((n, 3))
    axes = np.zeros((n, 3, 3))
    half = np.zeros((n, 3))
    for b in range(n):
        _, bh, bw = coords[b]
        rot, cam = camera_pose(int(chunk_of_block[b]))
        depths = rng.lognormal(mean=1.5, sigma=0.5, size=128)
        zlo, zhi = np.quantile(depths, [0.10, 0.90])
        zmid = 0.5 * (zlo + zhi)
        u0, u1, v0, v1 = rects[bh, bw]
        uc, vc = 0.5 * (u0 + u1), 0.5 * (v0 + v1)
        ray = np.array([(uc - TOKEN_W / 2) / FOCAL, (TOKEN_H / 2 - vc) / FOCAL, 1.0])
        centre[b] = cam + rot @ (zmid * ray)
        axes[b] = rot
        half[b] = (zmid * (u1 - u0) / (2 * FOCAL), zmid * (v1 - v0) / (2 * FOCAL),
                   0.5 * (zhi - zlo))
    return centre, axes, half


def obb_iou(ca, ra, ea, cb, rb, eb) -> np.ndarray:
    """IoU of every box A (rows) with every box B (columns) on a point lattice.

    The intersection volume is vol(A) times the fraction of an 8^3 cell-centre
    lattice of A that lies inside B.
    """
    t = (np.arange(LATTICE) + 0.5) / LATTICE * 2.0 - 1.0
    lat = np.stack(np.meshgrid(t, t, t, indexing="ij"), -1).reshape(-1, 3)  # [P,3]
    vol_a = 8.0 * np.prod(ea, axis=1)
    vol_b = 8.0 * np.prod(eb, axis=1)
    out = np.zeros((ca.shape[0], cb.shape[0]))
    for i in range(ca.shape[0]):
        pts = ca[i] + (lat * ea[i]) @ ra[i].T                          # [P,3] world
        rel = pts[None, :, :] - cb[:, None, :]                          # [M,P,3]
        local = np.einsum("mpk,mkj->mpj", rel, rb)                      # B frame
        inside = np.all(np.abs(local) <= eb[:, None, :], axis=2)        # [M,P]
        inter = inside.mean(axis=1) * vol_a[i]
        out[i] = inter / (vol_a[i] + vol_b - inter)
    return out


def assign_coverage(n_query: int, covered_fraction: float,
                    rng: np.random.Generator) -> np.ndarray:
    """rho in [0.9, 1) for round(fraction * N) random query blocks, else [0, 0.85).

    The uncovered range stops short of 0.9 so that rounding to fp32 can never
    carry an uncovered value onto the coverage threshold.
    """
    n_cov = int(round(covered_fraction * n_query))
    perm = rng.permutation(n_query)
    rho = rng.uniform(0.0, 0.85, size=n_query)
    rho[perm[:n_cov]] = rng.uniform(0.9, 1.0, size=n_cov)
    return rho.astype(np.float32)
