"""Synthetic frustum slabs and their world-space OBB overlaps.

Produces a synthetic scene: camera-facing OBBs of every block's frustum slab,
world points of the current chunk's tokens, and from them the routing inputs
g[i][r] (overlap of current query block i with history block r, in [0, 1]) and
the coverage rho[i]. Upstream these come from streaming reconstruction, which
is not part of this library. The overlaps here are a seeded Monte Carlo
estimate (random points), not the method's fixed-lattice estimator, so this
module shares no arithmetic with the geometry scorer or the router.

What the pages fix, and what this generator takes from them:
- Paper digest ("Velox: Spatial Memory Makes World Models Efficient"),
  Prerequisites, "frustum slab and OBB overlap": a historical KV block is
  summarised by its token rectangle and a percentile depth interval, approximated
  by a camera-facing OBB; two blocks correspond by intersection-volume ratio.
- Same digest, Method steps, step 1: the depth interval is the 10/90
  percentile of the block's depths.
- Velox project page, 02 · Method, "What the router sees": top overlaps of a
  query block with its best history blocks are around 0.4-0.7 (a magnitude
  check for this generator, not a value it must reproduce).
For the routing workloads rho is assigned directly to reach a target covered
fraction; the token points exist for the coverage kernel's own tests.
"""

from __future__ import annotations

import numpy as np

TOKEN_H, TOKEN_W = 29, 52      # latent token grid of an 832 x 464 clip
FOCAL = 26.0                   # tokens; about 90 degrees of horizontal FOV
MC_SAMPLES = 512               # random points per box for the overlap estimate


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


def _token_depths(rng: np.random.Generator, n: int) -> np.ndarray:
    return rng.lognormal(mean=1.5, sigma=0.5, size=(n, 128))


def slab_obbs(coords: np.ndarray, chunk_of_block: np.ndarray, blocks_h: int,
              blocks_w: int, rng: np.random.Generator, depths: np.ndarray | None = None):
    """Camera-facing OBBs (centre [n,3], axes [n,3,3], half-extents [n,3]).

    Per block: depth samples ~ lognormal(mu=1.5, sigma=0.5) (or `depths`),
    interval [Q10, Q90]; the box sits on the ray through the rectangle centre at
    the interval's mid-depth, its axes are the camera axes, its lateral extents
    are the rectangle's extents at mid-depth and its depth extent the interval.
    """
    rects = block_rectangles(blocks_h, blocks_w)
    n = coords.shape[0]
    if depths is None:
        depths = _token_depths(rng, n)
    centre = np.zeros((n, 3))
    axes = np.zeros((n, 3, 3))
    half = np.zeros((n, 3))
    for b in range(n):
        _, bh, bw = coords[b]
        rot, cam = camera_pose(int(chunk_of_block[b]))
        zlo, zhi = np.quantile(depths[b], [0.10, 0.90])
        zmid = 0.5 * (zlo + zhi)
        u0, u1, v0, v1 = rects[bh, bw]
        uc, vc = 0.5 * (u0 + u1), 0.5 * (v0 + v1)
        ray = np.array([(uc - TOKEN_W / 2) / FOCAL, (TOKEN_H / 2 - vc) / FOCAL, 1.0])
        centre[b] = cam + rot @ (zmid * ray)
        axes[b] = rot
        half[b] = (zmid * (u1 - u0) / (2 * FOCAL), zmid * (v1 - v0) / (2 * FOCAL),
                   0.5 * (zhi - zlo))
    return centre, axes, half


def token_points(coords: np.ndarray, chunk_of_block: np.ndarray, blocks_h: int, blocks_w: int,
                 depths: np.ndarray, rng: np.random.Generator, sky_fraction: float = 0.25):
    """World points [n,128,3] (float32) of each block's 128 tokens.

    Token positions are uniform in the block's rectangle; token a sits at depth
    depths[b][a] along its ray. In blocks of the top row a `sky_fraction` of
    the tokens has no depth (NaN point), like sky without reconstruction.
    """
    rects = block_rectangles(blocks_h, blocks_w)
    n = coords.shape[0]
    pts = np.zeros((n, 128, 3))
    for b in range(n):
        _, bh, bw = coords[b]
        rot, cam = camera_pose(int(chunk_of_block[b]))
        u0, u1, v0, v1 = rects[bh, bw]
        u = rng.uniform(u0, u1, size=128)
        v = rng.uniform(v0, v1, size=128)
        rays = np.stack([(u - TOKEN_W / 2) / FOCAL, (TOKEN_H / 2 - v) / FOCAL, np.ones(128)], 1)
        pts[b] = cam + (depths[b][:, None] * rays) @ rot.T
        if bh == 0:
            pts[b, rng.uniform(size=128) < sky_fraction] = np.nan
    return pts.astype(np.float32)


def pack_obbs(centre: np.ndarray, axes: np.ndarray, half: np.ndarray) -> np.ndarray:
    """float32 [n,16] records: centre (3), half-extents (3), axes row-major (9), 0.

    Axis j of box b (a unit vector in world space) is column j of axes[b], i.e.
    record entries 6 + 3 * row + j for row = 0, 1, 2.
    """
    n = centre.shape[0]
    out = np.zeros((n, 16), np.float32)
    out[:, 0:3] = centre
    out[:, 3:6] = half
    out[:, 6:15] = axes.reshape(n, 9)
    return out


def mc_overlap(ca, ra, ea, cb, rb, eb, rng: np.random.Generator,
               samples: int = MC_SAMPLES) -> np.ndarray:
    """Seeded Monte Carlo IoU of every box A (rows) with every box B (columns).

    The intersection volume is vol(A) times the fraction of `samples` uniform
    random points of A that lie inside B (float64 throughout).
    """
    vol_a = 8.0 * np.prod(ea, axis=1)
    vol_b = 8.0 * np.prod(eb, axis=1)
    out = np.zeros((ca.shape[0], cb.shape[0]))
    for i in range(ca.shape[0]):
        loc = rng.uniform(-1.0, 1.0, size=(samples, 3)) * ea[i]
        pts = ca[i] + loc @ ra[i].T                                    # [P,3] world
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
