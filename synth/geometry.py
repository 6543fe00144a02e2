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
    """Scene boxes (centre [n,3], axes [n,3,3], half-extents [n,3]) of the blocks.

    Per block, token depths ~ lognormal(mu=1.5, sigma=0.5) (or `depths`); the
    box sits on the ray through the block rectangle's centre at the mean depth,
    its axes are the camera axes, its lateral half-extents are the rectangle's
    half-size at the mean depth and its depth half-extent is 1.28 standard
    deviations of the depths (a normal spread's 10-90 half-width). A
    generator's moment recipe; the method's own slabs come from percentile
    intervals and are built by the slab-table kernel.
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
        zm, zs = float(np.mean(depths[b])), float(np.std(depths[b]))
        u0, u1, v0, v1 = rects[bh, bw]
        uc, vc = 0.5 * (u0 + u1), 0.5 * (v0 + v1)
        ray = np.array([(uc - TOKEN_W / 2) / FOCAL, (TOKEN_H / 2 - vc) / FOCAL, 1.0])
        centre[b] = cam + rot @ (zm * ray)
        axes[b] = rot
        half[b] = (zm * (u1 - u0) / (2 * FOCAL), zm * (v1 - v0) / (2 * FOCAL), 1.2816 * zs)
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


# ---------------------------------------------------------------- depth scene
#
# Inputs of the slab-table and multiwarp kernels: depth maps of an analytic
# scene (the inside of a sphere of radius 8 around the origin, which the
# looping camera never leaves) rendered from the trajectory's cameras, and the
# token cells plus depths of history blocks. The rendering is closed-form
# ray-sphere intersection, which is not part of the method.

ROOM_RADIUS = 8.0


def pack_camera(rot: np.ndarray, centre: np.ndarray) -> np.ndarray:
    """float32 [12]: R row-major (columns = camera axes in world), then centre."""
    out = np.zeros(12, np.float32)
    out[0:9] = np.asarray(rot, np.float64).reshape(9)
    out[9:12] = centre
    return out


def sphere_room_depth(rot, centre, width, height, pinhole, rng=None, invalid_fraction=0.0):
    """float32 [height*width] camera-z depth of the room wall through each pixel
    centre (col + 0.5, row + 0.5); a random `invalid_fraction` of pixels is NaN."""
    f, cx, cy = pinhole
    cols, rows = np.meshgrid(np.arange(width) + 0.5, np.arange(height) + 0.5)
    rays = np.stack([(cols - cx) / f, (cy - rows) / f, np.ones_like(cols)], -1).reshape(-1, 3)
    w = rays @ np.asarray(rot, np.float64).T                 # world directions (z-component 1 in camera)
    c = np.asarray(centre, np.float64)
    a = (w * w).sum(1)
    b = 2 * (w @ c)
    cc = c @ c - ROOM_RADIUS ** 2
    t = (-b + np.sqrt(b * b - 4 * a * cc)) / (2 * a)           # the far root: camera is inside
    depth = t.astype(np.float32)
    if rng is not None and invalid_fraction > 0:
        depth[rng.uniform(size=depth.size) < invalid_fraction] = np.nan
    return depth


def slab_inputs(seed: int = 7, n_chunks: int = 6, blocks_per_chunk: int = 36):
    """History blocks of n_chunks chunks: cells [nblk*128][2] int32, depth
    [nblk*128] float32 (10% unreliable), cams [n_chunks][12], cam_of_block."""
    rng = np.random.default_rng(seed)
    pin = (FOCAL, TOKEN_W / 2, TOKEN_H / 2)
    cams = np.stack([pack_camera(*camera_pose(c)) for c in range(n_chunks)])
    nblk = n_chunks * blocks_per_chunk
    cells = np.zeros((nblk * 128, 2), np.int32)
    depth = np.zeros(nblk * 128, np.float32)
    cam_of_block = np.repeat(np.arange(n_chunks), blocks_per_chunk).astype(np.int32)
    for b in range(nblk):
        c0, r0 = rng.integers(0, TOKEN_W - 8), rng.integers(0, TOKEN_H - 6)
        cw, rh = rng.integers(2, 9), rng.integers(2, 7)
        col = rng.integers(c0, c0 + cw, 128)
        row = rng.integers(r0, r0 + rh, 128)
        cells[128 * b:128 * b + 128] = np.stack([col, row], 1)
        rot, ctr = camera_pose(int(cam_of_block[b]))
        full = sphere_room_depth(rot, ctr, TOKEN_W, TOKEN_H, pin)
        z = full[row * TOKEN_W + col] * rng.lognormal(0.0, 0.05, 128).astype(np.float32)
        z[rng.uniform(size=128) < 0.1] = np.nan
        depth[128 * b:128 * b + 128] = z
    if nblk > 3:   # a few degenerate blocks: all unreliable, or barely any depth
        depth[128 * 1:128 * 2] = np.nan
        depth[128 * 2:128 * 3 - 3] = -1.0
    return cells, depth, cams, cam_of_block


def multiwarp_inputs(target_chunk: int = 48, n_cached: int = 30, scale: int = 4, seed: int = 11,
                     holes: bool = True):
    """Cached first/last-frame depth of the n_cached chunks before target_chunk
    at `scale` x the token resolution, their cameras, the target camera, the
    pinholes, and the token cells of the target chunk's 36 blocks. With
    `holes`, the newest chunk's frames lack depth in their left third and the
    one before in its top quarter (unreconstructed regions), so older frames
    must fill in."""
    rng = np.random.default_rng(seed)
    sw, sh = TOKEN_W * scale, TOKEN_H * scale
    src_pin = (FOCAL * scale, sw / 2, sh / 2)
    tgt_pin = (FOCAL, TOKEN_W / 2, TOKEN_H / 2)
    frames, cams = [], []
    for c in range(target_chunk - n_cached, target_chunk):
        for frac in (0.0, 0.9):            # first and last frame of the chunk
            rot, ctr = camera_pose(c + frac)
            frames.append(sphere_room_depth(rot, ctr, sw, sh, src_pin, rng, invalid_fraction=0.05))
            cams.append(pack_camera(rot, ctr))
    if holes and len(frames) >= 4:
        for k in (-1, -2):
            frames[k].reshape(sh, sw)[:, : sw // 3] = np.nan
        for k in (-3, -4):
            frames[k].reshape(sh, sw)[: sh // 4] = np.nan
    tgt = pack_camera(*camera_pose(target_chunk))
    # tokens of the 36 blocks on the 4 x 9 block grid: a block covers its
    # rectangle of cells (3 frames), padded to 128 by repeating its cells
    rects = block_rectangles(4, 9)
    cells = np.zeros((36 * 128, 2), np.int32)
    for b in range(36):
        u0, u1, v0, v1 = rects[b // 9, b % 9]
        cc = [(c, r) for r in range(int(np.floor(v0)), int(np.ceil(v1))) for c in range(int(np.floor(u0)),
                                                                                     int(np.ceil(u1)))]
        tok = (cc * ((128 // len(cc)) + 1))[:128]
        cells[128 * b:128 * b + 128] = tok
    return (np.stack(frames), np.stack(cams), (sw, sh), src_pin, tgt, (TOKEN_W, TOKEN_H), tgt_pin, cells)
