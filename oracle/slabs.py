"""CPU oracle for the slab table and the recency-priority multiwarp.

TEST INFRASTRUCTURE ONLY (imported by the tests, the smoke check and the
benchmark's CPU-baseline leg; the library never calls it and shares no code
with it).

What the pages fix:
- [digest] Method steps, step 1 (eq. 4-5): after a chunk is decoded, reliable
  depth is back-projected, bucketed by global (Gilbert) block, and each history
  block gets a slab: its token rectangle in the chunk's latent camera and the
  10/90 percentile interval of its depths, with validity statistics.
- [digest] Prerequisites "recency-priority multiwarp" and Method steps, step 2
  (eq. 6): the first and last frame depths of the last K = 30 reconstructed
  chunks are cached and forward-warped into the target camera; per token the
  depth is the median of the newest frame that supplies at least k_warp = 2
  samples.
- [digest] Prerequisites, "frustum slab and OBB overlap": a slab is
  approximated by a camera-facing oriented box.
- [onedev] "How it works": percentile depth interval per block fragment,
  warped first/last-frame depths, newest frame whose sample count clears the
  lower bound, its median.

Readings where the pages are silent (listed in the design notes):
- camera model: pinhole in token units, focal f, principal point (cx, cy); a
  token cell (col, row) has centre (col + 0.5, row + 0.5) and ray
  ((u - cx) / f, (cy - v) / f, 1) in camera axes (x right, y up, z forward);
  a pose is (R, c): world = c + R * camera;
- a sample is reliable iff its depth is finite and > 0; a block's slab is valid
  iff it has at least n_min reliable samples (invalid slabs get zero extents);
- the token rectangle spans the cells of the block's reliable tokens:
  [min col, max col + 1] x [min row, max row + 1];
- percentiles interpolate linearly between order statistics (q at rank
  (n - 1) * p); the median of an even count is the mean of the two middle
  values;
- the camera-facing box of a slab: centre on the ray through the rectangle
  centre at the interval's mid-depth, axes = the camera axes, lateral
  half-extents = the rectangle's half-size at mid-depth, depth half-extent =
  half the interval;
- multiwarp: the cached frames are depth maps at their own (pixel) resolution
  and pinhole; a source pixel lands in target token cell (floor(u'), floor(v'))
  when its point is in front of the target camera and inside the grid; frames
  are ranked by their index (higher = newer).

Precision: every decision (reliable or not, which cell a warped point lands in)
and every output is computed in IEEE float32, one rounding per operation, in the
order written below, so a GPU implementation matches exactly:
  ray        rx = (u - cx) / f,  ry = (cy - v) / f
  point      X_r = c_r + ((R_r0 (z rx) + R_r1 (z ry)) + R_r2 z)
  projection d = X - c_t;  p_j = (R_0j d0 + R_1j d1) + R_2j d2;
             u' = (f p0) / p2 + cx,  v' = cy - (f p1) / p2
  percentile h = (n - 1) * p;  i = floor(h);  q = x_i + (h - i) (x_{i+1} - x_i)
  box        uc = (u0 + u1) * 0.5, vc = (v0 + v1) * 0.5, zm = (zlo + zhi) * 0.5;
             centre = point of (uc, vc) at depth zm;
             e0 = (zm (u1 - u0)) / (2 f),  e1 = (zm (v1 - v0)) / (2 f),
             e2 = (zhi - zlo) * 0.5
"""

from __future__ import annotations

import math

import numpy as np

f32 = np.float32


def _pose(cam):
    cam = np.asarray(cam, dtype=f32)
    return cam[0:9].reshape(3, 3), cam[9:12]


def ray(u, v, f, cx, cy):
    return f32(f32(f32(u) - f32(cx)) / f32(f)), f32(f32(f32(cy) - f32(v)) / f32(f))


def world_point(cam, u, v, z, f, cx, cy):
    """float32 [3]: the point at depth z on the ray through (u, v)."""
    R, c = _pose(cam)
    rx, ry = ray(u, v, f, cx, cy)
    z = f32(z)
    a, b = f32(z * rx), f32(z * ry)
    out = np.empty(3, f32)
    for r in range(3):
        s = f32(f32(f32(R[r, 0] * a) + f32(R[r, 1] * b)) + f32(R[r, 2] * z))
        out[r] = f32(c[r] + s)
    return out


def project(cam, X, f, cx, cy):
    """(u', v', depth) of world point X in camera cam (float32)."""
    R, c = _pose(cam)
    d = [f32(f32(X[j]) - c[j]) for j in range(3)]
    p = [f32(f32(f32(R[0, j] * d[0]) + f32(R[1, j] * d[1])) + f32(R[2, j] * d[2])) for j in range(3)]
    f = f32(f)
    u = f32(f32(f32(f * p[0]) / p[2]) + f32(cx))
    v = f32(f32(cy) - f32(f32(f * p[1]) / p[2]))
    return u, v, p[2]


def reliable(z) -> bool:
    z = f32(z)
    return bool(np.isfinite(z) and z > 0)


def percentile(sorted_vals, p):
    """Linear-interpolation percentile of ascending float32 values (float32)."""
    n = len(sorted_vals)
    h = f32(f32(n - 1) * f32(p))
    i = int(math.floor(float(h)))
    fr = f32(h - f32(i))
    xi = f32(sorted_vals[i])
    if i + 1 >= n:
        return xi
    return f32(xi + f32(fr * f32(f32(sorted_vals[i + 1]) - xi)))


def slab_of_block(cols, rows, depths, n_min):
    """(u0, u1, v0, v1, zlo, zhi, count, valid) of one block's samples (float32)."""
    keep = [k for k in range(len(depths)) if reliable(depths[k])]
    n = len(keep)
    if n < n_min or n == 0:
        return np.array([0, 0, 0, 0, 0, 0, n, 0], dtype=f32)
    z = sorted(f32(depths[k]) for k in keep)
    u0 = min(int(cols[k]) for k in keep)
    u1 = max(int(cols[k]) for k in keep) + 1
    v0 = min(int(rows[k]) for k in keep)
    v1 = max(int(rows[k]) for k in keep) + 1
    return np.array([u0, u1, v0, v1, percentile(z, 0.1), percentile(z, 0.9), n, 1], dtype=f32)


def slab_box(slab, cam, f, cx, cy):
    """float32 [16] OBB record of a slab (zeros when the slab is invalid)."""
    rec = np.zeros(16, f32)
    if slab[7] == 0:
        return rec
    u0, u1, v0, v1, zlo, zhi = (f32(x) for x in slab[:6])
    half = f32(0.5)
    uc, vc, zm = f32(f32(u0 + u1) * half), f32(f32(v0 + v1) * half), f32(f32(zlo + zhi) * half)
    rec[0:3] = world_point(cam, uc, vc, zm, f, cx, cy)
    two_f = f32(f32(2.0) * f32(f))
    rec[3] = f32(f32(zm * f32(u1 - u0)) / two_f)
    rec[4] = f32(f32(zm * f32(v1 - v0)) / two_f)
    rec[5] = f32(f32(zhi - zlo) * half)
    R, _ = _pose(cam)
    rec[6:15] = R.reshape(9)
    return rec


def slab_table(cells, depth, cams, cam_of_block, f, cx, cy, n_min):
    """Slabs [nblk][8] and boxes [nblk][16] of blocks of 128 samples each.

    cells [nblk*128][2] int (col, row), depth [nblk*128] float32, cams [ncam][12]
    float32 (R row-major, centre), cam_of_block [nblk] int.
    """
    cells = np.asarray(cells)
    depth = np.asarray(depth, dtype=f32)
    nblk = depth.size // 128
    slabs = np.zeros((nblk, 8), f32)
    boxes = np.zeros((nblk, 16), f32)
    for b in range(nblk):
        sl = slice(128 * b, 128 * b + 128)
        slabs[b] = slab_of_block(cells[sl, 0], cells[sl, 1], depth[sl], n_min)
        boxes[b] = slab_box(slabs[b], cams[int(cam_of_block[b])], f, cx, cy)
    return slabs, boxes


def multiwarp(src_depth, src_cams, src_w, src_h, src_pin, tgt_cam, width, height, tgt_pin,
              k_warp=2):
    """(zq [height*width] float32, NaN = none; chosen frame [height*width] int, -1 = none).

    src_depth [K][src_h*src_w] float32 depth maps (row-major pixels) of frames
    with cameras src_cams [K][12] and pinhole src_pin = (f, cx, cy); frame k is
    newer than frame k-1. The target is a width x height token grid seen by
    tgt_cam with pinhole tgt_pin.
    """
    K = len(src_depth)
    C = width * height
    fs, cxs, cys = src_pin
    ft, cxt, cyt = tgt_pin
    samples = [[[] for _ in range(K)] for _ in range(C)]
    for k in range(K):
        for pix in range(src_w * src_h):
            z = src_depth[k][pix]
            if not reliable(z):
                continue
            col, row = pix % src_w, pix // src_w
            X = world_point(src_cams[k], f32(col) + f32(0.5), f32(row) + f32(0.5), z, fs, cxs, cys)
            u, v, dz = project(tgt_cam, X, ft, cxt, cyt)
            if not (dz > 0) or not (np.isfinite(u) and np.isfinite(v)):
                continue
            fu, fv = math.floor(float(u)), math.floor(float(v))
            if 0 <= fu < width and 0 <= fv < height:
                samples[fv * width + fu][k].append(f32(dz))
    zq = np.full(C, np.nan, f32)
    chosen = np.full(C, -1, np.int64)
    for c in range(C):
        for k in range(K - 1, -1, -1):
            if len(samples[c][k]) >= k_warp:
                s = sorted(samples[c][k])
                n = len(s)
                zq[c] = s[n // 2] if n % 2 == 1 else f32(f32(s[n // 2 - 1] + s[n // 2]) * f32(0.5))
                chosen[c] = k
                break
    return zq, chosen


def token_points(cells, zq, width, height, cam, f, cx, cy):
    """(depth [n] float32, points [n][3] float32) of tokens at cells [n][2]:
    the warped depth of the token's cell and its world point (NaN without
    depth)."""
    cells = np.asarray(cells)
    n = cells.shape[0]
    depth = np.empty(n, f32)
    pts = np.full((n, 3), np.nan, f32)
    for s_ in range(n):
        col = min(max(int(cells[s_, 0]), 0), width - 1)
        row = min(max(int(cells[s_, 1]), 0), height - 1)
        z = f32(zq[row * width + col])
        depth[s_] = z
        if reliable(z):
            pts[s_] = world_point(cam, f32(col) + f32(0.5), f32(row) + f32(0.5), z, f, cx, cy)
    return depth, pts
