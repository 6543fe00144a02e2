"""Pins of the slab-table and multiwarp oracle: numpy percentiles, hand-built
blocks, closed-form boxes of a known camera, projection round trips and
analytic planes seen from moved cameras. CPU only."""

import numpy as np
import pytest

from oracle import slabs

f32 = np.float32
F, CX, CY = 26.0, 26.0, 14.5          # token-unit pinhole of a 52 x 29 grid


def cam(R=np.eye(3), c=(0, 0, 0)):
    out = np.zeros(12, f32)
    out[0:9] = np.asarray(R, float).reshape(9)
    out[9:12] = c
    return out


def rot(axis, ang):
    a = np.asarray(axis, float) / np.linalg.norm(axis)
    K = np.array([[0, -a[2], a[1]], [a[2], 0, -a[0]], [-a[1], a[0], 0]])
    return np.eye(3) + np.sin(ang) * K + (1 - np.cos(ang)) * K @ K


@pytest.mark.parametrize("n", [1, 2, 3, 10, 57, 128])
def test_percentile_matches_numpy(n):
    rng = np.random.default_rng(n)
    x = np.sort(rng.lognormal(1.5, 0.5, n).astype(f32))
    for p in (0.1, 0.5, 0.9):
        ref = np.percentile(x.astype(np.float64), 100 * p)
        assert abs(float(slabs.percentile(list(x), p)) - ref) <= 2e-6 * ref


def test_slab_of_block_rectangle_interval_and_validity():
    cols = np.array([3, 4, 5, 3, 9, 7] + [4] * 122)
    rows = np.array([1, 1, 2, 3, 0, 2] + [2] * 122)
    z = np.full(128, np.nan, f32)
    z[:4] = [1.0, 2.0, 3.0, 4.0]
    z[4] = 0.0          # unreliable: the column 9 / row 0 cell must not count
    z[5] = -1.0         # unreliable
    s = slabs.slab_of_block(cols, rows, z, n_min=4)
    assert s.tolist()[:4] == [3, 6, 1, 4]
    # float32 interpolation: within one float32 rounding of numpy's float64 value
    assert abs(s[4] - 1.3) < 2e-6 * 1.3 and abs(s[5] - 3.7) < 2e-6 * 3.7
    assert s[6] == 4 and s[7] == 1
    assert slabs.slab_of_block(cols, rows, z, n_min=5)[7] == 0


def test_box_of_a_centred_slab_at_identity_camera():
    # a rectangle centred on the principal point, interval [2, 6]: the box sits
    # on the optical axis at depth 4 with half-extents 4 w / (2 f), 4 h / (2 f), 2
    slab = np.array([CX - 5, CX + 5, CY - 3, CY + 3, 2.0, 6.0, 100, 1], f32)
    rec = slabs.slab_box(slab, cam(), F, CX, CY)
    assert np.allclose(rec[0:3], [0, 0, 4], atol=1e-6)
    assert np.allclose(rec[3:6], [4 * 10 / (2 * F), 4 * 6 / (2 * F), 2], rtol=1e-6)
    assert (rec[6:15] == np.eye(3).reshape(9)).all()
    assert (slabs.slab_box(np.zeros(8, f32), cam(), F, CX, CY) == 0).all()


def test_box_face_corners_project_onto_the_rectangle():
    R = rot([0.2, 1.0, -0.3], 0.8)
    c = cam(R, (1.0, -2.0, 0.5))
    slab = np.array([10, 17, 4, 9, 3.0, 5.0, 50, 1], f32)
    rec = slabs.slab_box(slab, c, F, CX, CY)
    centre, e, Rb = rec[0:3].astype(float), rec[3:6].astype(float), rec[6:15].astype(float).reshape(3, 3)
    for sx, sy, u, v in ((-1, 1, 10, 4), (1, 1, 17, 4), (-1, -1, 10, 9), (1, -1, 17, 9)):
        corner = centre + Rb @ np.array([sx * e[0], sy * e[1], 0.0])
        pu, pv, pz = slabs.project(c, corner.astype(f32), F, CX, CY)
        assert abs(pu - u) < 1e-4 and abs(pv - v) < 1e-4 and abs(pz - 4.0) < 1e-5


def test_projection_round_trip():
    rng = np.random.default_rng(1)
    for _ in range(20):
        c = cam(rot(rng.normal(size=3), rng.uniform(0, 3)), rng.normal(size=3))
        u, v, z = rng.uniform(0, 52), rng.uniform(0, 29), rng.uniform(0.5, 20)
        X = slabs.world_point(c, u, v, z, F, CX, CY)
        pu, pv, pz = slabs.project(c, X, F, CX, CY)
        assert abs(pu - u) < 1e-3 and abs(pv - v) < 1e-3 and abs(pz - z) < 1e-4 * z


def _plane_depth(cam_rec, W, H, depth_along_axis):
    """Depth map of a fronto-parallel plane (all pixels at the same depth)."""
    return np.full(W * H, depth_along_axis, f32)


def test_identity_warp_returns_the_depth_map():
    W, H = 13, 7
    rng = np.random.default_rng(2)
    D = rng.uniform(1, 9, W * H).astype(f32)
    D[5] = np.nan
    c = cam(rot([1, 1, 0], 0.4), (0.3, 0.1, -2))
    pin = (F / 4, W / 2, H / 2)
    zq, chosen = slabs.multiwarp([D], [c], W, H, pin, c, W, H, pin, k_warp=1)
    ok = ~np.isnan(D)
    assert np.allclose(zq[ok], D[ok], rtol=1e-5) and np.isnan(zq[5])
    assert (chosen[ok] == 0).all() and chosen[5] == -1


def test_newest_frame_with_enough_samples_wins():
    # the target camera sits 2 units behind the source cameras (same axes), so
    # several source pixels land in each target cell. Frame 0 sees a plane at
    # depth 3, frame 1 (newer) one at depth 5 but only in the left half.
    W, H, f = 16, 10, 8.0
    src = cam(np.eye(3), (0, 0, 0))
    tgt = cam(np.eye(3), (0, 0, -2.0))
    D0 = _plane_depth(src, W, H, 3.0)
    D1 = _plane_depth(src, W, H, 5.0)
    D1.reshape(H, W)[:, W // 2:] = np.nan
    pin = (f, W / 2, H / 2)
    zq, chosen = slabs.multiwarp([D0, D1], [src, src], W, H, pin, tgt, W, H, pin, k_warp=2)
    zq, chosen = zq.reshape(H, W), chosen.reshape(H, W)
    assert (chosen == 1).sum() > 0 and (chosen == 0).sum() > 0
    assert np.allclose(zq[chosen == 1], 7.0, rtol=1e-5)     # 5 + 2 behind
    assert np.allclose(zq[chosen == 0], 5.0, rtol=1e-5)     # 3 + 2 behind
    # k_warp = 1 would take frame 1 wherever it lands at all
    _, ch1 = slabs.multiwarp([D0, D1], [src, src], W, H, pin, tgt, W, H, pin, k_warp=1)
    assert (ch1.reshape(H, W) == 1).sum() >= (chosen == 1).sum()


def test_median_of_a_slanted_plane_matches_brute_force():
    # a slanted plane seen by a source camera, warped into a rotated, shifted
    # target: each cell's value is the median of the float64 re-projection of
    # the newest frame's pixels that land in it
    W, H, f = 12, 9, 7.0
    src = cam(np.eye(3), (0, 0, 0))
    tgt = cam(rot([0, 1, 0], 0.15), (0.4, 0.1, -1.5))
    cols, rows = np.meshgrid(np.arange(W), np.arange(H))
    D = (4.0 + 0.15 * cols + 0.1 * rows).astype(f32).ravel()
    pin = (f, W / 2, H / 2)
    zq, chosen = slabs.multiwarp([D], [src], W, H, pin, tgt, W, H, pin, k_warp=2)
    R = tgt[0:9].astype(float).reshape(3, 3)
    t = tgt[9:12].astype(float)
    lists = {}
    for pix in range(W * H):
        u, v = pix % W + 0.5, pix // W + 0.5
        X = D[pix] * np.array([(u - W / 2) / f, (H / 2 - v) / f, 1.0])
        p = R.T @ (X - t)
        cu, cv = np.floor(f * p[0] / p[2] + W / 2), np.floor(H / 2 - f * p[1] / p[2])
        if p[2] > 0 and 0 <= cu < W and 0 <= cv < H:
            lists.setdefault(int(cv * W + cu), []).append(p[2])
    checked = 0
    for cidx, vals in lists.items():
        if len(vals) >= 2 and chosen[cidx] == 0:
            assert abs(zq[cidx] - np.median(vals)) < 1e-4
            checked += 1
    assert checked > 10


def test_higher_resolution_source_fills_every_cell():
    # a source frame at 4x the token resolution, seen from the same camera:
    # every target cell receives 16 samples of the same plane depth
    W, H, f = 10, 6, 5.0
    c = cam(rot([0, 0, 1], 0.3), (0.1, 0.2, 0.3))
    D = np.full(4 * W * 4 * H, 6.0, f32)
    zq, chosen = slabs.multiwarp([D], [c], 4 * W, 4 * H, (4 * f, 2 * W, 2 * H), c, W, H, (f, W / 2, H / 2),
                                 k_warp=16)
    assert (chosen == 0).all() and np.allclose(zq, 6.0, rtol=1e-5)
    zq2, chosen2 = slabs.multiwarp([D], [c], 4 * W, 4 * H, (4 * f, 2 * W, 2 * H), c, W, H, (f, W / 2, H / 2),
                                   k_warp=17)
    assert (chosen2 == -1).all() and np.isnan(zq2).all()


def test_token_points_closed_form_on_a_fronto_parallel_plane():
    # Camera at c = (1, 2, 3) looking down +z (R = I), pinhole f = 2,
    # (cx, cy) = (2, 1.5) on a 4 x 3 token grid; every cell at depth 4. A token
    # in cell (col, row) is lifted through the cell centre (col + 1/2, row + 1/2):
    #   X = 1 + 4 (col + 1/2 - 2) / 2,  Y = 2 + 4 (1.5 - row - 1/2) / 2,  Z = 3 + 4,
    # all exact in float32. Cells outside the grid take the nearest edge cell;
    # a cell without depth (NaN) or with depth <= 0 gives a NaN point.
    W, H, f, cx, cy = 4, 3, 2.0, 2.0, 1.5
    zq = np.full(W * H, 4.0, f32)
    zq[1 * W + 2] = np.nan        # cell (col 2, row 1)
    zq[2 * W + 3] = 0.0           # cell (col 3, row 2): unreliable
    cells = np.array([[0, 0], [3, 0], [1, 2], [2, 1], [3, 2], [-5, 1], [9, 7]], np.int32)
    depth, pts = slabs.token_points(cells, zq, W, H, cam(np.eye(3), (1.0, 2.0, 3.0)), f, cx, cy)

    def expect(col, row):
        return [1 + 4 * (col + 0.5 - cx) / f, 2 + 4 * (cy - row - 0.5) / f, 7.0]
    assert pts[0].tolist() == expect(0, 0) == [-2.0, 4.0, 7.0]
    assert pts[1].tolist() == expect(3, 0)
    assert pts[2].tolist() == expect(1, 2)
    assert np.isnan(pts[3]).all() and np.isnan(depth[3])
    assert np.isnan(pts[4]).all() and depth[4] == 0.0
    assert pts[5].tolist() == expect(0, 1) and depth[5] == 4.0     # clamped to column 0
    assert np.isnan(pts[6]).all()                                   # clamped onto (3, 2): depth 0


def test_slab_table_uses_each_blocks_own_camera():
    # [onedev] "How it works" / [digest] Method steps, step 1: a block's slab is
    # its token rectangle in the latent camera of the chunk it came from. Two
    # blocks with the same samples but different cameras: each box centre must
    # project back onto its rectangle centre at mid-depth in its own camera,
    # and not in the other block's camera.
    cams = np.stack([cam(rot([0.0, 1.0, 0.2], 0.4), (0.5, 0.0, -1.0)),
                     cam(rot([1.0, 0.3, 0.0], -0.6), (-2.0, 1.0, 0.5))])
    rng = np.random.default_rng(3)
    cols = rng.integers(10, 20, 128)
    rows = rng.integers(5, 12, 128)
    z = rng.uniform(2.0, 6.0, 128).astype(f32)
    cells = np.concatenate([np.stack([cols, rows], 1)] * 2)
    depth = np.concatenate([z, z])
    sl, boxes = slabs.slab_table(cells, depth, cams, np.array([0, 1]), F, CX, CY, 8)
    assert (sl[0] == sl[1]).all()
    for b, other in ((0, 1), (1, 0)):
        u0, u1, v0, v1, zlo, zhi = (float(x) for x in sl[b][:6])
        uc, vc, zm = (u0 + u1) / 2, (v0 + v1) / 2, (zlo + zhi) / 2
        pu, pv, pz = slabs.project(cams[b], boxes[b][0:3], F, CX, CY)
        assert abs(pu - uc) < 1e-4 and abs(pv - vc) < 1e-4 and abs(pz - zm) < 1e-5
        qu, qv, _ = slabs.project(cams[other], boxes[b][0:3], F, CX, CY)
        assert abs(qu - uc) + abs(qv - vc) > 1.0
