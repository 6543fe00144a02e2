"""Pins of the geometry oracle (slab overlaps g, coverage rho) against closed
forms, exact lattice counts, an independent float64 Monte Carlo estimate and
hand-built cases. CPU only."""

import numpy as np
import pytest

from oracle import geometry as geo

f32 = np.float32


def box(c=(0, 0, 0), e=(1, 1, 1), R=np.eye(3)):
    rec = np.zeros(16, f32)
    rec[0:3] = c
    rec[3:6] = e
    rec[6:15] = np.asarray(R, np.float64).reshape(9)
    return rec


def rot(axis, ang):
    a = np.asarray(axis, float) / np.linalg.norm(axis)
    K = np.array([[0, -a[2], a[1]], [a[2], 0, -a[0]], [-a[1], a[0], 0]])
    return np.eye(3) + np.sin(ang) * K + (1 - np.cos(ang)) * K @ K


def aabb_iou(c1, e1, c2, e2):
    lo = np.maximum(np.subtract(c1, e1), np.subtract(c2, e2))
    hi = np.minimum(np.add(c1, e1), np.add(c2, e2))
    inter = np.prod(np.clip(hi - lo, 0, None))
    v1, v2 = 8 * np.prod(e1), 8 * np.prod(e2)
    return inter / (v1 + v2 - inter)


def mc_iou(a, b, n=400_000, seed=0):
    """Independent float64 Monte Carlo IoU (random points of a, tested in b)."""
    rng = np.random.default_rng(seed)
    ca, ea, Ra = a[0:3].astype(float), a[3:6].astype(float), a[6:15].astype(float).reshape(3, 3)
    cb, eb, Rb = b[0:3].astype(float), b[3:6].astype(float), b[6:15].astype(float).reshape(3, 3)
    loc = rng.uniform(-1, 1, size=(n, 3)) * ea
    pts = ca + loc @ Ra.T
    inside = np.all(np.abs((pts - cb) @ Rb) <= eb, axis=1)
    va, vb = 8 * np.prod(ea), 8 * np.prod(eb)
    inter = inside.mean() * va
    return inter / (va + vb - inter)


def test_identical_boxes_give_exactly_one():
    for R in (np.eye(3), rot([1, 2, 3], 0.7)):
        a = box((1.5, -2, 3), (0.3, 0.7, 1.9), R)
        assert geo.overlap_pair(a, a) == f32(1.0)


def test_disjoint_boxes_give_zero():
    assert geo.overlap_pair(box(), box((5, 0, 0))) == 0.0
    assert geo.overlap_pair(box(), box((0, 2.01, 0))) == 0.0


def test_half_shift_gives_one_third_exactly():
    # shifting B by one half-extent along an axis puts exactly half of A's
    # lattice (the positive-coordinate columns) inside B: I = V/2, U = 3V/2
    for axis in range(3):
        c = [0.0, 0.0, 0.0]
        c[axis] = 1.0
        g = geo.overlap_pair(box(e=(1, 1, 1)), box(c=c, e=(1, 1, 1)), n=8)
        assert g == f32(f32(4.0) / f32(12.0))


def test_nested_box_gives_volume_ratio():
    a = box((0.1, 0.2, -0.1), (0.5, 0.4, 0.3))
    b = box((0, 0, 0), (2, 3, 4))
    va, vb = geo.obb_volume(a), geo.obb_volume(b)
    assert geo.overlap_pair(a, b) == f32(va / f32(f32(va + vb) - va))


def test_lattice_count_matches_hand_count():
    # B spans x in [0.6, 2.4] and all of A in y, z: it holds the lattice
    # columns at x = 0.625 and 0.875, 2 of 8 -> 128 of 512 points; narrowed
    # to [0.7, 2.3] it holds one column -> 64
    a = box(e=(1, 1, 1))
    pts = geo.lattice_points(a, 8)
    assert geo.inside_obb(pts, box(c=(1.5, 0, 0), e=(0.9, 5, 5))).sum() == 128
    assert geo.inside_obb(pts, box(c=(1.5, 0, 0), e=(0.8, 5, 5))).sum() == 64
    assert pts.shape == (512, 3)
    assert np.allclose(np.unique(pts[:, 0]), (np.arange(8) + 0.5) / 4 - 1)


@pytest.mark.parametrize("seed", range(6))
def test_axis_aligned_lattice_converges_to_closed_form(seed):
    rng = np.random.default_rng(seed)
    e1, e2 = rng.uniform(0.3, 2, 3), rng.uniform(0.3, 2, 3)
    c1, c2 = rng.uniform(-1, 1, 3), rng.uniform(-1, 1, 3)
    exact = aabb_iou(c1, e1, c2, e2)
    a, b = box(c1, e1), box(c2, e2)
    # per-axis covered fraction of the lattice differs from the true one by at
    # most 1/n, so the intersection fraction differs by at most 3/n
    for n in (8, 16, 32):
        g = float(geo.overlap_pair(a, b, n=n))
        va, vb = 8 * np.prod(e1), 8 * np.prod(e2)
        inter_est = g * (va + vb) / (1 + g)
        inter_true = exact * (va + vb) / (1 + exact)
        assert abs(inter_est - inter_true) <= 3.0 / n * va + 1e-5


@pytest.mark.parametrize("seed", range(4))
def test_rotated_pair_matches_independent_monte_carlo(seed):
    rng = np.random.default_rng(100 + seed)
    Ra, Rb = rot(rng.normal(size=3), rng.uniform(0, np.pi)), rot(rng.normal(size=3), rng.uniform(0, np.pi))
    a = box(rng.uniform(-0.3, 0.3, 3), rng.uniform(0.5, 1.5, 3), Ra)
    b = box(rng.uniform(-0.3, 0.3, 3), rng.uniform(0.5, 1.5, 3), Rb)
    ref = mc_iou(a, b)
    g = float(geo.overlap_pair(a, b, n=32))
    assert ref > 0.05
    assert abs(g - ref) < 0.03


def test_common_rotation_leaves_overlap_unchanged():
    # rotating both boxes (and their centres) by the same rotation: the lattice
    # rotates with A, so only float rounding at lattice points on B's faces
    # could change a count; these boxes keep every lattice point off B's faces
    e1, e2 = (1.0, 0.6, 0.8), (0.7, 1.1, 0.5)
    c1, c2 = np.array([0.0, 0.0, 0.0]), np.array([0.37, -0.21, 0.13])
    g0 = geo.overlap_pair(box(c1, e1), box(c2, e2))
    R = rot([0.3, -1.0, 0.5], 1.1)
    g1 = geo.overlap_pair(box(R @ c1, e1, R), box(R @ c2, e2, R))
    assert g0 == g1
    assert abs(float(g0) - aabb_iou(c1, e1, c2, e2)) < 0.1


def test_transposed_axes_would_be_caught():
    # B is A's extents turned 30 degrees about z, A sits off B's centre in x and
    # y: the overlap with B and with B turned the other way differ by 2x, so a
    # local transform that used R in place of its transpose would fail here
    R = rot([0, 0, 1], np.pi / 6)
    a = box(c=(1.0, 0.5, 0), e=(1.5, 0.3, 1))
    b = box(e=(1.5, 0.3, 1), R=R)
    b_mirror = box(e=(1.5, 0.3, 1), R=R.T)
    ref, ref_mirror = mc_iou(a, b), mc_iou(a, b_mirror)
    assert ref > 3 * ref_mirror
    assert abs(float(geo.overlap_pair(a, b, n=32)) - ref) < 0.01
    assert abs(float(geo.overlap_pair(a, b_mirror, n=32)) - ref_mirror) < 0.01
    # a 90-degree turn swaps the extents: the same solid as an axis-aligned box
    same = box(e=(0.3, 1.5, 1), R=rot([0, 0, 1], np.pi / 2))
    assert geo.overlap_pair(box(e=(1.5, 0.3, 1)), same) == f32(1.0)


def test_invalid_slabs():
    bad = box(e=(1, 0, 1))
    assert not geo.obb_valid(bad)
    assert geo.overlap_pair(box(), bad) == 0.0
    assert geo.overlap_pair(bad, box()) == 0.0
    g = geo.slab_overlap(np.stack([bad, box()]), np.stack([box(), bad]))
    assert g.tolist() == [[0.0, 0.0], [1.0, 0.0]]


def test_slab_overlap_matrix_equals_pairwise():
    rng = np.random.default_rng(7)
    qs = np.stack([box(rng.uniform(-1, 1, 3), rng.uniform(0.3, 1, 3), rot(rng.normal(size=3), 0.5))
                   for _ in range(3)])
    hs = np.stack([box(rng.uniform(-1, 1, 3), rng.uniform(0.3, 1, 3), rot(rng.normal(size=3), 1.0))
                   for _ in range(5)])
    g = geo.slab_overlap(qs, hs, n=4)
    for i in range(3):
        for r in range(5):
            assert g[i, r] == geo.overlap_pair(qs[i], hs[r], n=4)
    assert g.dtype == np.float32 and (g >= 0).all() and (g <= 1).all()


def test_coverage_counts_tokens():
    hs = np.stack([box((0, 0, 0), (1, 1, 1)), box((10, 0, 0), (1, 1, 1)), box((20, 0, 0), (1, 0, 1))])
    pts = np.zeros((2, 128, 3), f32)
    pts[0, :64] = (0.5, 0.5, 0.5)       # inside box 0
    pts[0, 64:96] = (10, 0.9, -0.9)     # inside box 1
    pts[0, 96:] = (5, 0, 0)             # between boxes
    pts[1, :] = (20, 0, 0)              # only inside the invalid box 2
    pts[1, :10] = np.nan                # no depth
    pts[1, 10:20] = (1.0, 1.0, 1.0)     # on the closed boundary of box 0
    rho = geo.slab_coverage(pts, hs)
    assert rho.tolist() == [96 / 128, 10 / 128]
    cov = geo.token_covered(pts, hs)
    assert cov[0, :96].all() and not cov[0, 96:].any()


def test_coverage_against_float64_brute_force():
    rng = np.random.default_rng(3)
    hs = np.stack([box(rng.uniform(-2, 2, 3), rng.uniform(0.2, 1, 3), rot(rng.normal(size=3), rng.uniform(0, 3)))
                   for _ in range(20)])
    pts = rng.uniform(-2.5, 2.5, size=(4, 128, 3)).astype(f32)
    cov = geo.token_covered(pts, hs)
    ref = np.zeros_like(cov)
    margin = np.full(cov.shape, np.inf)
    for rec in hs:
        c, e, R = rec[0:3].astype(float), rec[3:6].astype(float), rec[6:15].astype(float).reshape(3, 3)
        loc = (pts.astype(float) - c) @ R
        slack = np.max(np.abs(loc) - e, axis=-1)
        ref |= slack <= 0
        margin = np.minimum(margin, np.abs(slack))
    decided = margin > 1e-5
    assert (cov[decided] == ref[decided]).all()
    assert 0.05 < cov.mean() < 0.95
