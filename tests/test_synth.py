"""Synthetic-input generators: Gilbert rank map properties, chunk seams,
coverage assignment and overlap ranges. CPU only."""

import numpy as np
import pytest

import synth
from synth.geometry import assign_coverage, mc_overlap
from synth.blockgrid import chunk_block_coords, serpentine_cells


@pytest.mark.parametrize("w,h", [(9, 4), (2, 2), (1, 6), (8, 1), (5, 3)])
def test_serpentine_is_a_bijection_with_neighbour_steps(w, h):
    cells = serpentine_cells(w, h)
    assert len(cells) == w * h and len(set(cells)) == w * h
    steps = [abs(a[0] - b[0]) + abs(a[1] - b[1]) for a, b in zip(cells, cells[1:])]
    assert all(s == 1 for s in steps)


def test_chunk_seams_stay_adjacent():
    co = chunk_block_coords(6, 4, 9)
    assert co.shape == (6 * 36, 3)
    for c in range(5):
        last, first = co[c * 36 + 35], co[(c + 1) * 36]
        assert first[0] == last[0] + 1 and first[1] == last[1] and first[2] == last[2]
    # each chunk is a permutation of the 4x9 grid at its own t
    for c in range(6):
        cells = {(int(h), int(w)) for _, h, w in co[c * 36:(c + 1) * 36]}
        assert cells == {(h, w) for h in range(4) for w in range(9)}


def test_coverage_assignment():
    rng = np.random.default_rng(0)
    rho = assign_coverage(36, 0.6, rng)
    assert rho.dtype == np.float32
    assert int((rho >= np.float32(0.9)).sum()) == 22
    assert rho.min() >= 0 and rho.max() < 1


def test_mc_overlap_identical_and_disjoint_boxes():
    c = np.zeros((1, 3))
    r = np.eye(3)[None]
    e = np.ones((1, 3))
    rng = np.random.default_rng(0)
    assert mc_overlap(c, r, e, c, r, e, rng)[0, 0] == pytest.approx(1.0)
    assert mc_overlap(c, r, e, c + 10, r, e, rng)[0, 0] == 0.0
    half = mc_overlap(c, r, e, c + np.array([[1.0, 0, 0]]), r, e, rng, samples=20000)[0, 0]
    assert half == pytest.approx(1 / 3, abs=0.02)    # overlap 1/2 of each: IoU 1/3


def test_scene_records_and_points():
    w = synth.wan13()
    sc = w.scene
    assert sc["obb_hist"].shape == (143, 16) and sc["obb_query"].shape == (36, 16)
    assert sc["query_pts"].shape == (36, 128, 3) and sc["query_pts"].dtype == np.float32
    assert (sc["obb_hist"][:, 3:6] > 0).all()
    R = sc["obb_hist"][:, 6:15].reshape(-1, 3, 3).astype(float)
    assert np.allclose(R @ R.transpose(0, 2, 1), np.eye(3), atol=1e-5)
    # query token points lie on their own block's slab depth range
    c, e, Rq = sc["obb_query"][:, 0:3], sc["obb_query"][:, 3:6], sc["obb_query"][:, 6:15].reshape(-1, 3, 3)
    loc = np.einsum("npk,nkj->npj", sc["query_pts"].astype(float) - c[:, None], Rq)
    ok = ~np.isnan(loc).any(-1)
    frac = (np.abs(loc[..., 2]) <= e[:, None, 2] + 1e-4)[ok].mean()
    assert 0.7 < frac < 0.9                        # the 10/90 interval holds ~80%


def test_workload_shapes_and_overlap_range():
    w = synth.chunk48()
    assert (w.H, w.d, w.N, w.M) == (40, 128, 36, 1692)
    assert w.g.shape == (36, 1692) and w.coords.shape == (1728, 3)
    assert 0.0 <= w.g.min() and w.g.max() <= 1.0
    top = np.sort(w.g, axis=1)[:, -1]
    assert 0.2 < np.median(top) < 0.9
    assert w.route_cap == 176
    t = synth.tiny()
    assert t.coords.shape == (20, 3) and (t.g == 0).mean() > 0.5


def test_make_qkv_is_seeded_and_offset():
    w = synth.tiny()
    q1, k1, v1 = synth.make_qkv(w)
    q2, k2, v2 = synth.make_qkv(w)
    assert (q1 == q2).all() and (k1 == k2).all() and (v1 == v2).all()
    assert q1.shape == (2, 512, 64) and k1.shape == (2, 20 * 128, 64)
    w2 = synth.wan13()
    w2.H = 2
    q, k, _ = synth.make_qkv(w2)
    assert q.dtype.is_floating_point and str(q.dtype) == "torch.bfloat16"
    # per-block offsets make block means spread well beyond the 1/sqrt(128) noise
    km = k.float().view(2, -1, 128, 128).mean(2)
    assert km.std().item() > 0.3
