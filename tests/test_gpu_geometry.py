"""GPU parity of the geometry scorer (velox_slab_overlap, velox_slab_coverage)
against the float32 oracle: both take every inside/outside decision in float32
with the same operation order, so g, rho and the token masks must match
bit for bit."""

import numpy as np
import pytest
import torch

import geometry_routed_block_amd as velox
import synth
from oracle import geometry as geo
from gpu_common import say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _random_scene(seed, N, M, invalid=0.1):
    rng = np.random.default_rng(seed)

    def boxes(n):
        recs = np.zeros((n, 16), np.float32)
        for b in range(n):
            a = rng.normal(size=3)
            a /= np.linalg.norm(a)
            ang = rng.uniform(0, np.pi)
            K = np.array([[0, -a[2], a[1]], [a[2], 0, -a[0]], [-a[1], a[0], 0]])
            R = np.eye(3) + np.sin(ang) * K + (1 - np.cos(ang)) * K @ K
            recs[b, 0:3] = rng.uniform(-2, 2, 3)
            recs[b, 3:6] = rng.uniform(0.2, 1.5, 3)
            recs[b, 6:15] = R.reshape(9)
            if rng.uniform() < invalid:
                recs[b, 3 + rng.integers(0, 3)] = 0.0 if rng.uniform() < 0.5 else -1.0
        return recs

    pts = rng.uniform(-3, 3, size=(N, 128, 3)).astype(np.float32)
    pts[:, :5] = np.nan
    return boxes(N), boxes(M), pts


def _mask_bits(mask_words):
    w = mask_words.cpu().numpy().astype(np.int64) & 0xffffffff
    bits = (w[:, :, None] >> np.arange(32)) & 1
    return bits.reshape(w.shape[0], 128).astype(bool)


@pytest.mark.parametrize("name", ["chunk48", "wan13"])
def test_overlap_and_coverage_bit_exact_at_full_size(name):
    wl = getattr(synth, name)()
    sc = wl.scene
    say(f"geometry {name}: N={wl.N} M={wl.M}")
    q, h, pts = _dev(sc["obb_query"]), _dev(sc["obb_hist"]), _dev(sc["query_pts"])
    g = velox.slab_overlap(q, h, lattice=8)
    rho, mask = velox.slab_coverage(pts, h)
    torch.cuda.synchronize()
    g_ref = geo.slab_overlap(sc["obb_query"], sc["obb_hist"], n=8)
    cov_ref = geo.token_covered(sc["query_pts"], sc["obb_hist"])
    assert np.array_equal(g.cpu().numpy(), g_ref)
    assert np.array_equal(_mask_bits(mask), cov_ref)
    assert np.array_equal(rho.cpu().numpy(), geo.slab_coverage(sc["query_pts"], sc["obb_hist"]))
    assert (g_ref > 0).mean() > 0.02


@pytest.mark.parametrize("n", [1, 3, 8, 9, 16])
def test_lattice_sizes_and_invalid_boxes(n):
    qo, ho, pts = _random_scene(10 + n, 5, 77)
    say(f"geometry lattice n={n}")
    g = velox.slab_overlap(_dev(qo), _dev(ho), lattice=n)
    rho, mask = velox.slab_coverage(_dev(pts), _dev(ho))
    torch.cuda.synchronize()
    assert np.array_equal(g.cpu().numpy(), geo.slab_overlap(qo, ho, n=n))
    assert np.array_equal(_mask_bits(mask), geo.token_covered(pts, ho))
    assert np.array_equal(rho.cpu().numpy(), geo.slab_coverage(pts, ho))


def test_identical_boxes_and_empty_history():
    qo, ho, pts = _random_scene(3, 4, 4, invalid=0.0)
    say("geometry identical boxes")
    g = velox.slab_overlap(_dev(qo), _dev(qo), lattice=8).cpu().numpy()
    assert (np.diag(g) == 1.0).all()
    empty = torch.zeros(0, 16, dtype=torch.float32, device=DEV)
    rho, mask = velox.slab_coverage(_dev(pts), empty)
    torch.cuda.synchronize()
    assert (rho.cpu().numpy() == 0).all() and (mask.cpu().numpy() == 0).all()
    assert velox.slab_overlap(_dev(qo), empty).shape == (4, 0)


def test_reuse_of_outputs_clears_stale_bits():
    qo, ho, pts = _random_scene(4, 3, 50, invalid=0.0)
    say("geometry output reuse")
    rho = torch.full((3,), 7.0, device=DEV)
    mask = torch.full((3, 4), -1, dtype=torch.int32, device=DEV)
    velox.slab_coverage(_dev(pts), _dev(ho), rho=rho, token_mask=mask)
    torch.cuda.synchronize()
    assert np.array_equal(_mask_bits(mask), geo.token_covered(pts, ho))
    assert np.array_equal(rho.cpu().numpy(), geo.slab_coverage(pts, ho))
