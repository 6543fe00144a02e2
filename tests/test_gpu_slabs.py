"""GPU parity of the slab table, the recency-priority multiwarp and the token
points against the float32 oracle (bit for bit: both take every decision in
float32 with the same operation order), and of the whole geometry chain
depth -> slabs -> boxes -> overlaps / coverage."""

import numpy as np
import pytest
import torch

import geometry_routed_block_amd as velox
import synth.geometry as sg
from oracle import geometry as ogeo
from oracle import slabs as oslabs
from gpu_common import say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
PIN = (sg.FOCAL, sg.TOKEN_W / 2, sg.TOKEN_H / 2)


def _d(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _same(got, ref):
    """Bitwise-equal float arrays (NaN where NaN)."""
    got = np.asarray(got)
    ref = np.asarray(ref, dtype=got.dtype)
    return got.shape == ref.shape and np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_slab_table_bit_exact():
    cells, depth, cams, cob = sg.slab_inputs()
    say(f"slab table: {depth.size // 128} blocks")
    s_gpu, b_gpu = velox.slab_table(_d(cells), _d(depth), _d(cams), _d(cob), *PIN, n_min=8)
    torch.cuda.synchronize()
    s_ref, b_ref = oslabs.slab_table(cells, depth, cams, cob, *PIN, n_min=8)
    assert _same(s_gpu.cpu().numpy(), s_ref)
    assert _same(b_gpu.cpu().numpy(), b_ref)
    assert (s_ref[:, 7] == 0).sum() >= 2 and (s_ref[:, 7] == 1).sum() > 100


@pytest.mark.parametrize("n_cached,scale", [(4, 2), (2, 4)])
def test_multiwarp_bit_exact(n_cached, scale):
    fr, cams, ss, sp, tgt, ts, tp, cells = sg.multiwarp_inputs(n_cached=n_cached, scale=scale)
    say(f"multiwarp: {fr.shape[0]} frames of {ss[0]}x{ss[1]} -> {ts[0]}x{ts[1]}")
    zq, chosen = velox.multiwarp(_d(fr), _d(cams), ss, sp, _d(tgt), ts, tp, k_warp=2)
    torch.cuda.synchronize()
    zq_ref, ch_ref = oslabs.multiwarp(list(fr), list(cams), ss[0], ss[1], sp, tgt, ts[0], ts[1], tp, 2)
    assert np.array_equal(chosen.cpu().numpy(), ch_ref)
    assert _same(zq.cpu().numpy(), zq_ref)
    assert len(set(ch_ref[ch_ref >= 0].tolist())) >= 2          # recency fallback exercised


def test_multiwarp_without_frames_and_with_a_high_bar():
    fr, cams, ss, sp, tgt, ts, tp, cells = sg.multiwarp_inputs(n_cached=1, scale=2)
    say("multiwarp edge cases")
    empty = torch.zeros(0, dtype=torch.float32, device=DEV)
    zq, chosen = velox.multiwarp(empty, torch.zeros(0, 12, device=DEV), ss, sp, _d(tgt), ts, tp)
    torch.cuda.synchronize()
    assert torch.isnan(zq).all() and (chosen == -1).all()
    zq, chosen = velox.multiwarp(_d(fr), _d(cams), ss, sp, _d(tgt), ts, tp, k_warp=10 ** 6)
    torch.cuda.synchronize()
    assert torch.isnan(zq).all() and (chosen == -1).all()


def test_geometry_chain_bit_exact():
    # cached depth -> query depth -> token points and query slabs; history
    # slabs -> boxes; overlaps and coverage of the query blocks
    fr, cams, ss, sp, tgt, ts, tp, qcells = sg.multiwarp_inputs(n_cached=3, scale=2)
    hcells, hdepth, hcams, hcob = sg.slab_inputs(seed=3)
    say("geometry chain")
    zq, _ = velox.multiwarp(_d(fr), _d(cams), ss, sp, _d(tgt), ts, tp)
    qdepth, qpts = velox.token_points(_d(qcells), zq, ts[0], ts[1], _d(tgt), *tp)
    qcam_of_block = torch.zeros(36, dtype=torch.int32, device=DEV)
    _, qbox = velox.slab_table(_d(qcells), qdepth, _d(tgt).view(1, 12), qcam_of_block, *tp, n_min=8)
    _, hbox = velox.slab_table(_d(hcells), _d(hdepth), _d(hcams), _d(hcob), *PIN, n_min=8)
    g = velox.slab_overlap(qbox, hbox)
    rho, _ = velox.slab_coverage(qpts.view(36, 128, 3), hbox)
    torch.cuda.synchronize()
    zq_ref, _ = oslabs.multiwarp(list(fr), list(cams), ss[0], ss[1], sp, tgt, ts[0], ts[1], tp, 2)
    qd_ref, qp_ref = oslabs.token_points(qcells, zq_ref, ts[0], ts[1], tgt, *tp)
    assert _same(qdepth.cpu().numpy(), qd_ref) and _same(qpts.cpu().numpy(), qp_ref)
    _, qbox_ref = oslabs.slab_table(qcells, qd_ref, tgt[None], np.zeros(36, np.int32), *tp, n_min=8)
    _, hbox_ref = oslabs.slab_table(hcells, hdepth, hcams, hcob, *PIN, n_min=8)
    assert _same(qbox.cpu().numpy(), qbox_ref) and _same(hbox.cpu().numpy(), hbox_ref)
    g_ref = ogeo.slab_overlap(qbox_ref, hbox_ref)
    assert _same(g.cpu().numpy(), g_ref)
    assert _same(rho.cpu().numpy(), ogeo.slab_coverage(qp_ref.reshape(36, 128, 3), hbox_ref))
