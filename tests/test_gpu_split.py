"""GPU parity of split-row attention (velox_sparse_attn_split /
velox_dense_attn_split): every row's tiles cut into ranges handled by separate
workgroups and merged. Checked against the float64 oracle on sampled rows and
against the unsplit call on every row, at one GPU's share of the chunk-48
heads (5 heads), with more ranges than some rows have tiles, without the
current chunk, and on the fp32 path (which runs unsplit)."""

import numpy as np
import pytest
import torch

import geometry_routed_block_amd as velox
import synth
from gpu_common import check_attention_rows, check_routes_exact, run_path, say, to_np

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _close(a, b, atol):
    return float((a.float() - b.float()).abs().max()) <= atol


@pytest.mark.parametrize("n_split", [2, 3, 7, 16])
def test_split_at_five_heads_of_chunk48(n_split):
    wl = synth.chunk48(heads=5)
    say(f"chunk48 x 5 heads, n_split={n_split}")
    q, k, v = synth.make_qkv(wl, device=DEV)
    r = run_path(wl, q, k, v)
    routes = check_routes_exact(wl, r["p"], r["ids"], r["lens"], rows=[(0, 0), (4, 35)])
    routes = [[r["ids"][h, i, : int(r["lens"][h, i])].tolist() for i in range(wl.N)] for h in range(wl.H)]
    o_s, lse_s = velox.sparse_attn(q, k, v, r["ids"], r["lens"], wl.M, want_lse=True, n_split=n_split)
    torch.cuda.synchronize()
    # the same attention as the unsplit call, up to float rounding
    assert _close(o_s, r["o"], 8e-3) and _close(lse_s, r["lse"], 1e-4)
    rng = np.random.default_rng(n_split)
    rows = [(int(rng.integers(wl.H)), int(rng.integers(wl.N))) for _ in range(4)]
    qn, kn, vn = to_np(q), to_np(k), to_np(v)
    check_attention_rows(wl, qn, kn, vn, o_s, lse_s, routes, rows)
    o_d, lse_d = velox.dense_attn(q, k, v, wl.M, want_lse=True)
    o_ds, lse_ds = velox.dense_attn(q, k, v, wl.M, want_lse=True, n_split=n_split)
    torch.cuda.synchronize()
    assert _close(o_ds, o_d, 8e-3) and _close(lse_ds, lse_d, 1e-4)
    check_attention_rows(wl, qn, kn, vn, o_ds, lse_ds, None, rows[:1], dense=True)


def test_more_ranges_than_tiles_and_no_current_chunk():
    wl = synth.wan13()
    say("wan13: 16 ranges, short routes, no current chunk")
    q, k, v = synth.make_qkv(wl, device=DEV)
    r = run_path(wl, q, k, v, include_current=False)
    lens = r["lens"].clone()
    lens[:, ::3] = torch.clamp(lens[:, ::3], max=5)       # rows shorter than the range count
    lens[0, 1] = 0                                         # a row with no tile at all
    o, lse = velox.sparse_attn(q, k, v, r["ids"], lens, wl.M, include_current=False, want_lse=True)
    o_s, lse_s = velox.sparse_attn(q, k, v, r["ids"], lens, wl.M, include_current=False, want_lse=True,
                                   n_split=16)
    torch.cuda.synchronize()
    assert torch.all(o_s[0, 128:256] == 0) and torch.all(torch.isneginf(lse_s[0, 128:256]))
    fin = torch.isfinite(lse)
    assert torch.equal(fin, torch.isfinite(lse_s))
    assert _close(o_s, o, 8e-3) and float((lse_s[fin] - lse[fin]).abs().max()) <= 1e-4
    routes = [[r["ids"][h, i, : int(lens[h, i])].tolist() for i in range(wl.N)] for h in range(wl.H)]
    check_attention_rows(wl, to_np(q), to_np(k), to_np(v), o_s, lse_s, routes, [(0, 0), (3, 3), (11, 35)],
                         include_current=False)


def test_fp32_runs_unsplit():
    wl = synth.tiny()
    q, k, v = synth.make_qkv(wl, device=DEV)
    r = run_path(wl, q, k, v)
    o_s, lse_s = velox.sparse_attn(q, k, v, r["ids"], r["lens"], wl.M, want_lse=True, n_split=4)
    torch.cuda.synchronize()
    assert torch.equal(o_s, r["o"]) and torch.equal(lse_s, r["lse"])


@pytest.mark.parametrize("heads,n_split", [(40, 4), (40, 16), (5, 16)])
def test_adaptive_ranges_match_unsplit(heads, n_split):
    """The unit plan cuts each pair into as many ranges as one round of an
    XCD's CUs holds (none at 40 heads: 90 pairs per XCD, so every row has
    n_split - 1 unused ranges whose partials are the 0xFF fill; up to n_split
    at 5 heads): outputs equal the unsplit call's up to float rounding on
    every row."""
    wl = synth.chunk48(heads=heads)
    say(f"chunk48 x {heads} heads, adaptive ranges up to {n_split}")
    q, k, v = synth.make_qkv(wl, device=DEV)
    r = run_path(wl, q, k, v)
    ws = velox.split_workspace(q, n_split)
    ws.fill_(0xFF)  # stale workspace contents must not leak into the merge
    o_s, lse_s = velox.sparse_attn(q, k, v, r["ids"], r["lens"], wl.M, want_lse=True, n_split=n_split,
                                   workspace=ws)
    o_s2, lse_s2 = velox.sparse_attn(q, k, v, r["ids"], r["lens"], wl.M, want_lse=True, n_split=n_split,
                                     workspace=ws)
    torch.cuda.synchronize()
    assert _close(o_s, r["o"], 8e-3) and _close(lse_s, r["lse"], 1e-4)
    assert torch.equal(o_s, o_s2) and torch.equal(lse_s, lse_s2)
