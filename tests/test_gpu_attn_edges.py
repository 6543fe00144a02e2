"""GPU parity of the bf16 d = 128 sparse attention kernel on shapes the
benchmark does not reach: an odd number of query blocks (a workgroup whose
second team has no block), rows with no tile at all, attention without the
current chunk, and more query blocks than the in-kernel longest-first ordering
stages (its plain-order fallback). Rows are compared with the float64 oracle
at the bf16 tolerance. The unit schedule written to the workspace changes no
output bit against the in-kernel ranking used without one."""

import numpy as np
import pytest
import torch

import geometry_routed_block_amd as velox
import oracle
import synth
from gpu_common import LSE_ATOL, O_ATOL, say, to_np

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _case(H, N, M, lens, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(H, N * 128, 128, generator=g).to(torch.bfloat16)
    k = torch.randn(H, (M + N) * 128, 128, generator=g).to(torch.bfloat16)
    v = torch.randn(H, (M + N) * 128, 128, generator=g).to(torch.bfloat16)
    rng = np.random.default_rng(seed)
    L = max(1, int(lens.max()))
    ids = np.full((H, N, L), -1, np.int32)
    routes = [[[] for _ in range(N)] for _ in range(H)]
    for h in range(H):
        for i in range(N):
            r = np.sort(rng.choice(M, int(lens[h, i]), replace=False)).astype(np.int32)
            ids[h, i, : len(r)] = r
            routes[h][i] = r.tolist()
    return q, k, v, torch.from_numpy(ids), torch.from_numpy(lens.astype(np.int32)), routes


def _check(q, k, v, o, lse, routes, rows, M, N, include_current):
    qn, kn, vn = to_np(q), to_np(k), to_np(v)
    o_np, lse_np = to_np(o), lse.cpu().numpy()
    for h, i in rows:
        got = o_np[h, i * 128:(i + 1) * 128].astype(np.float64)
        if not include_current and len(routes[h][i]) == 0:   # no tile: o = 0, lse = -inf
            assert np.all(got == 0) and np.all(np.isneginf(lse_np[h, i * 128:(i + 1) * 128]))
            continue
        ref_o, ref_l = oracle.sparse_attention_block(qn, kn, vn, 128 ** -0.5, h, i, routes[h][i], M, N,
                                                     include_current)
        assert np.abs(got - ref_o).max() <= O_ATOL["bf16"], f"row ({h}, {i})"
        assert np.abs(lse_np[h, i * 128:(i + 1) * 128] - ref_l).max() <= LSE_ATOL["bf16"], f"row ({h}, {i})"


@pytest.mark.parametrize("include_current", [True, False])
def test_odd_query_blocks_and_empty_rows(include_current):
    H, N, M = 3, 7, 50
    rng = np.random.default_rng(7)
    lens = rng.integers(0, 30, size=(H, N))
    lens[0, 3] = 0
    lens[1, :] = 0          # a whole head without routed tiles
    lens[2, 6] = M          # every history tile
    say(f"odd N={N}, include_current={include_current}")
    q, k, v, ids, lt, routes = _case(H, N, M, lens, 11)
    o, lse = velox.sparse_attn(q.to(DEV), k.to(DEV), v.to(DEV), ids.to(DEV), lt.to(DEV), M,
                               include_current=include_current, want_lse=True)
    torch.cuda.synchronize()
    _check(q, k, v, o, lse, routes, [(h, i) for h in range(H) for i in range(N)], M, N, include_current)


def test_many_query_blocks_plain_order_fallback():
    # 1030 query blocks of one head: more rows than the longest-first ordering
    # stages in LDS, so the workgroups take the pairs in plain order
    H, N, M = 1, 1030, 24
    rng = np.random.default_rng(3)
    lens = rng.integers(0, M + 1, size=(H, N))
    say(f"many query blocks N={N}")
    q, k, v, ids, lt, routes = _case(H, N, M, lens, 5)
    o, lse = velox.sparse_attn(q.to(DEV), k.to(DEV), v.to(DEV), ids.to(DEV), lt.to(DEV), M,
                               include_current=False, want_lse=True)
    torch.cuda.synchronize()
    rows = [(0, int(i)) for i in rng.choice(N, 12, replace=False)] + [(0, int(np.argmax(lens[0])))]
    _check(q, k, v, o, lse, routes, rows, M, N, False)
    assert torch.isfinite(o.float()).all()


def _raw_sparse(q, k, v, ids, lens, M, workspace):
    """velox_sparse_attn through the C ABI with an explicit (possibly NULL) workspace."""
    import ctypes
    from geometry_routed_block_amd import _lib
    H, NT, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty(H, NT, dtype=torch.float32, device=q.device)
    lib = _lib.load()
    _lib.check(lib.velox_sparse_attn(q.data_ptr(), k.data_ptr(), v.data_ptr(), _lib.VELOX_BF16,
                                     q.stride(0), k.stride(0), H, NT // 128, M, d,
                                     ctypes.c_float(1.0 / d ** 0.5), ids.data_ptr(), lens.data_ptr(),
                                     ids.shape[-1], 1, o.data_ptr(), lse.data_ptr(),
                                     None if workspace is None else workspace.data_ptr(),
                                     torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("wlname,N", [("chunk48", 36), ("wan13", 35)])
def test_unit_plan_matches_in_kernel_ranking_bitwise(wlname, N):
    """The unit schedule written into the workspace only decides which rows
    share a workgroup and when they run: outputs are bitwise those of the
    call without a workspace (every workgroup ranking the units itself)."""
    wl = synth.chunk48() if wlname == "chunk48" else synth.wan13()
    say(f"unit plan vs in-kernel ranking on {wlname}, N={N}")
    q, k, v = synth.make_qkv(wl, device=DEV)
    q = q[:, : N * 128].contiguous()
    kbar = velox.block_mean(k[:, : wl.M * 128])
    p = velox.route_scores(q, kbar, wl.M)
    g = torch.from_numpy(wl.g[:N]).to(DEV)
    rho = torch.from_numpy(wl.rho[:N]).to(DEV)
    coord = torch.from_numpy(np.ascontiguousarray(
        np.concatenate([wl.coords[: wl.M], wl.coords[wl.M: wl.M + N]]), np.int32)).to(DEV)
    ids, lens = velox.route_select(p, g, rho, coord, wl.params)
    ws = velox.attn_workspace(q, ids.shape[-1])
    o1, l1 = _raw_sparse(q, k, v, ids, lens, wl.M, ws)
    o0, l0 = _raw_sparse(q, k, v, ids, lens, wl.M, None)
    assert torch.equal(o1, o0) and torch.equal(l1, l0)
    o2, l2 = velox.sparse_attn(q, k, v, ids, lens, wl.M, want_lse=True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("n_split", [2, 5, 16])
def test_adaptive_split_odd_blocks_and_few_pairs(n_split):
    """Split rows with few pairs per XCD (3 heads x 3 pairs: two XCDs hold two
    pairs, six hold one), a pair whose second row does not exist (N = 5), a
    row without routed tiles, and routes of very different lengths, so the
    unit plan cuts pairs into different numbers of ranges: every row equals
    the unsplit call's up to float rounding, sampled rows the oracle's."""
    H, N, M = 3, 5, 60
    rng = np.random.default_rng(11 + n_split)
    lens = rng.integers(1, 55, size=(H, N))
    lens[2, 4] = 0
    lens[0, 0] = 55
    q, k, v, ids, ln, routes = _case(H, N, M, lens, 20 + n_split)
    q, k, v, ids, ln = (t.to(DEV) for t in (q, k, v, ids, ln))
    say(f"adaptive split: H={H} N={N} M={M} n_split={n_split}")
    o, lse = velox.sparse_attn(q, k, v, ids, ln, M, want_lse=True)
    ws = velox.split_workspace(q, n_split)
    ws.fill_(0xFF)
    o_s, lse_s = velox.sparse_attn(q, k, v, ids, ln, M, want_lse=True, n_split=n_split, workspace=ws)
    torch.cuda.synchronize()
    assert float((o_s.float() - o.float()).abs().max()) <= 8e-3
    assert float((lse_s - lse).abs().max()) <= 1e-4
    _check(q, k, v, o_s, lse_s, routes, [(0, 0), (1, 4), (2, 4), (2, 1)], M, N, True)


def test_binding_rejects_misshaped_router_tensors():
    """The binding raises before any launch when kbar holds too few history
    rows or another head count / head dim, or when p is not [H][N][M]: the C
    ABI sees only pointers and would read or write out of bounds."""
    H, N, M, d = 2, 3, 10, 128
    q = torch.zeros(H, N * 128, d, dtype=torch.bfloat16, device=DEV)
    for bad in ((H, M - 1, d), (H + 1, M, d), (H, M, 64)):
        with pytest.raises(ValueError):
            velox.route_scores(q, torch.zeros(*bad, device=DEV), M)
        with pytest.raises(ValueError):
            velox.route_scores_shared(q, torch.zeros(*bad, device=DEV), M)
    kbar = torch.zeros(H, M, d, device=DEV)
    with pytest.raises(ValueError):
        velox.route_scores(q, kbar, M, out=torch.empty(H, N, M - 1, device=DEV))
    p = velox.route_scores(q, kbar, M)
    torch.cuda.synchronize()
    assert torch.allclose(p, torch.full_like(p, 1.0 / M))   # zero means: uniform importance


def test_binding_rejects_misshaped_block_mean_and_append_tensors():
    """block_mean: more blocks than x holds, or an output with too few rows;
    kv_append: a cache too short for the chunk at its offset, another head
    count, or a key-mean cache too short: all raise before any launch."""
    H, d = 2, 128
    x = torch.zeros(H, 4 * 128, d, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):
        velox.block_mean(x, nblk=5)
    with pytest.raises(ValueError):
        velox.block_mean(x, out=torch.empty(H, 3, d, device=DEV))
    T, Hl, Wl = 1, 16, 16                       # 256 tokens = 2 blocks
    new = torch.zeros(H, T * Hl * Wl, d, dtype=torch.bfloat16, device=DEV)
    cells = torch.from_numpy(velox.gilbert_curve(Wl, Hl)).to(DEV)
    short = torch.zeros(H, 3 * 128, d, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):             # offset 256 + 256 tokens > 384 rows
        velox.kv_append(new, new, T, Hl, Wl, 0, cells, short, short, 256)
    other = torch.zeros(H + 1, 4 * 128, d, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):
        velox.kv_append(new, new, T, Hl, Wl, 0, cells, other, other, 0)
    cache = torch.zeros(H, 4 * 128, d, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):
        velox.kv_append(new, new, T, Hl, Wl, 0, cells, cache, cache.clone(), 256,
                        kbar=torch.zeros(H, 3, d, device=DEV))
    kb = torch.zeros(H, 4, d, device=DEV)
    velox.kv_append(new, new, T, Hl, Wl, 0, cells, cache, cache.clone(), 256, kbar=kb)
    torch.cuda.synchronize()
    assert float(kb.abs().max()) == 0.0         # zero chunk: zero key means
