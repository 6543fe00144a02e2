"""GPU parity of the bf16 d = 128 sparse attention kernel on shapes the
benchmark does not reach: an odd number of query blocks (a workgroup whose
second team has no block), rows with no tile at all, attention without the
current chunk, and more query blocks than the in-kernel longest-first ordering
stages (its plain-order fallback). Rows are compared with the float64 oracle
at the bf16 tolerance."""

import numpy as np
import pytest
import torch

import geometry_routed_block_amd as velox
import oracle
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
