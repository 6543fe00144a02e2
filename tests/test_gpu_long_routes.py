"""GPU parity of the attention kernels that serve long routes: routes of more
than 2048 tiles use the one-block-per-workgroup kernel with route ids staged
in LDS (up to 4096), longer ones its register-staged variant. Sampled rows are
compared with the float64 oracle at the bf16 tolerance."""

import numpy as np
import pytest
import torch

import geometry_routed_block_amd as velox
import oracle
from gpu_common import LSE_ATOL, O_ATOL, say, to_np

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.mark.parametrize("M,route_lens", [(2600, [2500, 2100, 7, 2600]), (4500, [4300, 4097, 300, 0])])
def test_long_routes_bf16_d128(M, route_lens):
    H, N, d = 1, 4, 128
    say(f"long routes M={M} lens={route_lens}")
    g = torch.Generator().manual_seed(M)
    q = torch.randn(H, N * 128, d, generator=g).to(torch.bfloat16)
    k = torch.randn(H, (M + N) * 128, d, generator=g).to(torch.bfloat16)
    v = torch.randn(H, (M + N) * 128, d, generator=g).to(torch.bfloat16)
    rng = np.random.default_rng(M)
    L = max(route_lens)
    ids = np.full((H, N, L), -1, np.int32)
    lens = np.array([route_lens], np.int32)
    routes = []
    for i, n in enumerate(route_lens):
        r = np.sort(rng.choice(M, n, replace=False)).astype(np.int32)
        ids[0, i, :n] = r
        routes.append(r.tolist())
    o, lse = velox.sparse_attn(q.to(DEV), k.to(DEV), v.to(DEV), torch.from_numpy(ids).to(DEV),
                               torch.from_numpy(lens).to(DEV), M, want_lse=True)
    torch.cuda.synchronize()
    qn, kn, vn = to_np(q), to_np(k), to_np(v)
    o_np, lse_np = to_np(o), lse.cpu().numpy()
    for i in range(N):
        ref_o, ref_l = oracle.sparse_attention_block(qn, kn, vn, d ** -0.5, 0, i, routes[i], M, N)
        err = np.abs(o_np[0, i * 128:(i + 1) * 128].astype(np.float64) - ref_o).max()
        assert err <= O_ATOL["bf16"], f"row {i}: O error {err:.3g}"
        assert np.abs(lse_np[0, i * 128:(i + 1) * 128] - ref_l).max() <= LSE_ATOL["bf16"]
