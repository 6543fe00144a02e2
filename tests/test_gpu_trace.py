"""GPU parity along the 48-chunk rollout trace: chunk c has M = 36 (c - 1)
history blocks (the first chunk none), layer seeds 1000 + layer. For each
sampled (chunk, layer), the whole routed path runs on the GPU with 8 heads:
importance within 1e-5 relative, all routes bit-exact, sampled attention rows
and dense rows against the float64 oracle."""

import numpy as np
import pytest
import torch

import geometry_routed_block_amd as velox
import oracle
import synth
from gpu_common import P_RTOL, check_attention_rows, check_routes_exact, run_path, say, to_np

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
HEADS = 8


@pytest.mark.parametrize("chunk,layer", [(1, 0), (2, 3), (7, 11), (20, 39)])
def test_trace_chunk_full_path(chunk, layer):
    wl = synth.trace_chunk(chunk, layer, heads=HEADS)
    say(f"trace chunk {chunk} layer {layer}: M={wl.M}")
    q, k, v = synth.make_qkv(wl, device=DEV)
    r = run_path(wl, q, k, v)
    routes = check_routes_exact(wl, r["p"], r["ids"], r["lens"])
    qn, kn, vn = to_np(q), to_np(k), to_np(v)
    if wl.M > 0:
        qb = oracle.block_means(qn)
        kb = oracle.block_means(kn[:, : wl.M * 128])
        np.testing.assert_allclose(r["p"].cpu().numpy(), oracle.importance(qb, kb, wl.scale),
                                   rtol=P_RTOL, atol=1e-30)
        # the previous chunk is always routed once there is one
        prev = set(range(wl.M - min(36, wl.M), wl.M))
        assert all(prev <= set(routes[h][i]) for h in range(wl.H) for i in range(wl.N))
    else:
        assert all(len(routes[h][i]) == 0 for h in range(wl.H) for i in range(wl.N))
    rng = np.random.default_rng(chunk * 100 + layer)
    rows = [(int(rng.integers(wl.H)), int(rng.integers(wl.N))) for _ in range(6)]
    check_attention_rows(wl, qn, kn, vn, r["o"], r["lse"], routes, rows)
    o_d, lse_d = velox.dense_attn(q, k, v, wl.M, want_lse=True)
    torch.cuda.synchronize()
    check_attention_rows(wl, qn, kn, vn, o_d, lse_d, None, rows[:2], dense=True)
