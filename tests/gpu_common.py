"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
binding, and compare with the CPU oracle on the same seeded inputs."""

from __future__ import annotations

import sys

import numpy as np
import torch

import geometry_routed_block_amd as velox
import oracle
import synth

P_RTOL = 1e-5            # importance, relative (fp32 path vs float64 oracle)
O_ATOL = {"bf16": 2e-2, "f32": 1e-4}   # attention output, absolute
LSE_ATOL = {"bf16": 1e-2, "f32": 1e-4}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_np(t):
    return t.detach().to("cpu", torch.float32).numpy() if t.dtype == torch.bfloat16 else \
        t.detach().cpu().numpy()


def run_path(wl, q, k, v, include_current=True, L=None):
    """kbar -> p -> routes -> sparse attention, all on the GPU."""
    dev = q.device
    M, N = wl.M, wl.N
    kbar = velox.block_mean(k[:, : M * 128]) if M > 0 else torch.zeros(wl.H, 0, wl.d, device=dev)
    if M > 0:
        p = velox.route_scores(q, kbar, M)
    else:
        p = torch.zeros(wl.H, N, 0, device=dev)
    g = torch.from_numpy(wl.g).to(dev)
    rho = torch.from_numpy(wl.rho).to(dev)
    coord = torch.from_numpy(np.ascontiguousarray(wl.coords, dtype=np.int32)).to(dev)
    ids, lens = velox.route_select(p, g, rho, coord, wl.params, L=L)
    o, lse = velox.sparse_attn(q, k, v, ids, lens, M, include_current=include_current,
                               want_lse=True)
    torch.cuda.synchronize()
    return dict(kbar=kbar, p=p, ids=ids, lens=lens, o=o, lse=lse)


def routes_from_gpu(ids, lens):
    ids, lens = ids.cpu().numpy(), lens.cpu().numpy()
    H, N = lens.shape
    return [[ids[h, i, : lens[h, i]].tolist() for i in range(N)] for h in range(H)]


def check_routes_exact(wl, p_gpu, ids, lens, rows=None):
    """Routes bit-exact against the oracle fed with the GPU's fp32 importances."""
    p_np = p_gpu.cpu().numpy()
    got = routes_from_gpu(ids, lens)
    H, N = p_np.shape[0], p_np.shape[1]
    rows = rows if rows is not None else [(h, i) for h in range(H) for i in range(N)]
    L = ids.shape[-1]
    ids_np = ids.cpu().numpy()
    for h, i in rows:
        ref = oracle.route_row(p_np[h, i], wl.g[i], wl.rho[i], wl.params, wl.M, wl.coords, i)
        assert got[h][i] == ref, f"route mismatch at head {h} block {i}"
        assert np.all(ids_np[h, i, len(ref):] == -1) and len(ref) <= L
    return got


def check_attention_rows(wl, q_np, k_np, v_np, o_gpu, lse_gpu, routes, rows,
                         include_current=True, dense=False):
    o_np = to_np(o_gpu)
    lse_np = lse_gpu.cpu().numpy() if lse_gpu is not None else None
    tol, ltol = O_ATOL[wl.dtype], LSE_ATOL[wl.dtype]
    worst = 0.0
    for h, i in rows:
        if dense:
            ref_o, ref_l = oracle.dense_attention_block(q_np, k_np, v_np, wl.scale, h, i, wl.M, wl.N)
        else:
            ref_o, ref_l = oracle.sparse_attention_block(q_np, k_np, v_np, wl.scale, h, i,
                                                         routes[h][i], wl.M, wl.N,
                                                         include_current)
        got = o_np[h, i * 128:(i + 1) * 128].astype(np.float64)
        err = np.abs(got - ref_o).max()
        worst = max(worst, err)
        assert err <= tol, f"O error {err:.3g} > {tol} at head {h} block {i}"
        if lse_np is not None:
            lerr = np.abs(lse_np[h, i * 128:(i + 1) * 128] - ref_l).max()
            assert lerr <= ltol, f"LSE error {lerr:.3g} at head {h} block {i}"
    return worst


def sample_rows(wl, n, seed):
    """n (head, block) rows, both covered and uncovered blocks included."""
    rng = np.random.default_rng(seed)
    cov = [i for i in range(wl.N) if wl.rho[i] >= np.float32(wl.params.eta_cov)]
    unc = [i for i in range(wl.N) if i not in cov]
    rows = []
    for j in range(n):
        pool = cov if (j % 2 == 0 and cov) or not unc else unc
        rows.append((int(rng.integers(0, wl.H)), int(rng.choice(pool))))
    rows += [(0, 0), (wl.H - 1, wl.N - 1)]
    return sorted(set(rows))
