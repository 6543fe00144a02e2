"""Seeded synthetic workloads for the routed history-attention path.

Each workload fixes shapes, router settings and the seeds of every random
input. Both the oracle side and the GPU side take their inputs from here; this
module holds no routing or attention arithmetic.

Shapes follow the pages' setting: 128-token blocks (FlashAttention tile size),
36 blocks per generated chunk, 48-chunk rollouts (project page, 03 · Results,
Figure 3 caption; digest, Motivation). Router settings tau = 0.1, g_ref = 0.2,
lambda = 2, eta_cov = 0.9, K_cov = 80, K_unc = 150 are the pages' values (digest,
Core method; onedev summary, "What differs").

Recipe for q/k/v: standard normal draws (torch generator, seeded), plus a
per-(head, block) mean offset ~ N(0, sigma^2) added to all 128 tokens of the
block, so block importances are not uniform; cast to the workload dtype
(round-to-nearest-even for bf16).
"""

from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field

import numpy as np

from .geometry import _token_depths, assign_coverage, mc_overlap, pack_obbs, slab_obbs, token_points
from .blockgrid import chunk_block_coords

BLOCK = 128          # tokens per block = attention tile (b_tok)
CHUNK_BLOCKS = 36    # blocks per generated chunk
GRID_H, GRID_W = 4, 9


@dataclass
class RouteParams:
    """Router settings (plain container; the arithmetic lives elsewhere)."""
    tau: float = 0.1
    g_ref: float = 0.2
    lam: float = 2.0
    eta_cov: float = 0.9
    theta_cov: float = 1.0      # >= 1: no mass cut (pure top-K_cov)
    theta_unc: float = 0.9      # mass threshold for the uncovered prefix
    K_cov: int = 80
    K_unc: int = 150
    n_prev: int = 0             # last n_prev history ids are always kept
    neigh26: int = 0            # add Chebyshev-1 grid neighbours of the query block
    ref_ids: tuple = ()         # extra always-added history ids
    mode: int = 0               # covered rows: 0 fused, 1 model only, 2 geometry only

    def replace(self, **kw) -> "RouteParams":
        return dataclasses.replace(self, **kw)


@dataclass
class Workload:
    name: str
    H: int
    d: int
    dtype: str                   # "f32" | "bf16"
    N: int                       # query blocks (current chunk)
    M: int                       # visible history blocks
    seed: int
    offset_sigma: float
    params: RouteParams
    coords: np.ndarray           # [(M+N), 3] int32 (t, h, w) block grid
    g: np.ndarray                # [N, M] float32 overlaps in [0, 1]
    rho: np.ndarray              # [N] float32 coverage
    kv_blocks: int = 0           # KV capacity in blocks (>= M + N)
    notes: dict = field(default_factory=dict)
    # slab scene behind g (None for hand-made overlaps): "obb_hist" [M,16] and
    # "obb_query" [N,16] packed float32 OBB records, "query_pts" [N,128,3]
    # float32 token world points (NaN = no depth)
    scene: dict | None = None

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))

    @property
    def route_cap(self) -> int:
        """Route list length L that always suffices (ids are < M)."""
        p = self.params
        bound = max(p.K_cov, p.K_unc, p.n_prev) + 26 * p.neigh26 + len(p.ref_ids)
        return max(1, min(self.M, bound))


def _slab_geometry(coords: np.ndarray, M: int, N: int, seed: int):
    """Slab scene of M history + N query blocks; g by seeded Monte Carlo IoU."""
    rng = np.random.default_rng(seed)
    chunk = coords[:, 0]
    depths = _token_depths(rng, M + N)
    c, ax, hf = slab_obbs(coords, chunk, GRID_H, GRID_W, rng, depths=depths)
    pts = token_points(coords[M:], chunk[M:], GRID_H, GRID_W, depths[M:], rng)
    g = mc_overlap(c[M:], ax[M:], hf[M:], c[:M], ax[:M], hf[:M], rng)
    scene = {"obb_hist": pack_obbs(c[:M], ax[:M], hf[:M]),
             "obb_query": pack_obbs(c[M:], ax[M:], hf[M:]), "query_pts": pts}
    return g.astype(np.float32), rng, scene


def tiny() -> Workload:
    """2 heads, d = 64, fp32, 4 query blocks, 16 history blocks on a 4x2x2 grid."""
    rng = np.random.default_rng(0)
    N, M = 4, 16
    g = (rng.uniform(0.0, 1.0, size=(N, M)) * (rng.uniform(size=(N, M)) < 0.3))
    coords = chunk_block_coords(5, 2, 2)          # 4 history chunks + current at t=4
    prm = RouteParams(K_cov=6, K_unc=10, n_prev=4, neigh26=1)
    rho = np.array([0.95, 0.3, 0.95, 0.3], dtype=np.float32)
    return Workload("tiny", 2, 64, "f32", N, M, 0, 0.0, prm, coords,
                    g.astype(np.float32), rho, kv_blocks=M + N)


def wan13() -> Workload:
    """Wan-1.3B-like layer: 12 heads, d = 128, bf16, 36 query, 143 history blocks."""
    N, M = 36, 143
    coords = chunk_block_coords(5, GRID_H, GRID_W, first_id_offset=5 * 36 - (M + N))
    g, rng, scene = _slab_geometry(coords, M, N, seed=1)
    rho = assign_coverage(N, 0.6, rng)
    prm = RouteParams()
    return Workload("wan13", 12, 128, "bf16", N, M, 1, 0.5, prm, coords, g, rho,
                    kv_blocks=M + N, scene=scene)


def chunk48(covered_fraction: float = 0.6, seed: int = 48, name: str = "chunk48",
            heads: int = 40) -> Workload:
    """Chunk-48 late rollout: 40 heads, d = 128, bf16, 36 query, 1692 history blocks."""
    N = CHUNK_BLOCKS
    M = 47 * CHUNK_BLOCKS
    coords = chunk_block_coords(48, GRID_H, GRID_W)
    g, rng, scene = _slab_geometry(coords, M, N, seed=seed)
    rho = assign_coverage(N, covered_fraction, rng)
    prm = RouteParams(n_prev=CHUNK_BLOCKS, neigh26=1)
    return Workload(name, heads, 128, "bf16", N, M, seed, 0.5, prm, coords, g, rho,
                    kv_blocks=M + N, notes={"covered_fraction": covered_fraction}, scene=scene)


def sweep(covered_fraction: float) -> Workload:
    seed = {0.0: 480, 0.5: 481, 1.0: 482}[covered_fraction]
    return chunk48(covered_fraction, seed=seed,
                   name=f"chunk48_cov{int(round(covered_fraction * 100))}")


def trace_chunk(chunk: int, layer: int, heads: int = 40) -> Workload:
    """Chunk `chunk` (1-based) of a 48-chunk rollout, layer `layer` (seed 1000 + layer)."""
    N = CHUNK_BLOCKS
    M = CHUNK_BLOCKS * (chunk - 1)
    coords = chunk_block_coords(chunk, GRID_H, GRID_W)
    if M > 0:
        g, rng, scene = _slab_geometry(coords, M, N, seed=1000 + layer)
    else:
        g, rng, scene = np.zeros((N, 0), np.float32), np.random.default_rng(1000 + layer), None
    rho = assign_coverage(N, 0.6, rng)
    prm = RouteParams(n_prev=min(CHUNK_BLOCKS, M), neigh26=1)
    return Workload(f"trace_c{chunk}_l{layer}", heads, 128, "bf16", N, M, 1000 + layer,
                    0.5, prm, coords, g, rho, kv_blocks=M + N, scene=scene)


def make_qkv(wl: Workload, device="cpu", kv_blocks: int | None = None):
    """Seeded q [H][N*128][d], k and v [H][kv_blocks*128][d] as torch tensors.

    Draw order: q, k, v, then the q, k, v block offsets. kv_blocks defaults to
    wl.kv_blocks; blocks beyond M + N are filled with the same distribution.
    """
    import torch

    cap = kv_blocks if kv_blocks is not None else wl.kv_blocks
    assert cap >= wl.M + wl.N
    gen = torch.Generator(device=device)
    gen.manual_seed(wl.seed)
    H, d, N = wl.H, wl.d, wl.N
    q = torch.randn(H, N * BLOCK, d, generator=gen, device=device)
    k = torch.randn(H, cap * BLOCK, d, generator=gen, device=device)
    v = torch.randn(H, cap * BLOCK, d, generator=gen, device=device)
    if wl.offset_sigma > 0:
        for t, nb in ((q, N), (k, cap), (v, cap)):
            off = torch.randn(H, nb, 1, d, generator=gen, device=device) * wl.offset_sigma
            t.view(H, nb, BLOCK, d).add_(off)
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    return q.to(dt), k.to(dt), v.to(dt)


WORKLOADS = {
    "tiny": tiny,
    "wan13": wan13,
    "chunk48": chunk48,
}
