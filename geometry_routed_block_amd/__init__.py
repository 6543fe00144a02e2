"""Routed block-sparse history attention for MI355X (gfx950).

Thin PyTorch binding of libvelox.so: every function here only checks tensor
metadata, marshals pointers and the current HIP stream, and calls the C ABI of
include/velox.h, include/velox_geometry.h, include/velox_layout.h and
include/velox_slabs.h. All
computation runs in the library's HIP kernels (the curve of velox_gilbert_curve
is computed by the library's host code).

Layouts (row-major, token rows contiguous):
    q            [H][N*128][d]          bf16 or fp32
    k, v         [H][>=(M+N)*128][d]    history blocks 0..M-1, current chunk M..M+N-1
    kbar         [H][>=M][d]            fp32 key-mean cache
    p            [H][N][M]              fp32 importance
    g            [N][M] fp32, rho [N] fp32, coord [M+N][3] int32
    route_ids    [H][N][L] int32, route_len [H][N] int32
    o            [H][N*128][d]          dtype of q;  lse [H][N*128] fp32
    obb records  [n][16] fp32 (centre, half-extents, axes row-major, unused)
    q_pts        [N][128][3] fp32 token world points (NaN = no depth)
"""

from __future__ import annotations

import ctypes
import math

from . import _lib
from ._lib import VELOX_BLOCK, VeloxError

__all__ = ["VELOX_BLOCK", "VeloxError", "block_mean", "route_scores", "route_select",
           "route_bound", "sparse_attn", "dense_attn", "slab_overlap", "slab_coverage",
           "gilbert_curve", "kv_append", "route_scores_shared", "slab_table", "multiwarp",
           "token_points", "library_path", "split_workspace", "attn_workspace", "check_routes"]


def library_path() -> str:
    return _lib.LIB_PATH


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return _lib.VELOX_BF16
    if t.dtype == torch.float32:
        return _lib.VELOX_F32
    raise TypeError(f"unsupported dtype {t.dtype}: use bfloat16 or float32")


def _require_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must live on the GPU")


def _rows(t, name):
    """Head stride of a [H][T][d] tensor whose token rows are contiguous."""
    if t.dim() != 3 or t.stride(2) != 1 or t.stride(1) != t.shape[2]:
        raise ValueError(f"{name} must be [H][T][d] with contiguous token rows")
    return t.stride(0)


def _contig(t, name):
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(t) -> int:
    return _torch().cuda.current_stream(t.device).cuda_stream


def block_mean(x, nblk: int | None = None, out=None):
    """Per-block token means (fp32): xbar[h][b] = mean of x[h][128 b : 128 b + 128]."""
    torch = _torch()
    _require_cuda(x)
    H, T, d = x.shape
    nblk = T // VELOX_BLOCK if nblk is None else nblk
    if not 0 <= nblk <= T // VELOX_BLOCK:
        raise ValueError(f"nblk={nblk} blocks do not fit in x's {T} token rows")
    if out is None:
        out = torch.empty(H, nblk, d, dtype=torch.float32, device=x.device)
    _require_cuda(out)
    if out.dtype != torch.float32:
        raise TypeError("out must be float32")
    if out.dim() == 3 and (out.shape[0] != H or out.shape[1] < nblk or out.shape[2] != d):
        raise ValueError(f"out must be [H][>=nblk][d] = [{H}][>={nblk}][{d}] (got {tuple(out.shape)})")
    _rows(out.view(H, nblk, d) if out.dim() != 3 else out, "out")
    lib = _lib.load()
    _lib.check(lib.velox_block_mean(x.data_ptr(), _dtype_code(x), _rows(x, "x"), H, nblk, d,
                                    out.data_ptr(), out.stride(0), _stream(x)))
    return out


def _kbar_rows(kbar, H, M, d):
    """kbar must hold M key means of q's head dim for each of q's heads."""
    if kbar.dim() != 3 or kbar.shape[0] != H or kbar.shape[1] < M or kbar.shape[2] != d:
        raise ValueError(f"kbar must be [H][>=M][d] = [{H}][>={M}][{d}] (got {tuple(kbar.shape)})")


def route_scores(q, kbar, M: int, scale: float | None = None, out=None):
    """Block importance p [H][N][M] = softmax over history of scale * qbar . kbar."""
    torch = _torch()
    _require_cuda(q, kbar)
    H, NT, d = q.shape
    N = NT // VELOX_BLOCK
    if kbar.dtype != torch.float32:
        raise TypeError("kbar must be float32")
    _kbar_rows(kbar, H, M, d)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    if out is None:
        out = torch.empty(H, N, M, dtype=torch.float32, device=q.device)
    _require_cuda(out)
    _contig(out, "p")
    if out.dtype != torch.float32 or out.numel() != H * N * M:
        raise ValueError(f"p must be float32 [H][N][M] = [{H}][{N}][{M}] (got {tuple(out.shape)})")
    lib = _lib.load()
    _lib.check(lib.velox_route_scores(q.data_ptr(), _dtype_code(q), _rows(q, "q"), kbar.data_ptr(),
                                      _rows(kbar, "kbar"), H, N, M, d, ctypes.c_float(scale),
                                      out.data_ptr(), _stream(q)))
    return out


def route_scores_shared(q, kbar, M: int, scale: float | None = None, logits=None, out=None):
    """Head-shared importance p [1][N][M] (softmax of the head-mean logits).

    `logits` [H][N][M] fp32 is the per-head workspace (allocated if None).
    """
    torch = _torch()
    _require_cuda(q, kbar)
    H, NT, d = q.shape
    N = NT // VELOX_BLOCK
    if kbar.dtype != torch.float32:
        raise TypeError("kbar must be float32")
    _kbar_rows(kbar, H, M, d)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    if logits is None:
        logits = torch.empty(H, N, M, dtype=torch.float32, device=q.device)
    if out is None:
        out = torch.empty(1, N, M, dtype=torch.float32, device=q.device)
    _require_cuda(logits, out)
    _contig(logits, "logits")
    _contig(out, "p")
    if logits.numel() < H * N * M or out.numel() < N * M:
        raise ValueError("logits must hold H*N*M and out N*M floats")
    lib = _lib.load()
    _lib.check(lib.velox_route_scores_shared(q.data_ptr(), _dtype_code(q), _rows(q, "q"),
                                             kbar.data_ptr(), _rows(kbar, "kbar"), H, N, M, d,
                                             ctypes.c_float(scale), logits.data_ptr(),
                                             out.data_ptr(), _stream(q)))
    return out


def route_bound(params, M: int, n_ref: int | None = None) -> int:
    """Smallest route length L that always suffices (n_ref: number of
    reference ids, default len(params.ref_ids))."""
    kmax = max(int(params.K_cov), int(params.K_unc), int(params.n_prev))
    n_ref = len(tuple(params.ref_ids)) if n_ref is None else int(n_ref)
    bound = kmax + 26 * int(params.neigh26) + n_ref
    return max(1, min(M, bound))


def route_select(p, g, rho, coord, params, L: int | None = None, route_ids=None,
                 route_len=None, ref_ids=None, status=None):
    """Routes (route_ids [H][N][L] int32, route_len [H][N] int32).

    `params` is any object with the attributes tau, g_ref, lam, eta_cov,
    theta_cov, theta_unc, K_cov, K_unc, n_prev, neigh26 and ref_ids (a sequence
    of history ids), and optionally mode (0 fused, 1 model only, 2 geometry
    only; default 0).
    ref_ids: optional int32 device tensor of reference-frame ids; when given it
    replaces params.ref_ids and nothing is allocated or copied per call (the
    form a captured HIP graph needs). Without it, a non-empty params.ref_ids is
    copied to the device on every call.
    status: optional int32 device tensor of 2 elements that receives the
    input report (rows whose p or g break the fixed-point preconditions, and
    the smallest such row h * N + i, or H * N).
    """
    torch = _torch()
    _require_cuda(p, g, rho)
    H, N, M = p.shape
    for t, name in ((p, "p"), (g, "g"), (rho, "rho")):
        _contig(t, name)
        if t.dtype != torch.float32:
            raise TypeError(f"{name} must be float32")
    if tuple(g.shape) != (N, M) or rho.numel() != N:
        raise ValueError(f"g must be [N][M] = [{N}][{M}] and rho [N] (got {tuple(g.shape)}, "
                         f"{tuple(rho.shape)})")
    if coord is not None:
        _require_cuda(coord)
        _contig(coord, "coord")
        if coord.dtype != torch.int32:
            raise TypeError("coord must be int32")
        if coord.numel() < 3 * (M + N) or coord.numel() % 3:
            raise ValueError(f"coord must be [>=M+N][3] = [>={M + N}][3] (got {tuple(coord.shape)})")
    L = route_bound(params, M, None if ref_ids is None else ref_ids.numel()) if L is None else L
    if route_ids is None:
        route_ids = torch.empty(H, N, L, dtype=torch.int32, device=p.device)
    if route_len is None:
        route_len = torch.empty(H, N, dtype=torch.int32, device=p.device)
    _require_cuda(route_ids, route_len)
    _contig(route_ids, "route_ids")
    _contig(route_len, "route_len")
    if route_ids.dtype != torch.int32 or route_len.dtype != torch.int32:
        raise TypeError("route_ids and route_len must be int32")
    if route_ids.numel() != H * N * L or route_len.numel() != H * N:
        raise ValueError(f"route_ids must be [H][N][L] = [{H}][{N}][{L}] and route_len [H][N]")
    ref_t = None
    if ref_ids is not None:
        _require_cuda(ref_ids)
        _contig(ref_ids, "ref_ids")
        if ref_ids.dtype != torch.int32:
            raise TypeError("ref_ids must be int32")
        n_ref = ref_ids.numel()
        ref_ptr = ref_ids.data_ptr() if n_ref else None
    else:
        ref = tuple(int(r) for r in params.ref_ids)
        ref_t = torch.tensor(ref, dtype=torch.int32, device=p.device) if ref else None
        n_ref = len(ref)
        ref_ptr = ref_t.data_ptr() if ref_t is not None else None
    st_ptr = None
    if status is not None:
        _require_cuda(status)
        _contig(status, "status")
        if status.dtype != torch.int32 or status.numel() < 2:
            raise ValueError("status must be an int32 device tensor of 2 elements")
        st_ptr = status.data_ptr()
    c = _lib.RouteParamsC(params.tau, params.g_ref, params.lam, params.eta_cov, params.theta_cov,
                          params.theta_unc, int(params.K_cov), int(params.K_unc),
                          int(params.n_prev), int(params.neigh26), ref_ptr, n_ref,
                          int(getattr(params, "mode", 0)), st_ptr)
    lib = _lib.load()
    _lib.check(lib.velox_route_select(p.data_ptr(), g.data_ptr(), rho.data_ptr(),
                                      coord.data_ptr() if coord is not None else None, H, N, M,
                                      ctypes.byref(c), L, route_ids.data_ptr(),
                                      route_len.data_ptr(), _stream(p)))
    if ref_t is not None:
        ref_t.record_stream(torch.cuda.current_stream(p.device))
    return route_ids, route_len


def _attn_out(q, out, lse, want_lse):
    torch = _torch()
    H, NT, d = q.shape
    if out is None:
        out = torch.empty(H, NT, d, dtype=q.dtype, device=q.device)
    _require_cuda(out)
    _contig(out, "out")
    if out.dtype != q.dtype or out.numel() != H * NT * d:
        raise ValueError(f"out must be [H][N*128][d] = [{H}][{NT}][{d}] of q's dtype")
    if lse is None and want_lse:
        lse = torch.empty(H, NT, dtype=torch.float32, device=q.device)
    if lse is not None:
        _require_cuda(lse)
        _contig(lse, "lse")
        if lse.dtype != torch.float32 or lse.numel() != H * NT:
            raise ValueError(f"lse must be float32 [H][N*128] = [{H}][{NT}]")
    return out, lse


def _kv_rows(q, k, v, M):
    """k and v must hold the M history blocks and the N current ones."""
    H, NT, d = q.shape
    if k.shape[0] != H or k.shape[2] != d or k.shape[1] < M * VELOX_BLOCK + NT:
        raise ValueError(f"k and v must be [H][>=(M+N)*128][d] = [{H}][>={M * VELOX_BLOCK + NT}][{d}] "
                         f"(got {tuple(k.shape)})")


def check_routes(route_ids, route_len, M: int):
    """(number of invalid rows, smallest invalid row or -1): rows whose length
    is outside [0, L] or whose ids are not strictly ascending in [0, M)."""
    torch = _torch()
    _require_cuda(route_ids, route_len)
    _contig(route_ids, "route_ids")
    _contig(route_len, "route_len")
    if route_ids.dtype != torch.int32 or route_len.dtype != torch.int32:
        raise TypeError("route_ids and route_len must be int32")
    rows = route_len.numel()
    L = route_ids.shape[-1]
    if route_ids.numel() != rows * L:
        raise ValueError("route_ids must hold route_len.numel() rows of L ids")
    bad = torch.empty(2, dtype=torch.int32, device=route_ids.device)
    lib = _lib.load()
    _lib.check(lib.velox_route_check(route_ids.data_ptr(), route_len.data_ptr(), rows, M, L,
                                     bad.data_ptr(), _stream(route_ids)))
    n, first = (int(x) for x in bad.cpu().tolist())
    return n, (first if n > 0 else -1)


def attn_workspace(q, L: int):
    """A device workspace for sparse_attn (its unit schedule; uint8 tensor)."""
    torch = _torch()
    H, NT, d = q.shape
    nbytes = _lib.load().velox_sparse_attn_workspace_size(H, NT // VELOX_BLOCK, int(L), d)
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=q.device)


def split_workspace(q, n_split: int):
    """A device workspace for the split-row attention calls (uint8 tensor)."""
    torch = _torch()
    H, NT, _ = q.shape
    nbytes = _lib.load().velox_attn_split_workspace_size(H, NT // VELOX_BLOCK, int(n_split))
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=q.device)


def _split_args(q, n_split, workspace):
    if n_split == 1:
        return None, 0
    if workspace is None:
        workspace = split_workspace(q, n_split)
    _require_cuda(workspace)
    return workspace, workspace.numel() * workspace.element_size()


def sparse_attn(q, k, v, route_ids, route_len, M: int, include_current: bool = True,
                scale: float | None = None, out=None, lse=None, want_lse: bool = False,
                n_split: int = 1, workspace=None):
    """Attention of each query block over its routed history tiles (+ current chunk).

    route_ids [H][N][L] / route_len [H][N] give one route per head; [N][L] / [N]
    (or [1][N][L] / [1][N]) one route per query block shared by all heads.
    n_split > 1 cuts rows' tiles into ranges (per-head routes only): each pair
    of rows into at most n_split, as many as one round of an XCD's CUs holds
    (none when an XCD has more pairs than CUs); `workspace` is then a device
    buffer of split_workspace(q, n_split)'s size (allocated here when None). With per-head routes and n_split = 1 the
    workspace holds the call's unit schedule: attn_workspace(q, L) bytes
    (allocated here when None).
    """
    _require_cuda(q, k, v, route_ids, route_len)
    H, NT, d = q.shape
    N = NT // VELOX_BLOCK
    if k.dtype != q.dtype or v.dtype != q.dtype or k.stride() != v.stride():
        raise ValueError("q, k, v must share a dtype and k, v a layout")
    _contig(route_ids, "route_ids")
    _contig(route_len, "route_len")
    if route_ids.dtype != _torch().int32 or route_len.dtype != _torch().int32:
        raise TypeError("route_ids and route_len must be int32")
    _kv_rows(q, k, v, M)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    out, lse = _attn_out(q, out, lse, want_lse)
    lib = _lib.load()
    if route_len.numel() not in (N, H * N) or route_ids.numel() != route_len.numel() * route_ids.shape[-1]:
        raise ValueError("routes must be [H][N][L] + [H][N] (per head) or [N][L] + [N] (shared)")
    shared = route_len.numel() != H * N
    if n_split != 1:
        if shared:
            raise ValueError("split rows take per-head routes")
        ws, ws_bytes = _split_args(q, n_split, workspace)
        _lib.check(lib.velox_sparse_attn_split(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), _dtype_code(q), _rows(q, "q"), _rows(k, "k"),
            H, N, M, d, ctypes.c_float(scale), route_ids.data_ptr(), route_len.data_ptr(),
            route_ids.shape[-1], 1 if include_current else 0, int(n_split), ws.data_ptr(), ws_bytes,
            out.data_ptr(), lse.data_ptr() if lse is not None else None, _stream(q)))
        return (out, lse) if want_lse or lse is not None else out
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), _dtype_code(q), _rows(q, "q"),
            _rows(k, "k"), H, N, M, d, ctypes.c_float(scale), route_ids.data_ptr(),
            route_len.data_ptr(), route_ids.shape[-1], 1 if include_current else 0,
            out.data_ptr(), lse.data_ptr() if lse is not None else None)
    if shared:
        _lib.check(lib.velox_sparse_attn_shared(*args, _stream(q)))
    else:
        if workspace is None:
            workspace = attn_workspace(q, route_ids.shape[-1])
        _require_cuda(workspace)
        need = lib.velox_sparse_attn_workspace_size(H, N, route_ids.shape[-1], d)
        if workspace.numel() * workspace.element_size() < need:
            raise ValueError(f"workspace must hold {need} bytes")
        _lib.check(lib.velox_sparse_attn(*args, workspace.data_ptr(), _stream(q)))
    return (out, lse) if want_lse or lse is not None else out


def dense_attn(q, k, v, M: int, scale: float | None = None, out=None, lse=None,
               want_lse: bool = False, n_split: int = 1, workspace=None):
    """Dense baseline: every history tile and every current-chunk tile
    (n_split / workspace as for sparse_attn)."""
    _require_cuda(q, k, v)
    H, NT, d = q.shape
    N = NT // VELOX_BLOCK
    if k.dtype != q.dtype or v.dtype != q.dtype or k.stride() != v.stride():
        raise ValueError("q, k, v must share a dtype and k, v a layout")
    _kv_rows(q, k, v, M)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    out, lse = _attn_out(q, out, lse, want_lse)
    lib = _lib.load()
    if n_split != 1:
        ws, ws_bytes = _split_args(q, n_split, workspace)
        _lib.check(lib.velox_dense_attn_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), _dtype_code(q),
                                              _rows(q, "q"), _rows(k, "k"), H, N, M, d,
                                              ctypes.c_float(scale), int(n_split), ws.data_ptr(),
                                              ws_bytes, out.data_ptr(),
                                              lse.data_ptr() if lse is not None else None, _stream(q)))
        return (out, lse) if want_lse or lse is not None else out
    _lib.check(lib.velox_dense_attn(q.data_ptr(), k.data_ptr(), v.data_ptr(), _dtype_code(q),
                                    _rows(q, "q"), _rows(k, "k"), H, N, M, d,
                                    ctypes.c_float(scale), out.data_ptr(),
                                    lse.data_ptr() if lse is not None else None, _stream(q)))
    return (out, lse) if want_lse or lse is not None else out


def _obb(t, name):
    torch = _torch()
    if t.dtype != torch.float32 or t.dim() != 2 or t.shape[1] != _lib.VELOX_OBB_WORDS:
        raise ValueError(f"{name} must be float32 [n][{_lib.VELOX_OBB_WORDS}]")
    _contig(t, name)


def slab_overlap(q_obb, h_obb, lattice: int = 8, out=None):
    """g [N][M] fp32: lattice-approximated IoU of query and history slab boxes."""
    torch = _torch()
    _require_cuda(q_obb, h_obb)
    _obb(q_obb, "q_obb")
    _obb(h_obb, "h_obb")
    N, M = q_obb.shape[0], h_obb.shape[0]
    if out is None:
        out = torch.empty(N, M, dtype=torch.float32, device=q_obb.device)
    _require_cuda(out)
    _contig(out, "out")
    if out.shape != (N, M) or out.dtype != torch.float32:
        raise ValueError("out must be float32 [N][M]")
    lib = _lib.load()
    _lib.check(lib.velox_slab_overlap(q_obb.data_ptr(), h_obb.data_ptr(), N, M, lattice,
                                      out.data_ptr(), _stream(q_obb)))
    return out


def slab_coverage(q_pts, h_obb, rho=None, token_mask=None):
    """(rho [N] fp32, token_mask [N][4] int32 bit masks) of query token points."""
    torch = _torch()
    _require_cuda(q_pts, h_obb)
    _obb(h_obb, "h_obb")
    if q_pts.dtype != torch.float32 or q_pts.dim() != 3 or q_pts.shape[1:] != (VELOX_BLOCK, 3):
        raise ValueError("q_pts must be float32 [N][128][3]")
    _contig(q_pts, "q_pts")
    N, M = q_pts.shape[0], h_obb.shape[0]
    if rho is None:
        rho = torch.empty(N, dtype=torch.float32, device=q_pts.device)
    if token_mask is None:
        token_mask = torch.empty(N, 4, dtype=torch.int32, device=q_pts.device)
    _require_cuda(rho, token_mask)
    _contig(rho, "rho")
    _contig(token_mask, "token_mask")
    if rho.shape != (N,) or token_mask.shape != (N, 4) or token_mask.element_size() != 4:
        raise ValueError("rho must be [N] and token_mask [N][4] of 32-bit words")
    lib = _lib.load()
    _lib.check(lib.velox_slab_coverage(q_pts.data_ptr(), h_obb.data_ptr(), N, M,
                                       token_mask.data_ptr(), rho.data_ptr(), _stream(q_pts)))
    return rho, token_mask


def gilbert_curve(width: int, height: int):
    """numpy int32 [width*height]: y*width + x of the k-th cell along the curve."""
    import numpy as np
    cells = np.empty(width * height, dtype=np.int32)
    lib = _lib.load()
    _lib.check(lib.velox_gilbert_curve(width, height, cells.ctypes.data))
    return cells


def kv_append(k_new, v_new, T: int, height: int, width: int, chunk_index: int, cells,
              k_cache, v_cache, token_offset: int, kbar=None):
    """Write one chunk (THW-linear [H][T*height*width][d]) into the caches in
    global order at token_offset; refresh kbar for its blocks when given."""
    torch = _torch()
    _require_cuda(k_new, v_new, cells, k_cache, v_cache, kbar)
    if k_new.dtype != v_new.dtype or k_new.dtype != k_cache.dtype or k_cache.dtype != v_cache.dtype:
        raise ValueError("k_new, v_new and the caches must share one dtype")
    if k_new.shape != v_new.shape or k_cache.shape != v_cache.shape or k_cache.stride() != v_cache.stride():
        raise ValueError("k/v shapes or strides differ")
    if k_new.stride() != v_new.stride():
        raise ValueError("k_new and v_new strides differ")
    if cells.dtype != torch.int32 or cells.numel() != height * width:
        raise ValueError("cells must be int32 [height*width]")
    _contig(cells, "cells")
    H, _, d = k_new.shape
    n_tok = T * height * width
    if k_new.shape[1] < n_tok:
        raise ValueError(f"k_new and v_new must hold T*height*width = {n_tok} token rows per head")
    if (k_cache.dim() != 3 or k_cache.shape[0] != H or k_cache.shape[2] != d
            or k_cache.shape[1] < token_offset + n_tok):
        raise ValueError(f"k_cache and v_cache must be [H][>=token_offset+{n_tok}][d] = "
                         f"[{H}][>={token_offset + n_tok}][{d}] (got {tuple(k_cache.shape)})")
    kb_ptr, kb_ld = 0, 0
    if kbar is not None:
        if kbar.dtype != torch.float32:
            raise ValueError("kbar must be float32")
        nb_end = (token_offset + n_tok + VELOX_BLOCK - 1) // VELOX_BLOCK
        if kbar.dim() != 3 or kbar.shape[0] != H or kbar.shape[2] != d or kbar.shape[1] < nb_end:
            raise ValueError(f"kbar must be [H][>={nb_end}][d] (got {tuple(kbar.shape)})")
        kb_ptr, kb_ld = kbar.data_ptr(), _rows(kbar, "kbar")
    lib = _lib.load()
    _lib.check(lib.velox_kv_append(k_new.data_ptr(), v_new.data_ptr(), _dtype_code(k_new),
                                   _rows(k_new, "k_new"), H, T, height, width, d, chunk_index,
                                   cells.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                   _rows(k_cache, "k_cache"), token_offset, kb_ptr or None,
                                   kb_ld, _stream(k_new)))


def _f32c(t, name, shape_tail=None):
    torch = _torch()
    if t.dtype != torch.float32:
        raise ValueError(f"{name} must be float32")
    if shape_tail is not None and tuple(t.shape[1:]) != tuple(shape_tail):
        raise ValueError(f"{name} must be [n]{list(shape_tail)}")
    _contig(t, name)


def _i32c(t, name, shape_tail=None):
    torch = _torch()
    if t.dtype != torch.int32:
        raise ValueError(f"{name} must be int32")
    if shape_tail is not None and tuple(t.shape[1:]) != tuple(shape_tail):
        raise ValueError(f"{name} must be [n]{list(shape_tail)}")
    _contig(t, name)


def slab_table(cells, depth, cams, cam_of_block, f: float, cx: float, cy: float, n_min: int = 8):
    """(slabs [nblk][8], boxes [nblk][16]) of blocks of 128 (cell, depth) samples."""
    torch = _torch()
    _require_cuda(cells, depth, cams, cam_of_block)
    _i32c(cells, "cells", (2,))
    _f32c(depth, "depth")
    _f32c(cams, "cams", (12,))
    _i32c(cam_of_block, "cam_of_block")
    nblk = depth.numel() // VELOX_BLOCK
    if depth.numel() != nblk * VELOX_BLOCK or cells.shape[0] != depth.numel() or cam_of_block.numel() != nblk:
        raise ValueError("need 128 samples per block, one cell per sample, one camera per block")
    slabs = torch.empty(nblk, 8, dtype=torch.float32, device=depth.device)
    boxes = torch.empty(nblk, 16, dtype=torch.float32, device=depth.device)
    lib = _lib.load()
    _lib.check(lib.velox_slab_table(cells.data_ptr(), depth.data_ptr(), cams.data_ptr(),
                                    cam_of_block.data_ptr(), cams.shape[0], nblk, f, cx, cy, n_min,
                                    slabs.data_ptr(), boxes.data_ptr(), _stream(depth)))
    return slabs, boxes


def multiwarp(src_depth, src_cams, src_size, src_pinhole, tgt_cam, size, pinhole, k_warp: int = 2,
              workspace=None):
    """(zq [h*w] fp32, chosen [h*w] int32) by recency-priority multiwarp.

    src_depth [K][src_h*src_w] depth frames with cameras src_cams [K][12],
    src_size = (src_w, src_h), src_pinhole = (f, cx, cy) in pixels; the target
    is a size = (w, h) token grid of tgt_cam [12] with pinhole (f, cx, cy).
    """
    torch = _torch()
    _require_cuda(src_depth, src_cams, tgt_cam)
    _f32c(src_depth, "src_depth")
    _f32c(src_cams, "src_cams", (12,))
    _f32c(tgt_cam, "tgt_cam")
    K = src_cams.shape[0]
    (sw, sh), (w, h) = src_size, size
    if src_depth.numel() != K * sw * sh or tgt_cam.numel() != 12:
        raise ValueError("src_depth must be [K][src_h*src_w] and tgt_cam [12]")
    lib = _lib.load()
    need = lib.velox_multiwarp_workspace_size(K, sw, sh, w, h)
    if workspace is None:
        workspace = torch.empty(max(need, 4), dtype=torch.uint8, device=src_depth.device)
    _require_cuda(workspace)
    zq = torch.empty(w * h, dtype=torch.float32, device=src_depth.device)
    chosen = torch.empty(w * h, dtype=torch.int32, device=src_depth.device)
    _lib.check(lib.velox_multiwarp(src_depth.data_ptr(), src_cams.data_ptr(), K, sw, sh, *src_pinhole,
                                   tgt_cam.data_ptr(), *pinhole, w, h, k_warp, zq.data_ptr(),
                                   chosen.data_ptr(), workspace.data_ptr(),
                                   workspace.numel() * workspace.element_size(), _stream(src_depth)))
    return zq, chosen


def token_points(cells, zq, width: int, height: int, cam, f: float, cx: float, cy: float):
    """(depth [n] fp32, points [n][3] fp32) of tokens from the warped depth map."""
    torch = _torch()
    _require_cuda(cells, zq, cam)
    _i32c(cells, "cells", (2,))
    _f32c(zq, "zq")
    _f32c(cam, "cam")
    n = cells.shape[0]
    depth = torch.empty(n, dtype=torch.float32, device=cells.device)
    pts = torch.empty(n, 3, dtype=torch.float32, device=cells.device)
    lib = _lib.load()
    _lib.check(lib.velox_token_points(cells.data_ptr(), zq.data_ptr(), width, height, cam.data_ptr(), f, cx,
                                      cy, n, depth.data_ptr(), pts.data_ptr(), _stream(cells)))
    return depth, pts
