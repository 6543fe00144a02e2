"""ctypes view of libvelox.so (the C ABI declared in include/velox.h,
include/velox_geometry.h, include/velox_layout.h and include/velox_slabs.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libvelox.so")

VELOX_OK, VELOX_ERR_INVALID, VELOX_ERR_UNSUPPORTED, VELOX_ERR_LAUNCH = 0, 1, 2, 3
VELOX_F32, VELOX_BF16 = 0, 1
VELOX_BLOCK = 128
VELOX_MAX_HISTORY = 16384

EXPORTS = ("velox_last_error", "velox_version", "velox_block_mean", "velox_route_scores",
           "velox_route_select", "velox_sparse_attn", "velox_dense_attn",
           "velox_slab_overlap", "velox_slab_coverage", "velox_gilbert_curve",
           "velox_kv_append", "velox_route_scores_shared", "velox_sparse_attn_shared",
           "velox_slab_table", "velox_multiwarp_workspace_size", "velox_multiwarp",
           "velox_token_points", "velox_attn_split_workspace_size", "velox_sparse_attn_split",
           "velox_dense_attn_split", "velox_route_check", "velox_sparse_attn_workspace_size",
           "velox_sparse_attn_noalloc")
VELOX_ROUTE_FUSED, VELOX_ROUTE_MODEL_ONLY, VELOX_ROUTE_GEOMETRY_ONLY = 0, 1, 2
VELOX_OBB_WORDS = 16
VELOX_MAX_LATTICE = 16
VELOX_MAX_SPLIT = 16


class RouteParamsC(ctypes.Structure):
    """Mirror of velox_route_params_t."""
    _fields_ = [
        ("tau", ctypes.c_float), ("g_ref", ctypes.c_float), ("lambda_", ctypes.c_float),
        ("eta_cov", ctypes.c_float), ("theta_cov", ctypes.c_float), ("theta_unc", ctypes.c_float),
        ("K_cov", ctypes.c_int32), ("K_unc", ctypes.c_int32), ("n_prev", ctypes.c_int32),
        ("neigh26", ctypes.c_int32), ("ref_ids", ctypes.c_void_p), ("n_ref", ctypes.c_int32),
        ("mode", ctypes.c_int32), ("status", ctypes.c_void_p),
    ]


class VeloxError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"velox status {status}: {message}")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """The loaded library (built in place by geometry_routed_block_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m geometry_routed_block_amd.build` (there is no fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
    lib.velox_last_error.restype = ctypes.c_char_p
    lib.velox_last_error.argtypes = []
    lib.velox_version.restype = ctypes.c_int
    lib.velox_version.argtypes = []
    lib.velox_block_mean.restype = i32
    lib.velox_block_mean.argtypes = [vp, i32, i64, i32, i32, i32, vp, i64, vp]
    lib.velox_route_scores.restype = i32
    lib.velox_route_scores.argtypes = [vp, i32, i64, vp, i64, i32, i32, i32, i32, f32, vp, vp]
    lib.velox_route_select.restype = i32
    lib.velox_route_select.argtypes = [vp, vp, vp, vp, i32, i32, i32,
                                       ctypes.POINTER(RouteParamsC), i32, vp, vp, vp]
    lib.velox_sparse_attn.restype = i32
    lib.velox_sparse_attn.argtypes = [vp, vp, vp, i32, i64, i64, i32, i32, i32, i32, f32,
                                      vp, vp, i32, i32, vp, vp, vp, vp]
    lib.velox_sparse_attn_noalloc.restype = i32
    lib.velox_sparse_attn_noalloc.argtypes = [vp, vp, vp, i32, i64, i64, i32, i32, i32, i32, f32,
                                              vp, vp, i32, i32, vp, vp, vp]
    lib.velox_sparse_attn_workspace_size.restype = ctypes.c_size_t
    lib.velox_sparse_attn_workspace_size.argtypes = [i32, i32, i32, i32]
    lib.velox_slab_overlap.restype = i32
    lib.velox_slab_overlap.argtypes = [vp, vp, i32, i32, i32, vp, vp]
    lib.velox_slab_coverage.restype = i32
    lib.velox_slab_coverage.argtypes = [vp, vp, i32, i32, vp, vp, vp]
    lib.velox_gilbert_curve.restype = i32
    lib.velox_gilbert_curve.argtypes = [i32, i32, vp]
    lib.velox_kv_append.restype = i32
    lib.velox_kv_append.argtypes = [vp, vp, i32, i64, i32, i32, i32, i32, i32, i32, vp, vp, vp,
                                    i64, i64, vp, i64, vp]
    lib.velox_route_scores_shared.restype = i32
    lib.velox_route_scores_shared.argtypes = [vp, i32, i64, vp, i64, i32, i32, i32, i32, f32, vp, vp, vp]
    lib.velox_sparse_attn_shared.restype = i32
    lib.velox_sparse_attn_shared.argtypes = [vp, vp, vp, i32, i64, i64, i32, i32, i32, i32, f32,
                                             vp, vp, i32, i32, vp, vp, vp]
    lib.velox_slab_table.restype = i32
    lib.velox_slab_table.argtypes = [vp, vp, vp, vp, i32, i32, f32, f32, f32, i32, vp, vp, vp]
    lib.velox_multiwarp_workspace_size.restype = ctypes.c_size_t
    lib.velox_multiwarp_workspace_size.argtypes = [i32, i32, i32, i32, i32]
    lib.velox_multiwarp.restype = i32
    lib.velox_multiwarp.argtypes = [vp, vp, i32, i32, i32, f32, f32, f32, vp, f32, f32, f32, i32, i32,
                                    i32, vp, vp, vp, ctypes.c_size_t, vp]
    lib.velox_token_points.restype = i32
    lib.velox_token_points.argtypes = [vp, vp, i32, i32, vp, f32, f32, f32, i64, vp, vp, vp]
    lib.velox_dense_attn.restype = i32
    lib.velox_dense_attn.argtypes = [vp, vp, vp, i32, i64, i64, i32, i32, i32, i32, f32,
                                     vp, vp, vp]
    lib.velox_attn_split_workspace_size.restype = ctypes.c_size_t
    lib.velox_attn_split_workspace_size.argtypes = [i32, i32, i32]
    lib.velox_sparse_attn_split.restype = i32
    lib.velox_sparse_attn_split.argtypes = [vp, vp, vp, i32, i64, i64, i32, i32, i32, i32, f32,
                                            vp, vp, i32, i32, i32, vp, ctypes.c_size_t, vp, vp, vp]
    lib.velox_route_check.restype = i32
    lib.velox_route_check.argtypes = [vp, vp, i32, i32, i32, vp, vp]
    lib.velox_dense_attn_split.restype = i32
    lib.velox_dense_attn_split.argtypes = [vp, vp, vp, i32, i64, i64, i32, i32, i32, i32, f32,
                                           i32, vp, ctypes.c_size_t, vp, vp, vp]
    _lib = lib
    return lib


def check(status: int) -> None:
    if status != VELOX_OK:
        raise VeloxError(status, load().velox_last_error().decode())
