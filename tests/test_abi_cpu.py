"""The C-ABI library loads, exports every entry point its header declares, and
rejects invalid arguments on the host before any launch. No GPU needed: every
call below fails validation, so no device memory is ever touched."""

import ctypes
import os
import re

import pytest

from geometry_routed_block_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))

BAD = 0x1000  # a non-NULL pointer value that validation must reject before use


def _declared():
    text = "".join(open(h).read() for h in HEADERS)
    return sorted(set(re.findall(r"\b(velox_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    assert set(_declared()) == set(_lib.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    for name in _declared():
        assert hasattr(lib, name), name
    assert lib.velox_version() >= 100


def _status(fn, *args):
    return fn(*args)


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_block_mean_validation(lib):
    f = lib.velox_block_mean
    assert f(BAD, 0, 1 << 20, 1, 1, 96, BAD, 96, None) == _lib.VELOX_ERR_INVALID
    assert b"d must be 64 or 128" in lib.velox_last_error()
    assert f(BAD, 7, 1 << 20, 1, 1, 64, BAD, 64, None) == _lib.VELOX_ERR_INVALID
    assert f(None, 0, 1 << 20, 1, 1, 64, BAD, 64, None) == _lib.VELOX_ERR_INVALID
    assert f(BAD, 0, 10, 1, 1, 64, BAD, 64, None) == _lib.VELOX_ERR_INVALID    # ld too small
    assert f(None, 0, 0, 1, 0, 64, None, 0, None) == _lib.VELOX_OK             # nblk = 0: no-op


def test_route_scores_validation(lib):
    f = lib.velox_route_scores
    ok_ld = 4 * 128 * 64
    assert f(BAD, 1, ok_ld, BAD, 64 * 16, 0, 4, 16, 64, ctypes.c_float(0.125), BAD, None) == _lib.VELOX_ERR_INVALID
    assert f(BAD, 1, ok_ld, BAD, 64 * 16, 2, 4, -1, 64, ctypes.c_float(0.125), BAD, None) == _lib.VELOX_ERR_INVALID
    assert f(BAD, 1, ok_ld, BAD, 64 * 16, 2, 4, 20000, 64, ctypes.c_float(0.125), BAD, None) == _lib.VELOX_ERR_UNSUPPORTED
    assert f(BAD, 1, ok_ld, BAD, 10, 2, 4, 16, 64, ctypes.c_float(0.125), BAD, None) == _lib.VELOX_ERR_INVALID
    assert f(BAD, 1, ok_ld, BAD, 64 * 16, 2, 4, 16, 64, ctypes.c_float(float("nan")), BAD, None) == _lib.VELOX_ERR_INVALID
    # M = 0 writes nothing and launches nothing
    assert f(BAD, 1, ok_ld, BAD, 0, 2, 4, 0, 64, ctypes.c_float(0.125), BAD, None) == _lib.VELOX_OK


def _params(**kw):
    base = dict(tau=0.1, g_ref=0.2, lambda_=2.0, eta_cov=0.9, theta_cov=1.0, theta_unc=0.9,
                K_cov=80, K_unc=150, n_prev=0, neigh26=0, ref_ids=None, n_ref=0)
    base.update(kw)
    return _lib.RouteParamsC(**base)


def test_route_select_validation(lib):
    f = lib.velox_route_select

    def call(prm, L=150, M=200, coord=BAD):
        return f(BAD, BAD, BAD, coord, 2, 4, M, ctypes.byref(prm), L, BAD, BAD, None)

    assert f(BAD, BAD, BAD, BAD, 2, 4, 200, None, 150, BAD, BAD, None) == _lib.VELOX_ERR_INVALID
    assert call(_params(), L=149) == _lib.VELOX_ERR_INVALID                 # L below the bound
    assert b"route bound" in lib.velox_last_error()
    assert call(_params(neigh26=1), L=150) == _lib.VELOX_ERR_INVALID       # needs 176
    assert call(_params(neigh26=1), L=176, coord=None) == _lib.VELOX_ERR_INVALID
    assert call(_params(g_ref=0.0)) == _lib.VELOX_ERR_INVALID
    assert call(_params(lambda_=15.0)) == _lib.VELOX_ERR_INVALID
    assert call(_params(theta_unc=0.0)) == _lib.VELOX_ERR_INVALID
    assert call(_params(n_prev=201)) == _lib.VELOX_ERR_INVALID
    assert call(_params(K_cov=-1)) == _lib.VELOX_ERR_INVALID
    assert call(_params(n_ref=2)) == _lib.VELOX_ERR_INVALID                # NULL ref_ids
    assert call(_params(), M=20000) == _lib.VELOX_ERR_UNSUPPORTED


def test_attention_validation(lib):
    sp, de = lib.velox_sparse_attn, lib.velox_dense_attn
    H, N, M, d = 2, 4, 16, 64
    ldq, ldkv = N * 128 * d, (M + N) * 128 * d
    s = ctypes.c_float(0.125)
    A = 0x10000  # aligned fake pointer
    assert sp(A, A, A, 1, ldq, ldkv, H, N, M, 80, s, A, A, 16, 1, A, None, None, None) == _lib.VELOX_ERR_INVALID
    assert sp(A, A, A, 1, ldq, ldkv - 1, H, N, M, d, s, A, A, 16, 1, A, None, None, None) == _lib.VELOX_ERR_INVALID
    assert sp(A, A, A, 1, ldq, ldkv, H, N, M, d, s, None, A, 16, 1, A, None, None, None) == _lib.VELOX_ERR_INVALID
    assert sp(A, A, A, 1, ldq, ldkv, H, N, M, d, s, A, A, 0, 1, A, None, None, None) == _lib.VELOX_ERR_INVALID
    assert sp(A, A, A, 1, ldq, ldkv, H, N, M, d, s, A, A, 16, 2, A, None, None, None) == _lib.VELOX_ERR_INVALID
    assert sp(A + 2, A, A, 1, ldq, ldkv, H, N, M, d, s, A, A, 16, 1, A, None, None, None) == _lib.VELOX_ERR_INVALID
    assert sp(A, A, A, 1, ldq, ldkv, H, N, M, d, s, A, A, 16, 1, A, None, A + 8, None) == _lib.VELOX_ERR_INVALID
    assert de(A, A, A, 1, ldq, ldkv, H, N, M, d, ctypes.c_float(-1.0), A, None, None) == _lib.VELOX_ERR_INVALID
    assert de(A, A, A, 1, ldq, ldkv, 0, N, M, d, s, A, None, None) == _lib.VELOX_ERR_INVALID
    assert de(None, A, A, 1, ldq, ldkv, H, N, M, d, s, A, None, None) == _lib.VELOX_ERR_INVALID


def test_noalloc_attention_rejects_oversized_calls(lib):
    """The no-allocation entry point checks its fixed scratch limit on the host
    (nothing launched): H * ceil(N / 2) units of 16 bytes must fit."""
    na = lib.velox_sparse_attn_noalloc
    d, M, s, A = 128, 16, ctypes.c_float(0.125), 0x10000
    for H, N, ok in ((1, 131073, False), (2, 65537, False), (1, 131072, True)):
        if ok:
            continue   # a call within the limit would launch: GPU tests cover it
        ldq, ldkv = N * 128 * d, (M + N) * 128 * d
        assert na(A, A, A, 1, ldq, ldkv, H, N, M, d, s, A, A, 16, 1, A, None, None) == \
            _lib.VELOX_ERR_UNSUPPORTED
        assert b"no-allocation" in lib.velox_last_error()
    H, N = 2, 4
    ldq, ldkv = N * 128 * d, (M + N) * 128 * d
    assert na(A, A, A, 1, ldq, ldkv, H, N, M, d, s, None, A, 16, 1, A, None, None) == _lib.VELOX_ERR_INVALID


def test_split_attention_validation(lib):
    sp, de = lib.velox_sparse_attn_split, lib.velox_dense_attn_split
    H, N, M, d = 2, 4, 16, 128
    ldq, ldkv = N * 128 * d, (M + N) * 128 * d
    s = ctypes.c_float(0.125)
    A = 0x10000  # aligned fake pointer
    need = lib.velox_attn_split_workspace_size(H, N, 3)
    # partial outputs, then (routed calls) a unit plan of ceil(pairs / 8) * n_split
    # slots on each of the 8 XCDs
    assert need == 3 * H * N * 128 * 130 * 4 + 8 * ((H * ((N + 1) // 2) + 7) // 8) * 3 * 16
    assert lib.velox_sparse_attn_workspace_size(H, N, 16, d) == H * ((N + 1) // 2) * 16
    assert lib.velox_sparse_attn_workspace_size(H, 5, 16, d) == H * 3 * 16
    assert lib.velox_sparse_attn_workspace_size(0, N, 16, d) == 0
    assert lib.velox_attn_split_workspace_size(0, N, 3) == 0
    bad = [
        (0, A, need),                                 # n_split out of range
        (_lib.VELOX_MAX_SPLIT + 1, A, 1 << 40),
        (3, None, need),                              # no workspace
        (3, A, need - 1),                             # workspace too small
        (3, A + 4, need),                             # misaligned workspace
    ]
    for n_split, ws, nbytes in bad:
        assert sp(A, A, A, 1, ldq, ldkv, H, N, M, d, s, A, A, 16, 1, n_split, ws, nbytes, A, None,
                  None) == _lib.VELOX_ERR_INVALID
        assert de(A, A, A, 1, ldq, ldkv, H, N, M, d, s, n_split, ws, nbytes, A, None,
                  None) == _lib.VELOX_ERR_INVALID
    assert "workspace" in lib.velox_last_error().decode() or "n_split" in lib.velox_last_error().decode()


def test_route_check_validation(lib):
    A = 0x10000
    assert lib.velox_route_check(A, A, 4, 10, 8, None, None) == _lib.VELOX_ERR_INVALID
    assert lib.velox_route_check(None, A, 4, 10, 8, A, None) == _lib.VELOX_ERR_INVALID
    assert lib.velox_route_check(A, A, 4, 10, 0, A, None) == _lib.VELOX_ERR_INVALID
    assert lib.velox_route_check(A, A, -1, 10, 8, A, None) == _lib.VELOX_ERR_INVALID


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        _lib.load()


def test_geometry_validation(lib):
    ov, cv = lib.velox_slab_overlap, lib.velox_slab_coverage
    assert ov(BAD, BAD, 4, 16, 0, BAD, None) == _lib.VELOX_ERR_INVALID          # lattice 0
    assert b"lattice" in lib.velox_last_error()
    assert ov(BAD, BAD, 4, 16, 17, BAD, None) == _lib.VELOX_ERR_INVALID         # lattice 17
    assert ov(BAD, BAD, -1, 16, 8, BAD, None) == _lib.VELOX_ERR_INVALID
    assert ov(BAD, BAD, 70000, 16, 8, BAD, None) == _lib.VELOX_ERR_INVALID
    assert ov(None, BAD, 4, 16, 8, BAD, None) == _lib.VELOX_ERR_INVALID
    assert ov(None, None, 0, 16, 8, None, None) == _lib.VELOX_OK                # N = 0: no-op
    assert ov(None, None, 4, 0, 8, None, None) == _lib.VELOX_OK                 # M = 0: no-op
    assert cv(BAD, BAD, 4, 16, None, BAD, None) == _lib.VELOX_ERR_INVALID
    assert cv(None, BAD, 4, 16, BAD, BAD, None) == _lib.VELOX_ERR_INVALID
    assert cv(BAD, BAD, 4, -2, BAD, BAD, None) == _lib.VELOX_ERR_INVALID
    assert cv(None, None, 0, 5, None, None, None) == _lib.VELOX_OK


def test_gilbert_curve_matches_the_oracle_on_the_host(lib):
    # the curve is host code in the library: a full parity check without a GPU
    import numpy as np
    import geometry_routed_block_amd as velox
    from oracle import layout
    for w, h in [(1, 1), (2, 2), (9, 4), (4, 9), (52, 29), (29, 52), (48, 32), (16, 16), (13, 11),
                 (1, 7), (7, 1), (3, 5), (64, 64), (100, 3)]:
        got = velox.gilbert_curve(w, h)
        ref = [y * w + x for x, y in layout.gilbert_curve(w, h)]
        assert got.tolist() == ref, (w, h)


def test_layout_validation(lib):
    import numpy as np
    cells = np.empty(4, np.int32)
    assert lib.velox_gilbert_curve(0, 4, cells.ctypes.data) == _lib.VELOX_ERR_INVALID
    assert lib.velox_gilbert_curve(1 << 13, 1 << 12, cells.ctypes.data) == _lib.VELOX_ERR_INVALID
    assert lib.velox_gilbert_curve(2, 2, None) == _lib.VELOX_ERR_INVALID
    f = lib.velox_kv_append
    ld = 4608 * 128
    args = dict(kn=BAD, vn=BAD, dt=1, ldn=ld, H=2, T=3, hh=32, ww=48, d=128, ci=0, cells=BAD,
                kc=BAD, vc=BAD, ldkv=ld * 2, off=4608, kb=None, ldkb=0)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["kn"], a["vn"], a["dt"], a["ldn"], a["H"], a["T"], a["hh"], a["ww"], a["d"], a["ci"],
                 a["cells"], a["kc"], a["vc"], a["ldkv"], a["off"], a["kb"], a["ldkb"], None)
    assert call(T=1, hh=29, ww=52) == _lib.VELOX_ERR_UNSUPPORTED      # 1508 tokens: not whole blocks
    assert call(off=100) == _lib.VELOX_ERR_INVALID                     # unaligned offset
    assert call(d=96) == _lib.VELOX_ERR_INVALID
    assert call(ldkv=ld) == _lib.VELOX_ERR_INVALID                     # cache too small for offset + chunk
    assert call(kb=BAD, ldkb=10) == _lib.VELOX_ERR_INVALID             # kbar stride too small
    assert call(cells=None) == _lib.VELOX_ERR_INVALID
    assert call(ci=-1) == _lib.VELOX_ERR_INVALID
    assert call(kn=BAD + 8) == _lib.VELOX_ERR_INVALID                  # misaligned


def test_slabs_validation(lib):
    st = lib.velox_slab_table
    assert st(BAD, BAD, BAD, BAD, 1, 4, 26.0, 26.0, 14.5, 0, BAD, BAD, None) == _lib.VELOX_ERR_INVALID   # n_min 0
    assert st(BAD, BAD, BAD, BAD, 0, 4, 26.0, 26.0, 14.5, 8, BAD, BAD, None) == _lib.VELOX_ERR_INVALID   # ncam 0
    assert st(BAD, BAD, BAD, BAD, 1, 4, -1.0, 26.0, 14.5, 8, BAD, BAD, None) == _lib.VELOX_ERR_INVALID  # f <= 0
    assert st(None, None, None, None, 1, 0, 26.0, 26.0, 14.5, 8, None, None, None) == _lib.VELOX_OK      # nblk 0
    assert lib.velox_multiwarp_workspace_size(60, 208, 116, 52, 29) >= 60 * 208 * 116 * 12
    mw = lib.velox_multiwarp
    need = lib.velox_multiwarp_workspace_size(2, 16, 8, 8, 4)

    def call(k_warp=2, nbytes=need, ws=BAD, src=BAD, sf=8.0):
        return mw(src, BAD, 2, 16, 8, sf, 8.0, 4.0, BAD, 4.0, 4.0, 2.0, 8, 4, k_warp, BAD, BAD, ws, nbytes, None)
    assert call(k_warp=0) == _lib.VELOX_ERR_INVALID
    assert call(nbytes=need - 4) == _lib.VELOX_ERR_INVALID
    assert call(ws=BAD + 2) == _lib.VELOX_ERR_INVALID
    assert call(src=None) == _lib.VELOX_ERR_INVALID
    assert call(sf=0.0) == _lib.VELOX_ERR_INVALID
    tp = lib.velox_token_points
    assert tp(None, None, 8, 4, None, 4.0, 4.0, 2.0, 0, None, None, None) == _lib.VELOX_OK
    assert tp(BAD, BAD, 0, 4, BAD, 4.0, 4.0, 2.0, 10, BAD, BAD, None) == _lib.VELOX_ERR_INVALID
