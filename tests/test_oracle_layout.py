"""Pins of the global-order oracle (Gilbert curve, chunk token ranks, KV
append): the classic Hilbert curve on power-of-two squares, path properties
on arbitrary rectangles, the chunk-seam property the pages state for their
toy case, and the append as an exact permutation. CPU only."""

import numpy as np
import pytest

from oracle import layout


def hilbert_xy(order: int, d: int):
    """Textbook Hilbert curve on a 2^order square: cell of distance d."""
    x = y = 0
    t = d
    s = 1
    while s < (1 << order):
        rx = 1 & (t // 2)
        ry = 1 & (t ^ rx)
        if ry == 0:
            if rx == 1:
                x, y = s - 1 - x, s - 1 - y
            x, y = y, x
        x += s * rx
        y += s * ry
        t //= 4
        s *= 2
    return x, y


SYMS = [lambda x, y, n: (x, y), lambda x, y, n: (y, x),
        lambda x, y, n: (n - 1 - x, y), lambda x, y, n: (x, n - 1 - y),
        lambda x, y, n: (n - 1 - x, n - 1 - y), lambda x, y, n: (n - 1 - y, x),
        lambda x, y, n: (y, n - 1 - x), lambda x, y, n: (n - 1 - y, n - 1 - x)]


@pytest.mark.parametrize("order", [1, 2, 3, 4, 5])
def test_power_of_two_square_is_the_hilbert_curve(order):
    n = 1 << order
    got = layout.gilbert_curve(n, n)
    ref = [hilbert_xy(order, d) for d in range(n * n)]
    assert any(got == [f(x, y, n) for x, y in ref] for f in SYMS)


@pytest.mark.parametrize("w,h", [(9, 4), (4, 9), (2, 2), (52, 29), (29, 52), (4, 3), (5, 5),
                                 (16, 16), (3, 7), (1, 6), (8, 1), (48, 32), (13, 11)])
def test_curve_is_a_bijection_with_neighbour_steps(w, h):
    cells = layout.gilbert_curve(w, h)
    assert len(cells) == w * h and len(set(cells)) == w * h
    assert all(0 <= x < w and 0 <= y < h for x, y in cells)
    assert cells[0] == (0, 0)
    assert cells[-1] == ((w - 1, 0) if w >= h else (0, h - 1))
    steps = [(abs(a[0] - b[0]), abs(a[1] - b[1])) for a, b in zip(cells, cells[1:])]
    assert all(max(s) == 1 for s in steps)                 # always a grid neighbour
    diag = sum(1 for s in steps if s == (1, 1))
    assert diag == 0 if (w % 2 == 0 or w < h) and (h % 2 == 0 or h < w) else diag <= 1


def test_rank_map_inverts_the_curve():
    r = layout.cell_rank_map(29, 52)
    cells = layout.gilbert_curve(52, 29)
    assert sorted(r.ravel().tolist()) == list(range(29 * 52))
    assert all(r[y, x] == k for k, (x, y) in enumerate(cells))


def _positions(T, height, width, chunk):
    """(t, h, w) of every chunk-local rank."""
    ranks = layout.chunk_token_ranks(T, height, width, chunk)
    pos = [None] * ranks.size
    for t in range(T):
        for h in range(height):
            for w in range(width):
                pos[ranks[(t * height + h) * width + w]] = (t + T * chunk, h, w)
    return pos


def test_pages_toy_seam_adjacency_needs_the_flip():
    # latent height 3, width 4, chunks of three frames ([project] Figures 6-7):
    # with the flip the last token of chunk 0 and the first token of chunk 1
    # are the same cell at consecutive frames; repeating the map unflipped
    # breaks that adjacency
    T, H, W = 3, 3, 4
    c0, c1 = _positions(T, H, W, 0), _positions(T, H, W, 1)
    last, first = c0[-1], c1[0]
    assert (first[1], first[2]) == (last[1], last[2]) and first[0] == last[0] + 1
    plain = layout.chunk_token_ranks(T, H, W, 0)
    first_plain = None
    for t in range(T):
        for h in range(H):
            for w in range(W):
                if plain[(t * H + h) * W + w] == 0:
                    first_plain = (t + T, h, w)
    assert max(abs(a - b) for a, b in zip(first_plain[1:], last[1:])) > 1


@pytest.mark.parametrize("T,H,W,chunk", [(3, 3, 4, 0), (3, 3, 4, 1), (3, 32, 48, 0), (3, 32, 48, 1),
                                         (1, 29, 52, 1), (4, 4, 9, 0)])
def test_chunk_ranks_are_a_permutation_with_local_steps(T, H, W, chunk):
    ranks = layout.chunk_token_ranks(T, H, W, chunk)
    assert sorted(ranks.tolist()) == list(range(T * H * W))
    pos = _positions(T, H, W, chunk)
    for a, b in zip(pos, pos[1:]):
        same_cell = a[1:] == b[1:] and b[0] == a[0] + 1
        next_cell = max(abs(a[1] - b[1]), abs(a[2] - b[2])) == 1 and b[0] == a[0] - (T - 1)
        assert same_cell or next_cell


def test_single_column_with_one_frame_is_the_identity():
    # a 1-wide latent walks straight down: global order = THW-linear order
    assert layout.chunk_token_ranks(1, 7, 1, 0).tolist() == list(range(7))
    assert layout.chunk_token_ranks(2, 1, 1, 0).tolist() == [0, 1]


def test_kv_append_places_every_token_once_and_means_its_blocks():
    rng = np.random.default_rng(0)
    H, T, Hl, Wl, d = 2, 2, 8, 16, 4          # 256 tokens = 2 blocks
    n = T * Hl * Wl
    k_new = rng.normal(size=(H, n, d)).astype(np.float32)
    v_new = rng.normal(size=(H, n, d)).astype(np.float32)
    cap = 5 * 128
    k_cache = np.full((H, cap, d), np.nan, np.float32)
    v_cache = np.full((H, cap, d), np.nan, np.float32)
    kbar = np.zeros((H, 5, d))
    layout.kv_append(k_cache, v_cache, kbar, k_new, v_new, T, Hl, Wl, chunk_index=3,
                     token_offset=128 * 2, block_offset=2)
    placed = k_cache[:, 256:512]
    assert not np.isnan(placed).any() and np.isnan(k_cache[:, :256]).all()
    # same multiset of rows, and the permutation is the chunk rank map
    ranks = layout.chunk_token_ranks(T, Hl, Wl, 3)
    assert np.array_equal(placed[:, ranks], k_new)
    assert np.array_equal(v_cache[:, 256 + ranks], v_new)
    assert np.allclose(kbar[:, 2], placed[:, :128].astype(np.float64).mean(1))
    assert np.allclose(kbar[:, 3], placed[:, 128:].astype(np.float64).mean(1))
    assert (kbar[:, [0, 1, 4]] == 0).all()


@pytest.mark.parametrize("T,H,W", [(3, 3, 4), (3, 32, 48), (1, 29, 52), (2, 4, 9)])
def test_chunk_parity_of_the_flip(T, H, W):
    # [project] "Keeping neighbours adjacent in the block order", Figure 7
    # caption: chunk 0 keeps the single-chunk curve and chunk 1 is the one
    # flipped horizontally (alternate chunks). The curve starts at cell (0, 0)
    # (pinned above against the textbook Hilbert curve and the path test), so
    # the first token of chunk 0 is frame 0 at column 0 and the first token of
    # chunk 1 is frame 0 at the last column; chunk 2 repeats chunk 0.
    for chunk in range(4):
        pos = _positions(T, H, W, chunk)
        assert pos[0] == (T * chunk, 0, 0 if chunk % 2 == 0 else W - 1)
        rank = layout.cell_rank_map(H, W)
        ranks = layout.chunk_token_ranks(T, H, W, chunk)
        for h in range(H):
            for w in range(W):
                wq = w if chunk % 2 == 0 else W - 1 - w
                assert ranks[h * W + w] == rank[h, wq] * T
