"""CPU oracle for the global Gilbert order and the KV append.

TEST INFRASTRUCTURE ONLY (imported by the tests, the smoke check and the
benchmark's CPU-baseline leg; the library never calls it and shares no code
with it).

What the pages fix:
- [digest] Prerequisites, "Gilbert space-filling curve": a curve over a 2-D
  grid that keeps neighbouring points close in rank; the global order builds
  one chunk's rank map, flips in-chunk coordinates horizontally by chunk
  parity and concatenates, so neighbours across chunk seams stay adjacent with
  no seam table; the order is the KV storage layout, the 26-neighbour domain
  and the global block id.
- [project] 02 · Method, "Keeping neighbours adjacent in the block order" and
  Figures 6-7: chunk-by-chunk application breaks temporal adjacency, a
  horizontal flip on alternate chunks restores it (toy: latent 3 x 4, block
  size 2, chunks of three frames).
- [onedev] "How it works" / "How to use": the KV cache is stored in the routes'
  global Gilbert order.

Readings where the pages are silent (listed in the design notes):
- the curve is the generalised Hilbert ("Gilbert") curve over the latent
  (height, width) grid of one frame; a chunk of T latent frames is ordered
  cell by cell along it, and the T tokens of a cell follow each other in time
  order: chunk-local rank of token (t, h, w) = rank(h, w') * T + t, with
  w' = w on even chunks and width - 1 - w on odd chunks. The last cell of a
  chunk and the first cell of the next are then the same cell, so the seam
  tokens are consecutive in time;
- the new chunk arrives in THW-linear order (index (t * height + h) * width + w)
  and its T * height * width tokens fill whole 128-token blocks;
- the key-mean cache of the appended blocks is the plain block mean.

The curve is the published generalised-Hilbert construction for arbitrary
rectangles: a rectangle spanned by a major vector a and a minor vector b
(starting at its origin corner, ending at the far end of a on the same side of
b) is either a one-cell strip, or - when it is more than 1.5 times longer than
wide - two halves along a, or a U of three pieces: the first half of b walked
with the roles of a and b swapped, the remaining band walked along a, and a
returning piece; half lengths are nudged to even values so pieces join at
neighbouring cells. Here it is written as repeated refinement of an ordered
piece list.
"""

from __future__ import annotations

import numpy as np


def _sgn(v: int) -> int:
    return (v > 0) - (v < 0)


def _trunc_half(v: int) -> int:
    return int(v / 2)       # toward zero


def _refine(piece):
    """Sub-pieces of a rectangle piece in walking order, or None for a strip."""
    x, y, ax, ay, bx, by = piece
    la, lb = abs(ax + ay), abs(bx + by)
    if la == 1 or lb == 1:
        return None
    ua, ub = (_sgn(ax), _sgn(ay)), (_sgn(bx), _sgn(by))
    hax, hay = _trunc_half(ax), _trunc_half(ay)
    hbx, hby = _trunc_half(bx), _trunc_half(by)
    if 2 * la > 3 * lb:
        if abs(hax + hay) % 2 == 1 and la > 2:
            hax, hay = hax + ua[0], hay + ua[1]
        return [(x, y, hax, hay, bx, by),
                (x + hax, y + hay, ax - hax, ay - hay, bx, by)]
    if abs(hbx + hby) % 2 == 1 and lb > 2:
        hbx, hby = hbx + ub[0], hby + ub[1]
    return [(x, y, hbx, hby, hax, hay),
            (x + hbx, y + hby, ax, ay, bx - hbx, by - hby),
            (x + (ax - ua[0]) + (hbx - ub[0]), y + (ay - ua[1]) + (hby - ub[1]),
             -hbx, -hby, -(ax - hax), -(ay - hay))]


def _strip_cells(piece):
    x, y, ax, ay, bx, by = piece
    la, lb = abs(ax + ay), abs(bx + by)
    if lb == 1:
        step, n = (_sgn(ax), _sgn(ay)), la
    else:
        step, n = (_sgn(bx), _sgn(by)), lb
    return [(x + k * step[0], y + k * step[1]) for k in range(n)]


def gilbert_curve(width: int, height: int) -> list[tuple[int, int]]:
    """Cells (x, y) (x = column < width, y = row < height) in curve order."""
    if width <= 0 or height <= 0:
        return []
    pieces = [(0, 0, width, 0, 0, height) if width >= height else (0, 0, 0, height, width, 0)]
    while True:
        nxt, changed = [], False
        for pc in pieces:
            sub = _refine(pc)
            if sub is None:
                nxt.append(pc)
            else:
                nxt.extend(sub)
                changed = True
        pieces = nxt
        if not changed:
            break
    cells = []
    for pc in pieces:
        cells.extend(_strip_cells(pc))
    return cells


def cell_rank_map(height: int, width: int) -> np.ndarray:
    """rank[h][w]: position of cell (h, w) along the curve (even chunks)."""
    rank = np.full((height, width), -1, dtype=np.int64)
    for k, (x, y) in enumerate(gilbert_curve(width, height)):
        rank[y, x] = k
    return rank


def chunk_token_ranks(T: int, height: int, width: int, chunk_index: int) -> np.ndarray:
    """Chunk-local global-order rank of every token, indexed THW-linearly."""
    rank = cell_rank_map(height, width)
    out = np.empty(T * height * width, dtype=np.int64)
    for t in range(T):
        for h in range(height):
            for w in range(width):
                wq = width - 1 - w if chunk_index % 2 == 1 else w
                out[(t * height + h) * width + w] = rank[h, wq] * T + t
    return out


def kv_append(k_cache, v_cache, kbar, k_new, v_new, T: int, height: int, width: int,
              chunk_index: int, token_offset: int, block_offset: int):
    """Write one chunk into the caches in global order; refresh its key means.

    k_cache, v_cache [H][cap][d], kbar [H][nb][d] (float64 means), k_new, v_new
    [H][T*height*width][d]; arrays are modified in place and also returned.
    """
    ranks = chunk_token_ranks(T, height, width, chunk_index)
    n_tok = ranks.size
    for n in range(n_tok):
        dst = token_offset + int(ranks[n])
        k_cache[:, dst] = k_new[:, n]
        v_cache[:, dst] = v_new[:, n]
    for b in range(n_tok // 128):
        s = token_offset + 128 * b
        kbar[:, block_offset + b] = k_cache[:, s:s + 128].astype(np.float64).mean(axis=1)
    return k_cache, v_cache, kbar
