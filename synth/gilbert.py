"""Generalised-Hilbert ("Gilbert") rank map for rectangles, and the chunk-wise
global block order built from it.

This module produces *synthetic inputs only* (block coordinates indexed by
block id). It holds none of the routing or attention arithmetic.

Sources:
- Velox project page ("Velox: Spatial Memory Makes Long-context World Models
  Efficient"), 02 · Method, "Keeping neighbours adjacent in the block order":
  tokens (and hence blocks) follow a Gilbert curve; the per-chunk map is flipped
  horizontally on alternate chunks so neighbours stay adjacent across chunk seams.
- Paper digest ("Velox: Spatial Memory Makes World Models Efficient"),
  Prerequisites, "Gilbert space-filling curve": build one chunk's rank map,
  flip in-chunk coordinates by chunk parity, concatenate; the global order is
  both the KV storage order and the global block id.

The curve itself is the published generalised Hilbert construction for
arbitrary rectangles (J. Cervený, "gilbert"): a rectangle is cut either into two
halves along its long side (when it is much longer than wide) or into a
three-piece U (a transposed lower piece, the upper band, a returning piece),
with piece lengths nudged to even values so consecutive pieces join. The code
below is an explicit-stack restatement of that construction.
"""

from __future__ import annotations

import numpy as np


def _sign(x: int) -> int:
    return (x > 0) - (x < 0)


def _half(v: int) -> int:
    return -((-v) // 2) if v < 0 else v // 2


def gilbert_cells(width: int, height: int) -> list[tuple[int, int]]:
    """Cells (x, y) of a width x height grid in generalised-Hilbert order.

    The path starts at (0, 0); for width >= height it ends at (width - 1, 0).
    Every cell appears exactly once, and consecutive cells are grid neighbours
    (a single diagonal step can occur when the long side is odd).
    """
    if width <= 0 or height <= 0:
        return []
    out: list[tuple[int, int]] = []
    # A piece is (x, y, ax, ay, bx, by): origin cell, major axis vector a and
    # minor axis vector b (their lengths are the piece's cell counts). The
    # pieces are pushed in reverse so they pop in traversal order.
    if width >= height:
        stack = [(0, 0, width, 0, 0, height)]
    else:
        stack = [(0, 0, 0, height, width, 0)]
    while stack:
        x, y, ax, ay, bx, by = stack.pop()
        len_a = abs(ax + ay)
        len_b = abs(bx + by)
        ua = (_sign(ax), _sign(ay))          # unit step along the major axis
        ub = (_sign(bx), _sign(by))          # unit step along the minor axis
        if len_b == 1:                       # one-cell-wide strip: walk it
            for s in range(len_a):
                out.append((x + s * ua[0], y + s * ua[1]))
            continue
        if len_a == 1:
            for s in range(len_b):
                out.append((x + s * ub[0], y + s * ub[1]))
            continue
        hax, hay = _half(ax), _half(ay)      # halves, rounded toward zero
        hbx, hby = _half(bx), _half(by)
        half_a = abs(hax + hay)
        half_b = abs(hbx + hby)
        if 2 * len_a > 3 * len_b:
            # Long piece: two halves along a, both walked in direction a.
            if half_a % 2 == 1 and len_a > 2:
                hax, hay = hax + ua[0], hay + ua[1]
            second = (x + hax, y + hay, ax - hax, ay - hay, bx, by)
            first = (x, y, hax, hay, bx, by)
            stack.append(second)
            stack.append(first)
        else:
            # U shape: up along b (transposed), across the upper band, back down.
            if half_b % 2 == 1 and len_b > 2:
                hbx, hby = hbx + ub[0], hby + ub[1]
            first = (x, y, hbx, hby, hax, hay)
            middle = (x + hbx, y + hby, ax, ay, bx - hbx, by - hby)
            last = (x + (ax - ua[0]) + (hbx - ub[0]),
                    y + (ay - ua[1]) + (hby - ub[1]),
                    -hbx, -hby, -(ax - hax), -(ay - hay))
            stack.append(last)
            stack.append(middle)
            stack.append(first)
    return out


def chunk_block_coords(n_chunks: int, blocks_h: int, blocks_w: int,
                       first_id_offset: int = 0) -> np.ndarray:
    """(t, h, w) block-grid coordinates indexed by global block id.

    Chunk c occupies grid slab t = c. Inside a chunk, block rank k sits at the
    k-th cell of the Gilbert curve over the blocks_w x blocks_h grid; on odd
    chunks the column is mirrored (w -> blocks_w - 1 - w), so the last block of
    one chunk and the first block of the next share (h, w) and differ by one in t.

    With first_id_offset > 0 the first `first_id_offset` ids of chunk 0 are
    dropped (a history window that starts inside a chunk); ids are renumbered
    from 0.
    """
    cells = gilbert_cells(blocks_w, blocks_h)
    per = blocks_w * blocks_h
    coords = np.zeros((n_chunks * per, 3), dtype=np.int32)
    for c in range(n_chunks):
        for k, (cx, cy) in enumerate(cells):
            w = (blocks_w - 1 - cx) if (c % 2 == 1) else cx
            coords[c * per + k] = (c, cy, w)
    return coords[first_id_offset:]
