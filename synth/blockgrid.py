"""Block-grid coordinates of the synthetic workloads, indexed by block id.

This module produces *synthetic inputs only*. The router consumes block
coordinates for its 26-neighbour safeguards and block ids for the
previous-chunk reservation; the only properties it relies on are that ids are
a bijection onto the (t, h, w) block grid, that a chunk's blocks are
contiguous ids, and that chunks follow each other in t. The method's own
global order (a generalised-Hilbert curve per chunk, mirrored on alternate
chunks) is built by the library and by the oracle, not here: the generator
uses a plain serpentine instead, so it holds none of the method's arithmetic.
"""

from __future__ import annotations

import numpy as np


def serpentine_cells(width: int, height: int) -> list[tuple[int, int]]:
    """Cells (x, y) row by row, alternate rows walked right to left."""
    out = []
    for y in range(height):
        xs = range(width) if y % 2 == 0 else range(width - 1, -1, -1)
        out.extend((x, y) for x in xs)
    return out


def chunk_block_coords(n_chunks: int, blocks_h: int, blocks_w: int,
                       first_id_offset: int = 0) -> np.ndarray:
    """(t, h, w) block-grid coordinates indexed by global block id.

    Chunk c occupies grid slab t = c. Inside a chunk, block rank k sits at the
    k-th serpentine cell of the blocks_w x blocks_h grid; odd chunks walk the
    serpentine backwards, so the last block of one chunk and the first block of
    the next share (h, w) and differ by one in t.

    With first_id_offset > 0 the first `first_id_offset` ids of chunk 0 are
    dropped (a history window that starts inside a chunk); ids are renumbered
    from 0.
    """
    cells = serpentine_cells(blocks_w, blocks_h)
    per = blocks_w * blocks_h
    coords = np.zeros((n_chunks * per, 3), dtype=np.int32)
    for c in range(n_chunks):
        order = cells if c % 2 == 0 else cells[::-1]
        for k, (cx, cy) in enumerate(order):
            coords[c * per + k] = (c, cy, cx)
    return coords[first_id_offset:]
