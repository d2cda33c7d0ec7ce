"""Fixed 3-D tile blocks: a block is a tt x th x tw tile of the chunk's latent
grid, on a tile grid aligned to the chunk's origin, and a Gilbert curve over
the tile grid orders the blocks; the local window of a block is its 3 x 3 x 3
neighbourhood of tiles.

Test infrastructure: only tests and the benchmark's CPU baseline use this
module; the library never does.

Pages: [Light Interaction: Training-Free Inference Acceleration for
Interactive Video World Models -- abstract: 3-D block-sparse attention];
[Velox: Spatial Memory Makes World Models Efficient -- Key Contributions 3:
global-aligned Gilbert KV storage; Methodology, Step 5: a 26-neighbour local
window in the Gilbert block ordering; Step 6: neighbouring regions stay
contiguous in memory].

Readings where the pages are silent:

* the tile grid has ceil(T/tt) x ceil(H/th) x ceil(W/tw) tiles, the last
  along each axis clipped to the grid; every chunk uses the same tiles;
* the tiles are ordered by the Gilbert curve of the tile grid (the same
  construction as the token curve);
* a block holds its tile's cells in raster order (t, then h, then w) inside
  the tile, packed to the front; the remaining rows of the block are
  padding, so each block has a valid length like the last block of a run;
* the window of query block b (chunk c) is every block whose tile lies in
  the 3 x 3 x 3 neighbourhood of b's tile (itself included, cut at the
  spatial border); a tile step back in time from the first tile layer lands
  in chunk c-1's last tile layer, a step forward from the last one would
  land in chunk c+1 and is left out.
"""

from __future__ import annotations

import numpy as np

from .gilbert import gilbert_order


def tile_grid(grid, tile):
    T, H, W = grid
    tt, th, tw = tile
    return -(-T // tt), -(-H // th), -(-W // tw)


def tile_layout(grid, tile):
    """``(row_cell, block_len, tile_of_block)``: row_cell[r] is the raster
    cell of row r (-1 for padding) for rows 0 .. n_tiles*V - 1, V = tile
    volume; block_len[b] the valid rows of block b; tile_of_block[b] the
    tile-grid raster index of block b's tile."""
    T, H, W = grid
    tt, th, tw = tile
    nT, nH, nW = tile_grid(grid, tile)
    V = tt * th * tw
    order = gilbert_order(nT, nH, nW)[0]
    row_cell = np.full(len(order) * V, -1, dtype=np.int64)
    block_len = np.zeros(len(order), dtype=np.int64)
    for b, tix in enumerate(order):
        a, rem = divmod(int(tix), nH * nW)
        bh, bw = divmod(rem, nW)
        cells = [(t * H + h) * W + w
                 for t in range(a * tt, min(T, (a + 1) * tt))
                 for h in range(bh * th, min(H, (bh + 1) * th))
                 for w in range(bw * tw, min(W, (bw + 1) * tw))]
        row_cell[b * V: b * V + len(cells)] = cells
        block_len[b] = len(cells)
    return row_cell, block_len, np.asarray(order, dtype=np.int64)


def tile_window(grid, tile, q_chunk: int):
    """Window of every query block of chunk ``q_chunk`` under the tile
    layout: ascending absolute block indices of the blocks whose tiles are
    within one tile step along every axis."""
    nT, nH, nW = tile_grid(grid, tile)
    n_tiles = nT * nH * nW
    _, _, tile_of_block = tile_layout(grid, tile)
    block_of_tile = np.empty(n_tiles, dtype=np.int64)
    block_of_tile[tile_of_block] = np.arange(n_tiles)
    out = []
    for b in range(n_tiles):
        a, rem = divmod(int(tile_of_block[b]), nH * nW)
        bh, bw = divmod(rem, nW)
        found = set()
        for da in (-1, 0, 1):
            aa, chunk = a + da, q_chunk
            if aa < 0:
                aa, chunk = aa + nT, q_chunk - 1
            elif aa >= nT:
                continue
            if chunk < 0:
                continue
            for dh in (-1, 0, 1):
                for dw in (-1, 0, 1):
                    hh, ww = bh + dh, bw + dw
                    if 0 <= hh < nH and 0 <= ww < nW:
                        found.add(chunk * n_tiles + int(block_of_tile[(aa * nH + hh) * nW + ww]))
        out.append(np.array(sorted(found), dtype=np.int64))
    return out


def to_tiles(x_raster: np.ndarray, row_cell: np.ndarray) -> np.ndarray:
    """Raster ``[L][...]`` -> tiled rows ``[n_rows][...]`` (padding rows 0)."""
    out = np.zeros((len(row_cell),) + x_raster.shape[1:], dtype=x_raster.dtype)
    valid = row_cell >= 0
    out[valid] = x_raster[row_cell[valid]]
    return out
