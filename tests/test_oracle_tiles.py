"""Pins of the fixed 3-D tile layout: a bijection between valid rows and
cells with padding packed at the end of each block, every block inside one
tile in raster order, unit steps between consecutive tiles, and the tile
window equal to the token-level 3 x 3 x 3 neighbourhood union computed
independently."""

import itertools

import numpy as np
import pytest

from oracle import tiles as ot

CASES = [((3, 30, 52), (1, 8, 16)), ((3, 30, 52), (3, 4, 8)), ((3, 30, 52), (1, 8, 8)), ((2, 5, 7), (2, 2, 3)),
         ((4, 6, 6), (2, 3, 3))]


@pytest.mark.parametrize("grid,tile", CASES)
def test_layout_is_a_padded_bijection_of_tiles(grid, tile):
    T, H, W = grid
    tt, th, tw = tile
    L, V = T * H * W, tt * th * tw
    row_cell, block_len, tob = ot.tile_layout(grid, tile)
    nT, nH, nW = ot.tile_grid(grid, tile)
    assert len(block_len) == nT * nH * nW and len(row_cell) == len(block_len) * V
    assert sorted(row_cell[row_cell >= 0].tolist()) == list(range(L))
    assert sorted(tob.tolist()) == list(range(nT * nH * nW))
    for b in range(len(block_len)):
        rows = row_cell[b * V:(b + 1) * V]
        n = int(block_len[b])
        assert np.all(rows[:n] >= 0) and np.all(rows[n:] == -1)
        t, h, w = rows[:n] // (H * W), (rows[:n] // W) % H, rows[:n] % W
        tix = (t // tt * nH + h // th) * nW + w // tw
        assert np.all(tix == tob[b])                                  # one tile
        assert np.all(np.diff(rows[:n]) > 0)                          # raster order inside it
        a, rem = divmod(int(tob[b]), nH * nW)
        bh, bw = divmod(rem, nW)
        assert n == (min(T, (a + 1) * tt) - a * tt) * (min(H, (bh + 1) * th) - bh * th) * \
            (min(W, (bw + 1) * tw) - bw * tw)


def test_tile_order_takes_unit_steps():
    """Consecutive tiles share a face wherever the tile grid's parity lets a
    path of unit steps join the curve's two ends (an even number of tiles
    with both ends of one colour forces one longer step)."""
    checked = 0
    for grid, tile in CASES:
        _, _, tob = ot.tile_layout(grid, tile)
        nT, nH, nW = ot.tile_grid(grid, tile)
        c = np.stack([tob // (nH * nW), (tob // nW) % nH, tob % nW], axis=1)
        steps = np.abs(np.diff(c, axis=0)).sum(axis=1)
        feasible = len(tob) % 2 == 1 or c[0].sum() % 2 != c[-1].sum() % 2
        if feasible:
            assert np.all(steps == 1), (grid, tile)
            checked += 1
        else:
            assert np.sum(steps != 1) <= 1, (grid, tile)
    assert checked >= 3


def _token_window(grid, tile, q_chunk):
    """Token-level definition: blocks holding any 3 x 3 x 3 neighbour cell of
    any valid cell of the block."""
    T, H, W = grid
    V = int(np.prod(tile))
    row_cell, block_len, _ = ot.tile_layout(grid, tile)
    n_blocks = len(block_len)
    block_of_cell = np.empty(T * H * W, dtype=np.int64)
    valid = row_cell >= 0
    block_of_cell[row_cell[valid]] = np.nonzero(valid)[0] // V
    out = []
    for b in range(n_blocks):
        found = set()
        for cell in row_cell[b * V: b * V + int(block_len[b])]:
            t, h, w = cell // (H * W), (cell // W) % H, cell % W
            for dt, dh, dw in itertools.product((-1, 0, 1), repeat=3):
                tt_, hh, ww = t + dt, h + dh, w + dw
                if not (0 <= hh < H and 0 <= ww < W) or tt_ >= T:
                    continue
                chunk = q_chunk if tt_ >= 0 else q_chunk - 1
                if chunk < 0:
                    continue
                found.add(chunk * n_blocks + int(block_of_cell[((tt_ % T) * H + hh) * W + ww]))
        out.append(np.array(sorted(found), dtype=np.int64))
    return out


@pytest.mark.parametrize("grid,tile", CASES)
@pytest.mark.parametrize("q_chunk", [0, 2])
def test_tile_window_is_the_token_neighbourhood_union(grid, tile, q_chunk):
    tw = ot.tile_window(grid, tile, q_chunk)
    ref = _token_window(grid, tile, q_chunk)
    assert len(tw) == len(ref)
    for a, b in zip(tw, ref):
        assert np.array_equal(a, b)


def test_tile_window_sizes():
    grid, tile = (3, 30, 52), (1, 8, 16)
    nT, nH, nW = ot.tile_grid(grid, tile)
    _, _, tob = ot.tile_layout(grid, tile)
    win = ot.tile_window(grid, tile, 5)
    n_tiles = nT * nH * nW
    for b, wb in enumerate(win):
        a, rem = divmod(int(tob[b]), nH * nW)
        bh, bw = divmod(rem, nW)
        spatial = len([1 for dh in (-1, 0, 1) for dw in (-1, 0, 1) if 0 <= bh + dh < nH and 0 <= bw + dw < nW])
        layers = 2 if a == nT - 1 else 3              # the next chunk is not history
        assert len(wb) == spatial * layers
        assert (5 * n_tiles + b) in wb
        assert np.all((wb >= 4 * n_tiles) & (wb < 6 * n_tiles))


def test_to_tiles_round_trip():
    grid, tile = (2, 5, 7), (2, 2, 3)
    row_cell, _, _ = ot.tile_layout(grid, tile)
    x = np.arange(70 * 3).reshape(70, 3)
    y = ot.to_tiles(x, row_cell)
    assert np.all(y[row_cell < 0] == 0)
    back = np.zeros_like(x)
    back[row_cell[row_cell >= 0]] = y[row_cell >= 0]
    assert np.array_equal(back, x)
