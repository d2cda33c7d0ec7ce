"""GPU parity of the fixed 3-D tile layout against the oracle: the tile
index, the raster <-> tiled permutation, the tile window, and routed
attention (top-K and materialised routes) over tile blocks of a structured
raster workload."""

import numpy as np
import pytest
import torch

import workloads
from oracle import attention as oatt
from oracle import materialize as om
from oracle import route as oroute
from oracle import tiles as ot

from helpers import (BF16_MAX_ABS, BF16_MEAN_ABS, assert_lists_equal, csr_lists, err_summary, f64, need_gpu,
                     valid_rows)

pytestmark = pytest.mark.gpu

CASES = [((3, 30, 52), (1, 8, 16)), ((3, 30, 52), (1, 8, 8)), ((3, 30, 52), (2, 8, 8)), ((2, 5, 7), (2, 2, 3)),
         ((4, 6, 6), (2, 3, 3))]


@pytest.mark.parametrize("grid,tile", CASES)
def test_tile_index_matches_oracle(grid, tile):
    dev = need_gpu()
    import block_sparse_attention_gilbert_amd as bsa
    row_cell, block_len, cell_row = bsa.gilbert_tile_index(*grid, tile, device=dev)
    torch.cuda.synchronize()
    rc, bl, _ = ot.tile_layout(grid, tile)
    assert np.array_equal(row_cell.cpu().numpy(), rc)
    assert np.array_equal(block_len.cpu().numpy(), bl)
    cr = cell_row.cpu().numpy()
    assert np.array_equal(rc[cr], np.arange(int(np.prod(grid))))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_tile_perm_round_trip_and_oracle_layout(dtype):
    dev = need_gpu()
    import block_sparse_attention_gilbert_amd as bsa
    grid, tile = (3, 30, 52), (1, 8, 16)
    L = 4680
    row_cell, _, _ = bsa.gilbert_tile_index(*grid, tile, device=dev)
    rc = row_cell.cpu().numpy()
    heads, d = 3, 64
    x = torch.randn((L, heads, d), generator=torch.Generator().manual_seed(4)).to(dtype)
    # the tiled chunk lands in slot 1 of a 3-slot store (head-strided view)
    store = torch.full((heads, 3 * len(rc), d), 7.0, dtype=dtype, device=dev)
    slot = store[:, len(rc): 2 * len(rc)]
    bsa.tile_perm(x.to(dev), row_cell, dst=slot)
    back = bsa.tile_perm(slot, row_cell, inverse=True, L=L)
    torch.cuda.synchronize()
    ref = ot.to_tiles(x.float().numpy(), rc)                                         # [rows][heads][d]
    got = slot.cpu().float().numpy().transpose(1, 0, 2)
    assert np.array_equal(got, ref)                                                  # bitwise, padding zero
    assert torch.equal(back.cpu(), x)
    assert torch.all(store[:, : len(rc)] == 7.0) and torch.all(store[:, 2 * len(rc):] == 7.0)


@pytest.mark.parametrize("grid,tile", CASES)
@pytest.mark.parametrize("q_chunk", [0, 3])
def test_tile_window_matches_oracle(grid, tile, q_chunk):
    dev = need_gpu()
    import block_sparse_attention_gilbert_amd as bsa
    row_cell, _, cell_row = bsa.gilbert_tile_index(*grid, tile, device=dev)
    window, wlen = bsa.tile_block_window(row_cell, cell_row, grid, block=int(np.prod(tile)), q_chunk=q_chunk)
    torch.cuda.synchronize()
    ref = ot.tile_window(grid, tile, q_chunk)
    win, wl = window.cpu().numpy(), wlen.cpu().numpy()
    assert len(wl) == len(ref)
    for b, rb in enumerate(ref):
        assert np.array_equal(win[b, :wl[b]], rb), (b, win[b, :wl[b]], rb)


def _tiled_f64(x_raster_h, rc):
    """float64 tiled rows of one head's raster tensor [L][d] (bf16 exact)."""
    return ot.to_tiles(f64(x_raster_h), rc)


def test_routed_attention_over_tile_blocks():
    """Three chunks of the structured workload through the pipeline with
    (1, 8, 8) tiles: the step's top-K lists and attention output, then the
    materialised routes with the tile window, against the oracle on its own
    tile layout."""
    dev = need_gpu()
    from block_sparse_attention_gilbert_amd.pipeline import RoutedAttention
    grid, tile, n_chunks = (3, 30, 52), (1, 8, 8), 3
    w = workloads.c5(heads=[0, 7], n_chunks=n_chunks)
    ra = RoutedAttention(grid, w.heads, w.d, 64, n_chunks, device=dev, k_cap=20, tile=tile)
    for c in range(n_chunks - 1):
        ra.append(w.k_raster[c].to(dev), w.v_raster[c].to(dev), c)
    cur = n_chunks - 1
    q_r, k_r, v_r = w.q_raster.to(dev), w.k_raster[cur].to(dev), w.v_raster[cur].to(dev)
    o_r, r = ra.step(q_r, k_r, v_r, cur, k_fixed=20)
    torch.cuda.synchronize()
    got = csr_lists(r["row_ptr"], r["col_idx"], w.heads, ra.nbc)
    rc, bl, _ = ot.tile_layout(grid, tile)
    k_len = np.tile(bl, n_chunks)
    vmask = valid_rows(bl, 64)
    rows = np.nonzero(rc >= 0)[0]
    for hi in range(w.heads):
        q = _tiled_f64(w.q_raster[:, hi], rc)
        k = np.concatenate([_tiled_f64(w.k_raster[c][:, hi], rc) for c in range(n_chunks)])
        v = np.concatenate([_tiled_f64(w.v_raster[c][:, hi], rc) for c in range(n_chunks)])
        ref = oroute.route_head(q, k, bl, k_len, 64, scale=w.scale, k_per_row=np.full(len(bl), 20))
        assert_lists_equal(got[hi], ref["lists"], "head %d" % hi)
        o_ref, _ = oatt.block_sparse_head(q, k, v, bl, k_len, 64, ref["lists"], w.scale)
        # the step writes O in raster order: tiled row g is token rc[g]
        o_tiles = np.zeros_like(o_ref)
        o_tiles[rows] = f64(o_r[:, hi])[rc[rows]]
        mx, mean = err_summary(o_tiles, o_ref, vmask)
        assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, (hi, mx, mean)
    # materialised routes with the tile window (query chunk 2, previous chunk 1 reserved)
    cov = torch.tensor(np.linspace(0.5, 1.0, ra.nbc), dtype=torch.float32, device=dev)
    mat = dict(coverage=cov, k_cov=30, k_unc=40, mass=0.8, ref_blocks=(0, 2))
    rm = ra.route_materialized(cur, **mat)
    torch.cuda.synchronize()
    gotm = csr_lists(rm["row_ptr"], rm["col_idx"], w.heads, ra.nbc)
    win = ot.tile_window(grid, tile, cur)
    prev = ((cur - 1) * ra.nbc, cur * ra.nbc)
    for hi in range(w.heads):
        q = _tiled_f64(w.q_raster[:, hi], rc)
        k = np.concatenate([_tiled_f64(w.k_raster[c][:, hi], rc) for c in range(n_chunks)])
        ref = om.materialize_head(q, k, bl, k_len, 64, scale=w.scale, coverage=cov.cpu().numpy(), k_cov=30,
                                  k_unc=40, mass=0.8, prev_blocks=prev, windows=win, ref_blocks=(0, 2))
        assert_lists_equal(gotm[hi], ref["lists"], "materialised head %d" % hi)
