"""One attention call of a chunked model over its growing KV history, as a
chain of the library's entry points with every buffer allocated up front.

[Velox: Spatial Memory Makes World Models Efficient -- Methodology (chunks
are produced in sequence and the KV cache holds all earlier ones; what
changes is only the set of earlier KV blocks a region may attend to),
Steps 4-6; Key Contributions 3]

Per call (``RoutedAttention.step``):

1. the chunk's Gilbert order (computed once per grid shape and kept); blocks
   are runs of ``block`` tokens along it, or, with ``tile=(tt, th, tw)``,
   fixed tt x th x tw tiles ordered by the Gilbert curve of the tile grid
   [Light Interaction -- abstract: 3-D block-sparse attention];
2. K and V of the current chunk, raster token-major ``[L][heads][d]``, are
   permuted into Gilbert head-major block-padded layout in the current
   chunk's slot of the KV store (the store grows by appending); the
   permutation of K also writes its block means into the pooled-key cache.
   Q is only read for its block means (the pooled queries): with blocks
   that are runs of the curve the attention reads Q in raster order through
   the curve; fixed tiles permute Q into ``q_blk``.  With curve blocks and
   the pooled-key cache, Q, K and V go through one launch;
3. the router scores, fuses and selects over the visible history.  The
   pooled keys of the history are kept in a float64 cache across calls
   (the store only grows by appending), so a call pools only the blocks
   appended or rewritten since the previous call.  The selection is either
   a top-K per row, or the materialised route (``materialize=``): coverage-
   gated budgets, the previous chunk's reservation, the cumulative-mass
   prefix, and the chunk's local window in Gilbert block order (built on
   the GPU for each call) plus reference blocks [Velox -- Methodology,
   Step 5];
4. block-sparse attention over the selected blocks, whose epilogue writes
   O straight back in raster token order (the inverse permutation).

``q_blk`` therefore holds the permuted queries only where something put
them there (fixed tiles, or the caller, e.g. before ``route_and_attend`` or
``dense``).

Nothing here computes on the host: each step is one or more HIP kernels of
``libbsa.so`` on the current stream.
"""

from __future__ import annotations

import math
from typing import Optional

import torch

from . import (_check, _lib, _ptr, _stream, block_sparse_attn, block_sparse_attn_raster, dense_attn,
               gilbert_block_window, gilbert_index, gilbert_perm, gilbert_perm_pool, gilbert_perm_pool_batch,
               gilbert_tile_index, materialize_capacity, route_capacity, route_materialize, route_topk,
               tile_block_window, tile_perm)


def block_lengths(tokens: int, block: int, n_chunks: int = 1, device="cuda") -> torch.Tensor:
    nb = -(-tokens // block)
    one = [min(block, tokens - b * block) for b in range(nb)]
    return torch.tensor(one * n_chunks, dtype=torch.int32, device=device)


class RoutedAttention:
    """Buffers and state for routed attention over a KV store of
    ``store_chunks`` chunks of a ``grid`` = (T, H, W) latent chunk."""

    def __init__(self, grid, heads: int, d: int, block: int, store_chunks: int, dtype=torch.bfloat16,
                 device="cuda", k_cap: int = 50, n_dense_tail_chunks: int = 0,
                 k_store: Optional[torch.Tensor] = None, v_store: Optional[torch.Tensor] = None,
                 use_kpool: bool = True, tile=None):
        self.grid = tuple(grid)
        self.L = grid[0] * grid[1] * grid[2]
        self.heads, self.d, self.block, self.dtype, self.device = heads, d, block, dtype, device
        self.tile = None if tile is None else tuple(int(x) for x in tile)
        if self.tile is not None:
            if self.tile[0] * self.tile[1] * self.tile[2] != block:
                raise ValueError("the tile volume must equal the block size")
            self.row_cell, self.block_len, self.cell_row = gilbert_tile_index(*self.grid, self.tile, device=device)
            self.nbc = self.block_len.numel()        # blocks (tiles) per chunk
        else:
            self.nbc = -(-self.L // block)           # blocks per chunk
        self.rows_c = self.nbc * block
        self.store_chunks = store_chunks
        self.k_cap = k_cap
        self.n_dense_tail_chunks = n_dense_tail_chunks
        self.scale = 1.0 / math.sqrt(d)
        shape = (heads, store_chunks * self.rows_c, d)
        self.k_store = torch.zeros(shape, dtype=dtype, device=device) if k_store is None else k_store
        self.v_store = torch.zeros(shape, dtype=dtype, device=device) if v_store is None else v_store
        self.q_blk = torch.empty((heads, self.rows_c, d), dtype=dtype, device=device)
        self.o_blk = torch.empty((heads, self.rows_c, d), dtype=dtype, device=device)
        self.o_raster = torch.empty((self.L, heads, d), dtype=dtype, device=device)
        self.lse = torch.empty((heads, self.rows_c), dtype=torch.float32, device=device)
        if self.tile is not None:
            self.q_len = self.block_len.clone()
            self.kv_len = self.block_len.repeat(store_chunks)
        else:
            self.q_len = block_lengths(self.L, block, 1, device)
            self.kv_len = block_lengths(self.L, block, store_chunks, device)
        self.perm, self.inv = gilbert_index(*self.grid, device=device)
        nkb_max = store_chunks * self.nbc
        tail = n_dense_tail_chunks * self.nbc
        self.route_out = {
            "row_ptr": torch.empty(heads * self.nbc + 1, dtype=torch.int32, device=device),
            "col_idx": torch.empty(max(1, route_capacity(heads, self.nbc, nkb_max, k_cap, tail)),
                                   dtype=torch.int32, device=device),
            "fallback_counts": torch.zeros(2, dtype=torch.int32, device=device),
            "sel_keys": None,
        }
        self.workspace = None
        # pooled-key cache: blocks < _kpool_valid hold the means of the
        # store's current contents
        self.use_kpool = use_kpool
        self.kpool = torch.empty((heads, nkb_max, d), dtype=torch.float64, device=device) if use_kpool else None
        self._kpool_valid = 0
        # pooled queries of the current chunk, written by the permutation
        self.qbar = torch.empty((heads, self.nbc, d), dtype=torch.float64, device=device)
        # materialised routes: window rows of the current chunk, lists and
        # workspace (allocated on first use)
        self.window = torch.empty((self.nbc, 2 * self.nbc), dtype=torch.int32, device=device)
        self.window_len = torch.empty(self.nbc, dtype=torch.int32, device=device)
        self.mat_out = None
        self.mat_workspace = None

    def invalidate_kpool(self, first_block: int = 0):
        """Forget cached pooled keys from ``first_block`` on (call after
        writing the store other than through ``append``)."""
        self._kpool_valid = min(self._kpool_valid, max(0, int(first_block)))

    def slot(self, c: int):
        """K and V views of chunk ``c``'s slot of the store."""
        r0, r1 = c * self.rows_c, (c + 1) * self.rows_c
        return self.k_store[:, r0:r1, :], self.v_store[:, r0:r1, :]

    def to_blocks(self, src, dst, stream=None):
        """Raster ``[L][heads][d]`` -> this layout's blocks (``dst``)."""
        if self.tile is not None:
            return tile_perm(src, self.row_cell, dst=dst, stream=stream)
        return gilbert_perm(src, self.perm, block=self.block, dst=dst, stream=stream)

    def to_raster(self, src, dst, stream=None):
        """This layout's blocks -> raster ``[L][heads][d]`` (``dst``)."""
        if self.tile is not None:
            return tile_perm(src, self.row_cell, inverse=True, dst=dst, L=self.L, stream=stream)
        return gilbert_perm(src, self.perm, block=self.block, inverse=True, dst=dst, stream=stream)

    def append(self, k_raster, v_raster, c: int, stream=None):
        """Permute a chunk's raster K and V into slot ``c`` of the store; with
        the pooled-key cache (curve blocks), the chunk's pooled keys are
        written into it by the same pass."""
        ks, vs = self.slot(c)
        b0 = c * self.nbc
        self.invalidate_kpool(b0)
        if self.use_kpool and self.tile is None:
            gilbert_perm_pool(k_raster, self.perm, block=self.block, dst=ks, pool=self.kpool[:, b0:b0 + self.nbc],
                              stream=stream)
            if self._kpool_valid == b0:
                self._kpool_valid = b0 + self.nbc
        else:
            self.to_blocks(k_raster, ks, stream)
        self.to_blocks(v_raster, vs, stream)

    def permute_inputs(self, q_raster, k_raster, v_raster, c: int, stream=None, q_blocks: bool = True):
        """Append chunk ``c``'s K and V to the store and permute its queries
        into ``q_blk``.  With curve blocks the queries' block means are
        written by the same pass: returns them (``qbar``), else None.
        ``q_blocks=False`` (curve blocks only): the block means alone, the
        queries stay in raster order (the attention reads them there)."""
        if self.tile is None and self.use_kpool:
            # Q, K and V through one launch (the same bits as the three calls)
            ks, vs = self.slot(c)
            b0 = c * self.nbc
            self.invalidate_kpool(b0)
            gilbert_perm_pool_batch([(q_raster, self.q_blk if q_blocks else None, self.qbar),
                                     (k_raster, ks, self.kpool[:, b0:b0 + self.nbc]), (v_raster, vs, None)],
                                    self.perm, block=self.block, stream=stream)
            if self._kpool_valid == b0:
                self._kpool_valid = b0 + self.nbc
            return self.qbar
        self.append(k_raster, v_raster, c, stream)
        if self.tile is not None:
            self.to_blocks(q_raster, self.q_blk, stream)
            return None
        if q_blocks:
            gilbert_perm_pool(q_raster, self.perm, block=self.block, dst=self.q_blk, pool=self.qbar, stream=stream)
        else:
            gilbert_perm_pool(q_raster, self.perm, block=self.block, pool=self.qbar, pool_only=True, stream=stream)
        return self.qbar

    def step(self, q_raster, k_raster, v_raster, c: int, *, k_fixed: Optional[int] = None,
             k_per_row: Optional[torch.Tensor] = None, overlap: Optional[torch.Tensor] = None,
             lam=2.0, g_ref=0.2, tau=0.1, materialize: Optional[dict] = None, refresh_index: bool = False,
             stream=None, attn_events=None):
        """One attention call for chunk ``c`` (0-based) over chunks 0..c.
        Returns ``(o_raster, route_out)``.  ``attn_events``: optional list
        that receives a (start, end) pair of timing events recorded around
        the attention kernel on the stream it runs on.  ``materialize``:
        keyword arguments of ``route_materialize`` (``coverage``,
        ``eta_cov``, ``k_cov``, ``k_unc``, ``mass``, ``ref_blocks``; plus
        ``window=False`` to leave the local window out) to route with the
        materialised lists instead of a top-K.  The chunk's Gilbert order is
        fixed by its grid: it is computed when the object is built and kept;
        ``refresh_index`` recomputes it into the same buffers first."""
        if refresh_index:
            self._index(stream)
        # curve blocks: Q stays raster (its block means taken in one read),
        # the attention reads it and writes O through the curve
        q_raster_in = q_raster if self.tile is None else None
        qpool = self.permute_inputs(q_raster, k_raster, v_raster, c, stream, q_blocks=self.tile is not None)
        r = self.route_and_attend(c, k_fixed=k_fixed, k_per_row=k_per_row, overlap=overlap, lam=lam, g_ref=g_ref,
                                  tau=tau, materialize=materialize, qpool=qpool, out_raster=True,
                                  q_raster=q_raster_in, stream=stream, attn_events=attn_events)
        return self.o_raster, r

    def route_and_attend(self, c: int, *, k_fixed: Optional[int] = None, k_per_row: Optional[torch.Tensor] = None,
                         overlap: Optional[torch.Tensor] = None, lam=2.0, g_ref=0.2, tau=0.1,
                         materialize: Optional[dict] = None, qpool=None, out_raster: bool = False, q_raster=None,
                         stream=None, attn_events=None):
        """Route the already permuted queries over chunks 0..c of the store
        and attend; the result stays in Gilbert layout (``o_blk``, ``lse``),
        or with ``out_raster`` goes straight to ``o_raster`` (``o_blk`` is
        then not written).  ``qpool``: their pooled means, when already
        computed; ``q_raster``: the queries in raster order, read by the
        attention in place of ``q_blk`` (needs ``qpool`` and
        ``out_raster``)."""
        nkb = (c + 1) * self.nbc
        k_hist, v_hist = self.k_store[:, : nkb * self.block], self.v_store[:, : nkb * self.block]
        if materialize is not None:
            r = self.route_materialized(c, overlap=overlap, lam=lam, g_ref=g_ref, tau=tau, qpool=qpool,
                                        stream=stream, **materialize)
        else:
            r = self.route(c, k_fixed=k_fixed, k_per_row=k_per_row, overlap=overlap, lam=lam, g_ref=g_ref, tau=tau,
                           qpool=qpool, stream=stream)
        return self._attend(r, nkb, k_hist, v_hist, stream, attn_events, out_raster, q_raster)

    def route(self, c: int, *, k_fixed: Optional[int] = None, k_per_row: Optional[torch.Tensor] = None,
              overlap: Optional[torch.Tensor] = None, lam=2.0, g_ref=0.2, tau=0.1, qpool=None, stream=None):
        """Top-K routes of the already permuted queries over chunks 0..c
        (``qpool``: their pooled means, when already computed)."""
        nkb = (c + 1) * self.nbc
        k_hist = self.k_store[:, : nkb * self.block]
        tail = self.n_dense_tail_chunks * self.nbc
        kf = self.k_cap if k_fixed is None else k_fixed
        n_cand = nkb - tail
        valid = min(self._kpool_valid, n_cand)
        r = route_topk(self.q_blk, k_hist, block=self.block, nqb=self.nbc, nkb=nkb, scale=self.scale,
                       q_block_len=self.q_len, kv_block_len=self.kv_len[:nkb], overlap=overlap, lam=lam,
                       g_ref=g_ref, tau=tau, k_fixed=kf, k_per_row=k_per_row,
                       k_max=self.k_cap if k_per_row is not None else None, n_dense_tail_blocks=tail,
                       kpool=self.kpool, kpool_valid_blocks=valid if self.use_kpool else 0, qpool=qpool,
                       out=self.route_out, workspace=self.workspace, stream=stream)
        self.workspace = r["workspace"]
        if self.use_kpool:
            self._kpool_valid = max(valid, n_cand)
        return r

    def route_materialized(self, c: int, *, coverage=None, eta_cov=0.9, k_cov=80, k_unc=150, mass=0.9,
                           ref_blocks=(0, 0), window: bool = True, overlap=None, lam=2.0, g_ref=0.2, tau=0.1,
                           qpool=None, stream=None):
        """Materialised routes of the current queries over chunks 0..c:
        chunk c-1 is the reserved previous chunk; the local window of chunk
        c is rebuilt into the preallocated rows first."""
        nkb = (c + 1) * self.nbc
        k_hist = self.k_store[:, : nkb * self.block]
        if window and self.tile is not None:
            tile_block_window(self.row_cell, self.cell_row, self.grid, block=self.block, q_chunk=c,
                              out=(self.window, self.window_len), stream=stream)
        elif window:
            gilbert_block_window(self.perm, self.inv, self.grid, block=self.block, q_chunk=c,
                                 out=(self.window, self.window_len), stream=stream)
        prev = ((c - 1) * self.nbc, c * self.nbc) if c > 0 else (0, 0)
        cap = materialize_capacity(self.heads, self.nbc, nkb, k_cov=k_cov, k_unc=k_unc, prev_blocks=prev,
                                   window_stride=self.window.stride(0) if window else 0, ref_blocks=ref_blocks)
        if self.mat_out is None or self.mat_out["col_idx"].numel() < cap:
            self.mat_out = {"row_ptr": torch.empty(self.heads * self.nbc + 1, dtype=torch.int32, device=self.device),
                            "col_idx": torch.empty(max(1, cap), dtype=torch.int32, device=self.device),
                            "sel_keys": None}
        valid = min(self._kpool_valid, nkb)
        r = route_materialize(self.q_blk, k_hist, block=self.block, nqb=self.nbc, nkb=nkb, scale=self.scale,
                              q_block_len=self.q_len, kv_block_len=self.kv_len[:nkb], overlap=overlap, lam=lam,
                              g_ref=g_ref, tau=tau, coverage=coverage, eta_cov=eta_cov, k_cov=k_cov, k_unc=k_unc,
                              mass=mass, prev_blocks=prev, window=self.window if window else None,
                              window_len=self.window_len if window else None, ref_blocks=ref_blocks,
                              kpool=self.kpool, kpool_valid_blocks=valid if self.use_kpool else 0, qpool=qpool,
                              out=self.mat_out, workspace=self.mat_workspace, stream=stream)
        self.mat_workspace = r["workspace"]
        if self.use_kpool:
            self._kpool_valid = max(valid, nkb)
        return r

    def _attend(self, r, nkb, k_hist, v_hist, stream, attn_events, out_raster=False, q_raster=None):
        if attn_events is not None:
            ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            ev[0].record(stream)
        if out_raster:
            # the inverse permutation in the kernel's epilogue: row g -> token
            # row_map[g] (and, for raster queries, the forward one in its loads)
            row_map = self.perm if self.tile is None else self.row_cell
            block_sparse_attn_raster(self.q_blk if q_raster is None else q_raster, k_hist, v_hist, r["row_ptr"],
                                     r["col_idx"], row_map, block=self.block, scale=self.scale,
                                     q_block_len=self.q_len, kv_block_len=self.kv_len[:nkb], out=self.o_raster,
                                     lse=self.lse, q_raster=q_raster is not None, stream=stream)
        else:
            block_sparse_attn(self.q_blk, k_hist, v_hist, r["row_ptr"], r["col_idx"], block=self.block,
                              scale=self.scale, q_block_len=self.q_len, kv_block_len=self.kv_len[:nkb],
                              out=self.o_blk, lse=self.lse, stream=stream)
        if attn_events is not None:
            ev[1].record(stream)
            attn_events.append(ev)
        return r

    def _index(self, stream=None):
        """Recompute the chunk's Gilbert order (or tile layout) into the
        preallocated buffers."""
        if self.tile is not None:
            _check(_lib.bsa_gilbert_tile_index(self.grid[0], self.grid[1], self.grid[2], *self.tile,
                                               _ptr(self.row_cell), _ptr(self.block_len), _ptr(self.cell_row),
                                               _stream(stream)))
            return
        _check(_lib.bsa_gilbert_index(self.grid[0], self.grid[1], self.grid[2], _ptr(self.perm), _ptr(self.inv),
                                      _stream(stream)))

    def dense(self, c: int, stream=None):
        """Dense attention of the current (already permuted) queries over
        chunks 0..c, through the same kernel."""
        nkb = (c + 1) * self.nbc
        return dense_attn(self.q_blk, self.k_store[:, : nkb * self.block], self.v_store[:, : nkb * self.block],
                          block=self.block, scale=self.scale, q_block_len=self.q_len,
                          kv_block_len=self.kv_len[:nkb], out=self.o_blk, lse=self.lse, stream=stream)
