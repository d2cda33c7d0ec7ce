"""Routed, indexed block-sparse attention over a Gilbert-ordered KV history,
for AMD Instinct MI355X (gfx950).

A thin ctypes binding of ``libbsa.so`` (C ABI in ``include/bsa.h``).  The
functions here only marshal arguments: every step of the path runs in the
library's HIP kernels, on ``torch.cuda.current_stream()`` unless a stream is
given.  PyTorch provides device memory and streams.  If the library has not
been built, importing this package raises ImportError; there is no fallback.

Entry points (same names as the C ABI, without the ``bsa_`` prefix):
``gilbert_index``, ``gilbert_perm``, ``gilbert_block_window``,
``gilbert_tile_index``, ``tile_perm``, ``tile_block_window``,
``slab_overlap``, ``slab_coverage``, ``route_topk`` (with
``route_workspace_size``), ``route_topk_static`` (no workspace), ``route_materialize`` (with
``route_materialize_workspace_size``), ``block_sparse_attn``,
``dense_attn``.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbsa.so")

BSA_OK, BSA_EINVAL, BSA_EUNSUPPORTED, BSA_EWORKSPACE, BSA_EHIP = range(5)
BSA_BF16, BSA_F32 = 0, 1

if not os.path.exists(LIB_PATH):
    raise ImportError(
        "libbsa.so is not built: run `python block_sparse_attention_gilbert_amd/build.py` "
        "(or __graft_entry__.build()) first")

_lib = ctypes.CDLL(LIB_PATH)

_p = ctypes.c_void_p
_i = ctypes.c_int
_i64 = ctypes.c_int64
_f = ctypes.c_float


class RouteArgs(ctypes.Structure):
    """Mirror of ``bsa_route_args``."""
    _fields_ = [
        ("struct_size", ctypes.c_size_t),
        ("q", _p), ("k", _p), ("dtype", _i),
        ("heads", _i), ("d", _i), ("block", _i), ("nqb", _i), ("nkb", _i),
        ("q_head_stride", _i64), ("k_head_stride", _i64),
        ("q_block_len", _p), ("kv_block_len", _p),
        ("scale", ctypes.c_double),
        ("overlap", _p), ("overlap_row_stride", _i64),
        ("lam", ctypes.c_double), ("g_ref", ctypes.c_double), ("tau", ctypes.c_double),
        ("k_fixed", _i), ("k_per_row", _p), ("k_max", _i),
        ("n_dense_tail_blocks", _i),
        ("kpool", _p), ("kpool_valid_blocks", _i), ("kpool_head_blocks", _i),
        ("row_ptr", _p), ("col_idx", _p), ("col_capacity", _i64),
        ("fallback_counts", _p), ("sel_keys", _p),
        ("qpool", _p), ("qpool_head_stride", _i64),
    ]


class MaterializeArgs(ctypes.Structure):
    """Mirror of ``bsa_materialize_args``."""
    _fields_ = [
        ("struct_size", ctypes.c_size_t),
        ("coverage", _p), ("eta_cov", ctypes.c_double),
        ("k_cov", _i), ("k_unc", _i), ("mass", ctypes.c_double),
        ("prev_begin", _i), ("prev_end", _i),
        ("window", _p), ("window_len", _p), ("window_stride", _i),
        ("ref_begin", _i), ("ref_end", _i),
    ]


class PermJob(ctypes.Structure):
    """Mirror of ``bsa_perm_job``."""
    _fields_ = [
        ("src", _p), ("dst", _p), ("raster_token_stride", _i64), ("gilbert_head_stride", _i64),
        ("pool", _p), ("pool_head_stride", _i64),
    ]


MAX_PERM_JOBS = 4  # BSA_MAX_PERM_JOBS

_lib.bsa_version.restype = _i
_lib.bsa_strerror.restype = ctypes.c_char_p
_lib.bsa_strerror.argtypes = [_i]
_lib.bsa_last_error_detail.restype = ctypes.c_char_p
_lib.bsa_gilbert_index.restype = _i
_lib.bsa_gilbert_index.argtypes = [_i, _i, _i, _p, _p, _p]
_lib.bsa_gilbert_perm.restype = _i
_lib.bsa_gilbert_perm.argtypes = [_p, _p, _p, _i, _i, _i, _i, _i64, _i64, _i, _i, _p]
_lib.bsa_gilbert_perm_pool.restype = _i
_lib.bsa_gilbert_perm_pool.argtypes = [_p, _p, _p, _i, _i, _i, _i, _i64, _i64, _i, _p, _i64, _p]
_lib.bsa_gilbert_perm_pool_batch.restype = _i
_lib.bsa_gilbert_perm_pool_batch.argtypes = [ctypes.POINTER(PermJob), _i, _p, _i, _i, _i, _i, _i, _p]
_lib.bsa_gilbert_block_window.restype = _i
_lib.bsa_gilbert_block_window.argtypes = [_p, _p, _i, _i, _i, _i, _i, _p, _p, _i, _p]
_lib.bsa_route_materialize_workspace_size.restype = ctypes.c_size_t
_lib.bsa_route_materialize_workspace_size.argtypes = [ctypes.POINTER(RouteArgs), ctypes.POINTER(MaterializeArgs)]
_lib.bsa_route_materialize.restype = _i
_lib.bsa_route_materialize.argtypes = [ctypes.POINTER(RouteArgs), ctypes.POINTER(MaterializeArgs), _p,
                                       ctypes.c_size_t, _p]
_lib.bsa_gilbert_tile_index.restype = _i
_lib.bsa_gilbert_tile_index.argtypes = [_i, _i, _i, _i, _i, _i, _p, _p, _p, _p]
_lib.bsa_tile_perm.restype = _i
_lib.bsa_tile_perm.argtypes = [_p, _p, _p, _i, _i, _i, _i, _i64, _i64, _i, _i, _p]
_lib.bsa_tile_block_window.restype = _i
_lib.bsa_tile_block_window.argtypes = [_p, _p, _i, _i, _i, _i, _i, _i, _p, _p, _i, _p]
_lib.bsa_slab_overlap.restype = _i
_lib.bsa_slab_overlap.argtypes = [_p, _i, _p, _p, _p, _i, _i, _p, _p, _p, _i, _i, _i, _p, _i64, _p]
_lib.bsa_slab_coverage.restype = _i
_lib.bsa_slab_coverage.argtypes = [_p, _i, _p, _i, _i, _i, _i, _p, _p, _p, _p, _i, _p, _p, ctypes.c_size_t, _p]
_lib.bsa_slab_coverage_workspace_size.restype = ctypes.c_size_t
_lib.bsa_slab_coverage_workspace_size.argtypes = [_i, _i, _i]
_lib.bsa_diag_mfma_bf16.restype = _i
_lib.bsa_diag_mfma_bf16.argtypes = [_i, _i, _p, _p]
_lib.bsa_route_workspace_size.restype = ctypes.c_size_t
_lib.bsa_route_workspace_size.argtypes = [ctypes.POINTER(RouteArgs)]
_lib.bsa_route_topk.restype = _i
_lib.bsa_route_topk.argtypes = [ctypes.POINTER(RouteArgs), _p, ctypes.c_size_t, _p]
_lib.bsa_route_topk_static.restype = _i
_lib.bsa_route_topk_static.argtypes = [ctypes.POINTER(RouteArgs), _p]
_ATTN_COMMON = [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i64, _i64, _i64, _i64, _p, _p]
_lib.bsa_block_sparse_attn.restype = _i
_lib.bsa_block_sparse_attn.argtypes = _ATTN_COMMON + [_p, _p, _i64, _f, _p]
_lib.bsa_block_sparse_attn_raster.restype = _i
_lib.bsa_block_sparse_attn_raster.argtypes = [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _i64, _i64, _i64, _p,
                                              _i, _i64, _p, _p, _p, _p, _i64, _f, _p]
_lib.bsa_dense_attn.restype = _i
_lib.bsa_dense_attn.argtypes = _ATTN_COMMON + [_f, _p]

EXPORTED = ("bsa_version", "bsa_strerror", "bsa_last_error_detail", "bsa_gilbert_index", "bsa_gilbert_perm",
            "bsa_gilbert_perm_pool", "bsa_gilbert_perm_pool_batch", "bsa_gilbert_block_window",
            "bsa_gilbert_tile_index", "bsa_tile_perm", "bsa_tile_block_window", "bsa_route_workspace_size",
            "bsa_route_topk", "bsa_route_topk_static", "bsa_route_materialize_workspace_size", "bsa_route_materialize", "bsa_slab_overlap",
            "bsa_slab_coverage", "bsa_slab_coverage_workspace_size", "bsa_block_sparse_attn",
            "bsa_block_sparse_attn_raster", "bsa_dense_attn", "bsa_diag_mfma_bf16")


class BsaError(RuntimeError):
    def __init__(self, code: int, detail: str):
        self.code = code
        self.detail = detail
        super().__init__("%s: %s" % (_lib.bsa_strerror(code).decode(), detail))


def _check(code: int) -> None:
    if code != BSA_OK:
        raise BsaError(code, _lib.bsa_last_error_detail().decode())


def version() -> int:
    return _lib.bsa_version()


def library():
    """The loaded ctypes library (for direct C-ABI calls)."""
    return _lib


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BSA_BF16
    if t.dtype == torch.float32:
        return BSA_F32
    raise TypeError("dtype %s: bfloat16 or float32 expected" % t.dtype)


def _need_gpu(*ts):
    for t in ts:
        if isinstance(t, torch.Tensor) and not t.is_cuda:
            raise ValueError("tensors must be on a GPU device")


def _heads_rows(t: torch.Tensor, d: int):
    if t.dim() != 3 or t.shape[2] != d or t.stride(2) != 1 or t.stride(1) != d:
        raise ValueError("expected a [heads][rows][d] tensor with contiguous rows, got shape %s strides %s"
                         % (tuple(t.shape), t.stride()))
    return t.shape[0], t.shape[1], t.stride(0)


def _i32(t: Optional[torch.Tensor], name: str):
    if t is None:
        return None
    if t.dtype != torch.int32 or not t.is_contiguous():
        raise ValueError("%s must be a contiguous int32 tensor" % name)
    return t


# --------------------------------------------------------------------- curve

def gilbert_index(T: int, H: int, W: int, device="cuda", stream=None, with_inverse=True):
    """Gilbert order of a T x H x W grid: ``(perm, inv)`` int32 tensors."""
    n = T * H * W
    perm = torch.empty(n, dtype=torch.int32, device=device)
    inv = torch.empty(n, dtype=torch.int32, device=device) if with_inverse else None
    _check(_lib.bsa_gilbert_index(T, H, W, _ptr(perm), _ptr(inv), _stream(stream)))
    return perm, inv


def gilbert_perm(src: torch.Tensor, perm: torch.Tensor, *, block: int, inverse: bool = False,
                 dst: Optional[torch.Tensor] = None, L: Optional[int] = None, stream=None):
    """Raster ``[L][heads][d]`` -> Gilbert ``[heads][n_blocks*block][d]``
    (``inverse=False``) or back.  ``dst`` may be a head-strided view (e.g. a
    chunk slot of a KV store); it is allocated when omitted."""
    _need_gpu(src, perm, dst)
    perm = _i32(perm, "perm")
    if not inverse:
        L_, heads, d = src.shape
        if src.stride(2) != 1 or src.stride(1) != d:
            raise ValueError("raster src must have contiguous [heads][d] per token")
        rows = -(-L_ // block) * block
        if dst is None:
            dst = torch.empty((heads, rows, d), dtype=src.dtype, device=src.device)
        _, drows, ghs = _heads_rows(dst, d)
        if drows < rows:
            raise ValueError("dst holds %d rows per head, %d needed" % (drows, rows))
        rts = src.stride(0)
        _check(_lib.bsa_gilbert_perm(_ptr(src), _ptr(dst), _ptr(perm), L_, heads, d, block, rts, ghs, 0,
                                     _dtype_code(src), _stream(stream)))
        return dst
    heads, rows, ghs = _heads_rows(src, src.shape[2])
    d = src.shape[2]
    L_ = perm.numel() if L is None else L
    if dst is None:
        dst = torch.empty((L_, heads, d), dtype=src.dtype, device=src.device)
    if dst.stride(2) != 1 or dst.stride(1) != d:
        raise ValueError("raster dst must have contiguous [heads][d] per token")
    _check(_lib.bsa_gilbert_perm(_ptr(src), _ptr(dst), _ptr(perm), L_, heads, d, block, dst.stride(0), ghs, 1,
                                 _dtype_code(src), _stream(stream)))
    return dst


def gilbert_perm_pool(src: torch.Tensor, perm: torch.Tensor, *, block: int, dst: Optional[torch.Tensor] = None,
                      pool: Optional[torch.Tensor] = None, pool_only: bool = False, stream=None):
    """Raster ``[L][heads][d]`` -> Gilbert ``[heads][n_blocks*block][d]``
    like ``gilbert_perm``, plus the float64 block means of the valid rows
    into ``pool`` ``[heads][>= n_blocks][d]`` (a head-strided view such as
    a slice of a pooled-key cache is fine).  ``pool_only``: the block means
    alone (nothing permuted; ``dst`` is None).  Returns ``(dst, pool)``."""
    _need_gpu(src, perm, dst, pool)
    perm = _i32(perm, "perm")
    L_, heads, d = src.shape
    if src.stride(2) != 1 or src.stride(1) != d:
        raise ValueError("raster src must have contiguous [heads][d] per token")
    nb = -(-L_ // block)
    ghs = 0
    if pool_only:
        if dst is not None:
            raise ValueError("pool_only takes no dst")
    else:
        if dst is None:
            dst = torch.empty((heads, nb * block, d), dtype=src.dtype, device=src.device)
        _, drows, ghs = _heads_rows(dst, d)
        if drows < nb * block:
            raise ValueError("dst holds %d rows per head, %d needed" % (drows, nb * block))
    if pool is None:
        pool = torch.empty((heads, nb, d), dtype=torch.float64, device=src.device)
    if pool.dtype != torch.float64 or pool.dim() != 3 or pool.shape[0] != heads or pool.shape[1] < nb \
            or pool.shape[2] != d or pool.stride(2) != 1 or pool.stride(1) != d:
        raise ValueError("pool must be float64 [heads][>= n_blocks][d] with contiguous blocks")
    _check(_lib.bsa_gilbert_perm_pool(_ptr(src), _ptr(dst), _ptr(perm), L_, heads, d, block, src.stride(0), ghs,
                                      _dtype_code(src), _ptr(pool), pool.stride(0), _stream(stream)))
    return dst, pool


def gilbert_perm_pool_batch(jobs, perm: torch.Tensor, *, block: int, stream=None):
    """Several raster tensors of one chunk through one launch: ``jobs`` is a
    list of ``(src, dst, pool)`` with ``src`` raster ``[L][heads][d]`` (the
    same shape and dtype for every job), ``dst`` a Gilbert
    ``[heads][>= n_blocks*block][d]`` view or None (block means only) and
    ``pool`` a float64 ``[heads][>= n_blocks][d]`` view or None (the
    permutation only); a job needs one of them.  Each job's results equal
    ``gilbert_perm_pool`` (or ``gilbert_perm``) on it alone.  Returns
    ``jobs``."""
    if not 1 <= len(jobs) <= MAX_PERM_JOBS:
        raise ValueError("1 to %d jobs, got %d" % (MAX_PERM_JOBS, len(jobs)))
    _need_gpu(perm, *[t for job in jobs for t in job])
    perm = _i32(perm, "perm")
    shape, dtype = jobs[0][0].shape, jobs[0][0].dtype
    L_, heads, d = shape
    nb = -(-L_ // block)
    arr = (PermJob * len(jobs))()
    for z, (src, dst, pool) in enumerate(jobs):
        if src.shape != shape or src.dtype != dtype:
            raise ValueError("job %d: every src must have the shape and dtype of the first" % z)
        if src.stride(2) != 1 or src.stride(1) != d:
            raise ValueError("job %d: raster src must have contiguous [heads][d] per token" % z)
        if dst is None and pool is None:
            raise ValueError("job %d: needs a dst or a pool" % z)
        ghs = 0
        if dst is not None:
            _, drows, ghs = _heads_rows(dst, d)
            if drows < nb * block or dst.dtype != dtype:
                raise ValueError("job %d: dst must be %s with >= %d rows per head" % (z, dtype, nb * block))
        if pool is not None and (pool.dtype != torch.float64 or pool.dim() != 3 or pool.shape[0] != heads
                                 or pool.shape[1] < nb or pool.shape[2] != d or pool.stride(2) != 1
                                 or pool.stride(1) != d):
            raise ValueError("job %d: pool must be float64 [heads][>= n_blocks][d] with contiguous blocks" % z)
        arr[z] = PermJob(_ptr(src), _ptr(dst) if dst is not None else None, src.stride(0), ghs,
                         _ptr(pool) if pool is not None else None, pool.stride(0) if pool is not None else 0)
    _check(_lib.bsa_gilbert_perm_pool_batch(arr, len(jobs), _ptr(perm), L_, heads, d, block,
                                            _dtype_code(jobs[0][0]), _stream(stream)))
    return jobs


def gilbert_block_window(perm: torch.Tensor, inv: torch.Tensor, grid, *, block: int, q_chunk: int,
                         out=None, stream=None):
    """Local window of every query block of chunk ``q_chunk``: ``(window,
    window_len)`` with ``window`` int32 ``[n_blocks][2*n_blocks]`` (row b's
    first ``window_len[b]`` entries are its absolute KV block indices,
    ascending)."""
    _need_gpu(perm, inv)
    perm, inv = _i32(perm, "perm"), _i32(inv, "inv")
    T, H, W = grid
    nbc = -(-(T * H * W) // block)
    if out is None:
        out = (torch.empty((nbc, 2 * nbc), dtype=torch.int32, device=perm.device),
               torch.empty(nbc, dtype=torch.int32, device=perm.device))
    window, window_len = out
    if window.dtype != torch.int32 or window.dim() != 2 or window.stride(1) != 1 or window.shape[0] < nbc:
        raise ValueError("window must be int32 [n_blocks][stride] with contiguous rows")
    _check(_lib.bsa_gilbert_block_window(_ptr(perm), _ptr(inv), T, H, W, block, q_chunk, _ptr(window),
                                         _ptr(_i32(window_len, "window_len")), window.stride(0), _stream(stream)))
    return window, window_len


def tile_grid(grid, tile):
    """Tiles along each axis of a chunk grid."""
    return tuple(-(-g // t) for g, t in zip(grid, tile))


def gilbert_tile_index(T: int, H: int, W: int, tile, device="cuda", stream=None, with_cell_row=True):
    """Fixed 3-D tile layout of a chunk: ``(row_cell, block_len, cell_row)``
    int32 tensors (``row_cell[r]`` = raster cell of row r, -1 for padding)."""
    tt, th, tw = tile
    n_tiles = 1
    for x in tile_grid((T, H, W), tile):
        n_tiles *= x
    row_cell = torch.empty(n_tiles * tt * th * tw, dtype=torch.int32, device=device)
    block_len = torch.empty(n_tiles, dtype=torch.int32, device=device)
    cell_row = torch.empty(T * H * W, dtype=torch.int32, device=device) if with_cell_row else None
    _check(_lib.bsa_gilbert_tile_index(T, H, W, tt, th, tw, _ptr(row_cell), _ptr(block_len), _ptr(cell_row),
                                       _stream(stream)))
    return row_cell, block_len, cell_row


def tile_perm(src: torch.Tensor, row_cell: torch.Tensor, *, inverse: bool = False,
              dst: Optional[torch.Tensor] = None, L: Optional[int] = None, stream=None):
    """Raster ``[L][heads][d]`` -> tiled ``[heads][n_rows][d]``
    (``inverse=False``) or back, through the tile layout's ``row_cell``."""
    _need_gpu(src, row_cell, dst)
    row_cell = _i32(row_cell, "row_cell")
    n_rows = row_cell.numel()
    if not inverse:
        L_, heads, d = src.shape
        if src.stride(2) != 1 or src.stride(1) != d:
            raise ValueError("raster src must have contiguous [heads][d] per token")
        if dst is None:
            dst = torch.empty((heads, n_rows, d), dtype=src.dtype, device=src.device)
        _, drows, ths = _heads_rows(dst, d)
        if drows < n_rows:
            raise ValueError("dst holds %d rows per head, %d needed" % (drows, n_rows))
        _check(_lib.bsa_tile_perm(_ptr(src), _ptr(dst), _ptr(row_cell), n_rows, L_, heads, d, src.stride(0), ths, 0,
                                  _dtype_code(src), _stream(stream)))
        return dst
    d = src.shape[2]
    heads, _, ths = _heads_rows(src, d)
    if L is None:
        raise ValueError("L (tokens of the chunk) is required for the inverse permutation")
    if dst is None:
        dst = torch.empty((L, heads, d), dtype=src.dtype, device=src.device)
    if dst.stride(2) != 1 or dst.stride(1) != d:
        raise ValueError("raster dst must have contiguous [heads][d] per token")
    _check(_lib.bsa_tile_perm(_ptr(src), _ptr(dst), _ptr(row_cell), n_rows, L, heads, d, dst.stride(0), ths, 1,
                              _dtype_code(src), _stream(stream)))
    return dst


def tile_block_window(row_cell: torch.Tensor, cell_row: torch.Tensor, grid, *, block: int, q_chunk: int, out=None,
                      stream=None):
    """Local window of every tile block of chunk ``q_chunk``: ``(window,
    window_len)`` as ``gilbert_block_window``."""
    _need_gpu(row_cell, cell_row)
    row_cell, cell_row = _i32(row_cell, "row_cell"), _i32(cell_row, "cell_row")
    T, H, W = grid
    n_rows = row_cell.numel()
    nbc = n_rows // block
    if out is None:
        out = (torch.empty((nbc, 2 * nbc), dtype=torch.int32, device=row_cell.device),
               torch.empty(nbc, dtype=torch.int32, device=row_cell.device))
    window, window_len = out
    if window.dtype != torch.int32 or window.dim() != 2 or window.stride(1) != 1 or window.shape[0] < nbc:
        raise ValueError("window must be int32 [n_blocks][stride] with contiguous rows")
    _check(_lib.bsa_tile_block_window(_ptr(row_cell), _ptr(cell_row), n_rows, T, H, W, block, q_chunk, _ptr(window),
                                      _ptr(_i32(window_len, "window_len")), window.stride(0), _stream(stream)))
    return window, window_len


# --------------------------------------------------------------------- geometry

def _f64(t: Optional[torch.Tensor], name: str, cols: Optional[int] = None):
    if t is None:
        return None
    if t.dtype != torch.float64 or not t.is_contiguous() or (cols is not None and (t.dim() != 2 or t.shape[1] != cols)):
        raise ValueError("%s must be a contiguous float64 tensor%s" % (name, "" if cols is None else
                                                                        " of shape [n][%d]" % cols))
    return t


def slab_overlap(cams, q_slab_ptr, q_slab_cam, q_slab_geom, h_slab_ptr, h_slab_cam, h_slab_geom, *,
                 grid_n: int = 8, out: Optional[torch.Tensor] = None, stream=None):
    """Overlap ``[nqb][nkb]`` float32 of query blocks with historical blocks
    from their frustum slabs (CSR per block: ``*_ptr``, ``*_cam``,
    ``*_geom`` float64 ``[n][6]``)."""
    _need_gpu(cams, q_slab_ptr, q_slab_cam, q_slab_geom, h_slab_ptr, h_slab_cam, h_slab_geom, out)
    cams = _f64(cams, "cams", 16)
    q_slab_geom, h_slab_geom = _f64(q_slab_geom, "q_slab_geom", 6), _f64(h_slab_geom, "h_slab_geom", 6)
    q_slab_ptr, h_slab_ptr = _i32(q_slab_ptr, "q_slab_ptr"), _i32(h_slab_ptr, "h_slab_ptr")
    q_slab_cam, h_slab_cam = _i32(q_slab_cam, "q_slab_cam"), _i32(h_slab_cam, "h_slab_cam")
    nqb, nkb = q_slab_ptr.numel() - 1, h_slab_ptr.numel() - 1
    if out is None:
        out = torch.empty((nqb, nkb), dtype=torch.float32, device=cams.device)
    if out.dtype != torch.float32 or out.dim() != 2 or out.stride(1) != 1:
        raise ValueError("out must be float32 [nqb][stride] with contiguous rows")
    _check(_lib.bsa_slab_overlap(_ptr(cams), cams.shape[0], _ptr(q_slab_ptr), _ptr(q_slab_cam), _ptr(q_slab_geom),
                                 nqb, q_slab_cam.numel(), _ptr(h_slab_ptr), _ptr(h_slab_cam), _ptr(h_slab_geom), nkb,
                                 h_slab_cam.numel(), grid_n, _ptr(out), out.stride(0), _stream(stream)))
    return out


def slab_coverage(cams, perm, grid, frame_cam, depth, h_slab_cam, h_slab_geom, *, block: int,
                  out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None, stream=None):
    """Coverage ``[ceil(T*H*W / block)]`` float32 of the query blocks of a
    chunk by the historical slabs.  ``workspace`` (uint8, at least
    ``bsa_slab_coverage_workspace_size`` bytes) may be passed in to avoid an
    allocation."""
    _need_gpu(cams, perm, frame_cam, depth, h_slab_cam, h_slab_geom, out)
    cams = _f64(cams, "cams", 16)
    h_slab_geom = _f64(h_slab_geom, "h_slab_geom", 6)
    T, H, W = grid
    if depth.dtype != torch.float32 or not depth.is_contiguous() or depth.numel() != T * H * W:
        raise ValueError("depth must be a contiguous float32 raster of T*H*W values")
    nqb = -(-(T * H * W) // block)
    if out is None:
        out = torch.empty(nqb, dtype=torch.float32, device=cams.device)
    need = _lib.bsa_slab_coverage_workspace_size(T, H, W)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 4), dtype=torch.uint8, device=cams.device)
    _check(_lib.bsa_slab_coverage(_ptr(cams), cams.shape[0], _ptr(_i32(perm, "perm")), T, H, W, block,
                                  _ptr(_i32(frame_cam, "frame_cam")), _ptr(depth),
                                  _ptr(_i32(h_slab_cam, "h_slab_cam")), _ptr(h_slab_geom),
                                  h_slab_cam.numel(), _ptr(out), _ptr(workspace), workspace.numel(),
                                  _stream(stream)))
    return out


# --------------------------------------------------------------------- router
# --------------------------------------------------------------------- router

def _route_args(q, k, *, block, nqb, nkb, q_block_len, kv_block_len, scale, overlap, lam, g_ref, tau,
                k_fixed, k_per_row, k_max, n_dense_tail_blocks, kpool, kpool_valid_blocks,
                row_ptr, col_idx, fallback_counts, sel_keys, qpool=None):
    d = q.shape[2]
    heads, _, qhs = _heads_rows(q, d)
    _, _, khs = _heads_rows(k, d)
    a = RouteArgs()
    a.struct_size = ctypes.sizeof(RouteArgs)
    a.q, a.k, a.dtype = q.data_ptr(), k.data_ptr(), _dtype_code(q)
    a.heads, a.d, a.block, a.nqb, a.nkb = heads, d, block, nqb, nkb
    a.q_head_stride, a.k_head_stride = qhs, khs
    a.q_block_len = None if q_block_len is None else q_block_len.data_ptr()
    a.kv_block_len = None if kv_block_len is None else kv_block_len.data_ptr()
    a.scale = float(scale)
    if overlap is not None:
        if overlap.dtype != torch.float32 or overlap.stride(1) != 1:
            raise ValueError("overlap must be float32 with contiguous rows")
        a.overlap, a.overlap_row_stride = overlap.data_ptr(), overlap.stride(0)
    a.lam, a.g_ref, a.tau = float(lam), float(g_ref), float(tau)
    a.k_fixed = int(k_fixed)
    a.k_per_row = None if k_per_row is None else k_per_row.data_ptr()
    a.k_max = int(k_max) if k_max is not None else int(k_fixed)
    a.n_dense_tail_blocks = int(n_dense_tail_blocks)
    if kpool is not None:
        if kpool.dtype != torch.float64 or kpool.dim() != 3 or kpool.shape[2] != d or kpool.stride(2) != 1 \
                or kpool.stride(1) != d or kpool.stride(0) % d:
            raise ValueError("kpool must be float64 [heads][blocks][d] with contiguous blocks")
        if kpool.shape[0] != heads or kpool.shape[1] < nkb - n_dense_tail_blocks:
            raise ValueError("kpool must hold heads x (nkb - n_dense_tail_blocks) pooled keys")
        a.kpool, a.kpool_head_blocks = kpool.data_ptr(), kpool.stride(0) // d
    a.kpool_valid_blocks = int(kpool_valid_blocks)
    if row_ptr is not None:
        a.row_ptr, a.col_idx, a.col_capacity = row_ptr.data_ptr(), col_idx.data_ptr(), col_idx.numel()
    a.fallback_counts = None if fallback_counts is None else fallback_counts.data_ptr()
    a.sel_keys = None if sel_keys is None else sel_keys.data_ptr()
    if qpool is not None:
        if qpool.dtype != torch.float64 or qpool.dim() != 3 or qpool.shape[2] != d or qpool.stride(2) != 1 \
                or qpool.stride(1) != d or qpool.shape[0] != heads or qpool.shape[1] < nqb:
            raise ValueError("qpool must be float64 [heads][>= nqb][d] with contiguous blocks")
        a.qpool, a.qpool_head_stride = qpool.data_ptr(), qpool.stride(0)
    return a


def route_capacity(heads: int, nqb: int, nkb: int, k_cap: int, n_dense_tail_blocks: int = 0) -> int:
    """Entries ``col_idx`` must hold."""
    n_cand = nkb - n_dense_tail_blocks
    return heads * nqb * (min(k_cap, n_cand) + n_dense_tail_blocks)


def _route_topk_args(q, k, *, block, nqb, nkb, scale, q_block_len, kv_block_len, overlap, lam, g_ref, tau,
                     k_fixed, k_per_row, k_max, n_dense_tail_blocks, kpool, kpool_valid_blocks, qpool, want_keys,
                     out):
    _need_gpu(q, k, q_block_len, kv_block_len, overlap, k_per_row, kpool, qpool)
    heads = q.shape[0]
    n_cand = nkb - n_dense_tail_blocks
    k_cap = k_max if k_per_row is not None else k_fixed
    if k_per_row is not None and k_max is None:
        raise ValueError("k_max is required with k_per_row")
    dev = q.device
    if out is None:
        out = {
            "row_ptr": torch.empty(heads * nqb + 1, dtype=torch.int32, device=dev),
            "col_idx": torch.empty(max(1, route_capacity(heads, nqb, nkb, k_cap, n_dense_tail_blocks)),
                                   dtype=torch.int32, device=dev),
            "fallback_counts": torch.zeros(2, dtype=torch.int32, device=dev),
            "sel_keys": torch.empty((heads, nqb, n_cand), dtype=torch.float64, device=dev) if want_keys else None,
        }
    a = _route_args(q, k, block=block, nqb=nqb, nkb=nkb, q_block_len=_i32(q_block_len, "q_block_len"),
                    kv_block_len=_i32(kv_block_len, "kv_block_len"), scale=scale, overlap=overlap, lam=lam,
                    g_ref=g_ref, tau=tau, k_fixed=k_fixed, k_per_row=_i32(k_per_row, "k_per_row"), k_max=k_max,
                    n_dense_tail_blocks=n_dense_tail_blocks, kpool=kpool, kpool_valid_blocks=kpool_valid_blocks,
                    row_ptr=out["row_ptr"], col_idx=out["col_idx"], fallback_counts=out["fallback_counts"],
                    sel_keys=out.get("sel_keys"), qpool=qpool)
    return a, out


def route_topk(q: torch.Tensor, k: torch.Tensor, *, block: int, nqb: int, nkb: int, scale: float,
               q_block_len=None, kv_block_len=None, overlap=None, lam: float = 2.0, g_ref: float = 0.2,
               tau: float = 0.1, k_fixed: int = 50, k_per_row=None, k_max: Optional[int] = None,
               n_dense_tail_blocks: int = 0, kpool=None, kpool_valid_blocks: int = 0, qpool=None,
               want_keys: bool = False, out: Optional[dict] = None, workspace=None, stream=None):
    """Pool, score, fuse and select.  Returns a dict with ``row_ptr``,
    ``col_idx`` (capacity-sized; the first ``row_ptr[-1]`` entries are the
    lists), ``fallback_counts`` and optionally ``sel_keys``.  ``out`` and
    ``workspace`` may be passed in to avoid allocations.  ``qpool``: the
    pooled queries (``gilbert_perm_pool``), so ``q`` is not pooled again."""
    a, out = _route_topk_args(q, k, block=block, nqb=nqb, nkb=nkb, scale=scale, q_block_len=q_block_len,
                              kv_block_len=kv_block_len, overlap=overlap, lam=lam, g_ref=g_ref, tau=tau,
                              k_fixed=k_fixed, k_per_row=k_per_row, k_max=k_max,
                              n_dense_tail_blocks=n_dense_tail_blocks, kpool=kpool,
                              kpool_valid_blocks=kpool_valid_blocks, qpool=qpool, want_keys=want_keys, out=out)
    need = _lib.bsa_route_workspace_size(ctypes.byref(a))
    if need == 0:
        _check(_lib.bsa_route_topk(ctypes.byref(a), None, 0, _stream(stream)))
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    out["workspace"] = workspace
    _check(_lib.bsa_route_topk(ctypes.byref(a), _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


ROUTE_STATIC_SCRATCH_BYTES = 32 << 20  # BSA_ROUTE_STATIC_SCRATCH_BYTES


def route_topk_static(q: torch.Tensor, k: torch.Tensor, *, block: int, nqb: int, nkb: int, scale: float,
                      out: dict, q_block_len=None, kv_block_len=None, overlap=None, lam: float = 2.0,
                      g_ref: float = 0.2, tau: float = 0.1, k_fixed: int = 50, k_per_row=None,
                      k_max: Optional[int] = None, n_dense_tail_blocks: int = 0, kpool=None,
                      kpool_valid_blocks: int = 0, qpool=None, stream=None):
    """``route_topk`` through ``bsa_route_topk_static``: the library's fixed
    per-GPU scratch instead of a workspace, so the call allocates nothing.
    ``out`` (``row_ptr``, ``col_idx``, ``fallback_counts`` and optionally
    ``sel_keys``) is required.  Calls that overlap on one GPU race on the
    shared scratch."""
    for name in ("row_ptr", "col_idx", "fallback_counts"):
        if out.get(name) is None:
            raise ValueError("out[%r] is required" % name)
    a, out = _route_topk_args(q, k, block=block, nqb=nqb, nkb=nkb, scale=scale, q_block_len=q_block_len,
                              kv_block_len=kv_block_len, overlap=overlap, lam=lam, g_ref=g_ref, tau=tau,
                              k_fixed=k_fixed, k_per_row=k_per_row, k_max=k_max,
                              n_dense_tail_blocks=n_dense_tail_blocks, kpool=kpool,
                              kpool_valid_blocks=kpool_valid_blocks, qpool=qpool, want_keys=False, out=out)
    _check(_lib.bsa_route_topk_static(ctypes.byref(a), _stream(stream)))
    return out


def route_workspace_size(q, k, **kw) -> int:
    """Workspace bytes ``route_topk`` needs for these arguments."""
    a = _route_args(q, k, row_ptr=None, col_idx=None, fallback_counts=None, sel_keys=None, **kw)
    return _lib.bsa_route_workspace_size(ctypes.byref(a))


def _materialize_args(coverage, eta_cov, k_cov, k_unc, mass, prev_blocks, window, window_len, ref_blocks):
    m = MaterializeArgs()
    m.struct_size = ctypes.sizeof(MaterializeArgs)
    if coverage is not None:
        if coverage.dtype != torch.float32 or not coverage.is_contiguous():
            raise ValueError("coverage must be a contiguous float32 tensor")
        m.coverage = coverage.data_ptr()
    m.eta_cov, m.k_cov, m.k_unc, m.mass = float(eta_cov), int(k_cov), int(k_unc), float(mass)
    m.prev_begin, m.prev_end = int(prev_blocks[0]), int(prev_blocks[1])
    if window is not None:
        if window.dtype != torch.int32 or window.dim() != 2 or window.stride(1) != 1:
            raise ValueError("window must be int32 [nqb][stride] with contiguous rows")
        m.window, m.window_len, m.window_stride = (window.data_ptr(), _i32(window_len, "window_len").data_ptr(),
                                                   window.stride(0))
    m.ref_begin, m.ref_end = int(ref_blocks[0]), int(ref_blocks[1])
    return m


def materialize_capacity(heads: int, nqb: int, nkb: int, *, k_cov: int, k_unc: int, prev_blocks=(0, 0),
                         window_stride: int = 0, ref_blocks=(0, 0)) -> int:
    """Entries ``col_idx`` must hold for ``route_materialize``."""
    clip = lambda x: min(int(x), nkb)
    per_row = max(clip(prev_blocks[1]) - clip(prev_blocks[0]), k_cov, k_unc) + window_stride \
        + clip(ref_blocks[1]) - clip(ref_blocks[0])
    return heads * nqb * min(nkb, per_row)


def route_materialize(q: torch.Tensor, k: torch.Tensor, *, block: int, nqb: int, nkb: int, scale: float,
                      q_block_len=None, kv_block_len=None, overlap=None, lam: float = 2.0, g_ref: float = 0.2,
                      tau: float = 0.1, coverage=None, eta_cov: float = 0.9, k_cov: int = 80, k_unc: int = 150,
                      mass: float = 0.9, prev_blocks=(0, 0), window=None, window_len=None, ref_blocks=(0, 0),
                      kpool=None, kpool_valid_blocks: int = 0, qpool=None, want_keys: bool = False,
                      out: Optional[dict] = None, workspace=None, stream=None):
    """Materialised routes: coverage-gated budgets, the previous chunk's
    reservation, the cumulative-mass prefix, the local window and the
    reference blocks.  Returns a dict with ``row_ptr`` and ``col_idx``
    (capacity-sized; the first ``row_ptr[-1]`` entries are the lists) and
    optionally ``sel_keys``.  ``qpool`` as in ``route_topk``."""
    _need_gpu(q, k, q_block_len, kv_block_len, overlap, coverage, window, window_len, kpool, qpool)
    heads = q.shape[0]
    dev = q.device
    wstride = 0 if window is None else window.stride(0)
    if out is None:
        cap = materialize_capacity(heads, nqb, nkb, k_cov=k_cov, k_unc=k_unc, prev_blocks=prev_blocks,
                                   window_stride=wstride, ref_blocks=ref_blocks)
        out = {
            "row_ptr": torch.empty(heads * nqb + 1, dtype=torch.int32, device=dev),
            "col_idx": torch.empty(max(1, cap), dtype=torch.int32, device=dev),
            "sel_keys": torch.empty((heads, nqb, nkb), dtype=torch.float64, device=dev) if want_keys else None,
        }
    a = _route_args(q, k, block=block, nqb=nqb, nkb=nkb, q_block_len=_i32(q_block_len, "q_block_len"),
                    kv_block_len=_i32(kv_block_len, "kv_block_len"), scale=scale, overlap=overlap, lam=lam,
                    g_ref=g_ref, tau=tau, k_fixed=0, k_per_row=None, k_max=0, n_dense_tail_blocks=0, kpool=kpool,
                    kpool_valid_blocks=kpool_valid_blocks, row_ptr=out["row_ptr"], col_idx=out["col_idx"],
                    fallback_counts=None, sel_keys=out.get("sel_keys"), qpool=qpool)
    m = _materialize_args(coverage, eta_cov, k_cov, k_unc, mass, prev_blocks, window, window_len, ref_blocks)
    need = _lib.bsa_route_materialize_workspace_size(ctypes.byref(a), ctypes.byref(m))
    if need == 0:
        _check(_lib.bsa_route_materialize(ctypes.byref(a), ctypes.byref(m), None, 0, _stream(stream)))
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    out["workspace"] = workspace
    _check(_lib.bsa_route_materialize(ctypes.byref(a), ctypes.byref(m), _ptr(workspace), workspace.numel(),
                                      _stream(stream)))
    return out


def route_materialize_workspace_size(q, k, *, block, nqb, nkb, scale, q_block_len=None, kv_block_len=None,
                                     overlap=None, coverage=None, eta_cov=0.9, k_cov=80, k_unc=150, mass=0.9,
                                     prev_blocks=(0, 0), window=None, window_len=None, ref_blocks=(0, 0),
                                     kpool=None, kpool_valid_blocks=0, col_capacity=None) -> int:
    """Workspace bytes ``route_materialize`` needs for these arguments."""
    a = _route_args(q, k, block=block, nqb=nqb, nkb=nkb, q_block_len=q_block_len, kv_block_len=kv_block_len,
                    scale=scale, overlap=overlap, lam=2.0, g_ref=0.2, tau=0.1, k_fixed=0, k_per_row=None, k_max=0,
                    n_dense_tail_blocks=0, kpool=kpool, kpool_valid_blocks=kpool_valid_blocks, row_ptr=None,
                    col_idx=None, fallback_counts=None, sel_keys=None)
    a.row_ptr, a.col_idx = 1, 1
    wstride = 0 if window is None else window.stride(0)
    a.col_capacity = col_capacity if col_capacity is not None else materialize_capacity(
        q.shape[0], nqb, nkb, k_cov=k_cov, k_unc=k_unc, prev_blocks=prev_blocks, window_stride=wstride,
        ref_blocks=ref_blocks)
    m = _materialize_args(coverage, eta_cov, k_cov, k_unc, mass, prev_blocks, window, window_len, ref_blocks)
    return _lib.bsa_route_materialize_workspace_size(ctypes.byref(a), ctypes.byref(m))


# --------------------------------------------------------------------- attention

def _attn_prep(q, k, v, out, lse, block):
    _need_gpu(q, k, v, out, lse)
    d = q.shape[2]
    heads, qrows, qhs = _heads_rows(q, d)
    _, krows, khs = _heads_rows(k, d)
    _, vrows, vhs = _heads_rows(v, d)
    if k.shape[0] != heads or v.shape[0] != heads or vrows < krows:
        raise ValueError("q, k, v head counts / rows disagree")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("k and v must have q's dtype (%s), got %s and %s" % (q.dtype, k.dtype, v.dtype))
    if qrows % block or krows % block:
        raise ValueError("row counts must be multiples of the block size")
    if out is None:
        out = torch.empty((heads, qrows, d), dtype=q.dtype, device=q.device)
    _, orows, ohs = _heads_rows(out, d)
    if out.dtype != q.dtype:
        raise ValueError("out must have q's dtype (%s), got %s" % (q.dtype, out.dtype))
    if out.shape[0] != heads or orows < qrows:
        raise ValueError("out must hold %d heads x %d rows" % (heads, qrows))
    lse = _lse_arg(lse, heads, qrows, q.device)
    return d, heads, qrows // block, krows // block, qhs, khs, vhs, out, ohs, lse


def _lse_arg(lse, heads, qrows, device):
    if lse is True:
        return torch.empty((heads, qrows), dtype=torch.float32, device=device)
    if lse is not None:
        if lse.dtype != torch.float32 or not lse.is_contiguous():
            raise ValueError("lse must be a contiguous float32 tensor")
        if lse.numel() < heads * qrows:
            raise ValueError("lse holds %d values, heads*nqb*block = %d needed" % (lse.numel(), heads * qrows))
    return lse


def _attn_sizes(heads, nqb, nkb, nkb_rows, q_block_len, kv_block_len, row_ptr=None):
    """Sizes the C ABI cannot see: every device array must cover what the
    kernels read from it."""
    if nkb < 1 or nkb > nkb_rows:
        raise ValueError("nkb = %d outside [1, %d] (the KV rows / block)" % (nkb, nkb_rows))
    if q_block_len is not None and q_block_len.numel() < nqb:
        raise ValueError("q_block_len holds %d entries, nqb = %d needed" % (q_block_len.numel(), nqb))
    if kv_block_len is not None and kv_block_len.numel() < nkb:
        raise ValueError("kv_block_len holds %d entries, nkb = %d needed" % (kv_block_len.numel(), nkb))
    if row_ptr is not None and row_ptr.numel() < heads * nqb + 1:
        raise ValueError("row_ptr holds %d entries, heads*nqb+1 = %d needed" % (row_ptr.numel(), heads * nqb + 1))


def block_sparse_attn(q, k, v, row_ptr, col_idx, *, block: int, scale: Optional[float] = None,
                      q_block_len=None, kv_block_len=None, out=None, lse=None, nkb: Optional[int] = None,
                      stream=None):
    """Attention of every (head, query block) over its listed KV blocks.
    ``lse=True`` allocates and returns the log-sum-exp.  Returns ``(O, LSE)``."""
    _need_gpu(row_ptr, col_idx)
    d, heads, nqb, nkb_, qhs, khs, vhs, out, ohs, lse = _attn_prep(q, k, v, out, lse, block)
    nkb = nkb_ if nkb is None else nkb
    _attn_sizes(heads, nqb, nkb, nkb_, q_block_len, kv_block_len, row_ptr)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    _check(_lib.bsa_block_sparse_attn(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _dtype_code(q), heads, d, block, nqb, nkb, qhs, khs,
        vhs, ohs, _ptr(_i32(q_block_len, "q_block_len")), _ptr(_i32(kv_block_len, "kv_block_len")),
        _ptr(_i32(row_ptr, "row_ptr")), _ptr(_i32(col_idx, "col_idx")), col_idx.numel(), scale,
        _stream(stream)))
    return out, lse


def block_sparse_attn_raster(q, k, v, row_ptr, col_idx, row_map, *, block: int, scale: Optional[float] = None,
                             q_block_len=None, kv_block_len=None, out=None, tokens: Optional[int] = None, lse=None,
                             nkb: Optional[int] = None, q_raster: bool = False, nqb: Optional[int] = None,
                             stream=None):
    """``block_sparse_attn`` with the output written in raster token order:
    query row g goes to token ``row_map[g]`` of ``out`` ``[tokens][heads][d]``
    (negative entries: padding, not written).  With ``q_raster`` the queries
    are raster ``[tokens][heads][d]`` too, row g read from token
    ``row_map[g]`` (``nqb`` query blocks: given, or the length of
    ``q_block_len``).  ``tokens`` defaults to ``row_map.numel()`` when
    ``out`` is allocated here.  Returns ``(O, LSE)`` (LSE in the blocked
    layout)."""
    _need_gpu(row_ptr, col_idx, row_map, out)
    row_map = _i32(row_map, "row_map")
    if q_raster:
        _need_gpu(q, k, v, lse)
        heads, d = k.shape[0], k.shape[2]
        if q.dim() != 3 or q.shape[1] != heads or q.shape[2] != d or q.stride(2) != 1 or q.stride(1) != d:
            raise ValueError("raster q must be [tokens][heads][d] with contiguous [heads][d] per token")
        if nqb is None:
            if q_block_len is None:
                raise ValueError("raster q needs nqb or q_block_len")
            nqb = q_block_len.numel()
        _, krows, khs = _heads_rows(k, d)
        _, vrows, vhs = _heads_rows(v, d)
        if v.shape[0] != heads or vrows < krows or krows % block:
            raise ValueError("k, v head counts / rows disagree")
        if k.dtype != q.dtype or v.dtype != q.dtype:
            raise ValueError("k and v must have q's dtype (%s), got %s and %s" % (q.dtype, k.dtype, v.dtype))
        nkb_, qs = krows // block, q.stride(0)
        lse = _lse_arg(lse, heads, nqb * block, q.device)
    else:
        d, heads, nqb, nkb_, qs, khs, vhs, _, _, lse = _attn_prep(q, k, v, q, lse, block)
    nkb = nkb_ if nkb is None else nkb
    _attn_sizes(heads, nqb, nkb, nkb_, q_block_len, kv_block_len, row_ptr)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    if out is None:
        out = torch.empty((row_map.numel() if tokens is None else tokens, heads, d), dtype=q.dtype, device=q.device)
    if out.dim() != 3 or out.shape[1] != heads or out.shape[2] != d or out.stride(2) != 1 or out.stride(1) != d:
        raise ValueError("raster out must be [tokens][heads][d] with contiguous [heads][d] per token")
    if out.dtype != q.dtype:
        raise ValueError("out must have q's dtype (%s), got %s" % (q.dtype, out.dtype))
    _check(_lib.bsa_block_sparse_attn_raster(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _dtype_code(q), heads, d, block, nqb, nkb,
        1 if q_raster else 0, qs, khs, vhs, _ptr(row_map), row_map.numel(), out.stride(0),
        _ptr(_i32(q_block_len, "q_block_len")), _ptr(_i32(kv_block_len, "kv_block_len")),
        _ptr(_i32(row_ptr, "row_ptr")), _ptr(_i32(col_idx, "col_idx")), col_idx.numel(), scale, _stream(stream)))
    return out, lse


def dense_attn(q, k, v, *, block: int, scale: Optional[float] = None, q_block_len=None, kv_block_len=None,
               out=None, lse=None, nkb: Optional[int] = None, stream=None):
    """Dense attention over every KV block, through the same kernel."""
    d, heads, nqb, nkb_, qhs, khs, vhs, out, ohs, lse = _attn_prep(q, k, v, out, lse, block)
    nkb = nkb_ if nkb is None else nkb
    _attn_sizes(heads, nqb, nkb, nkb_, q_block_len, kv_block_len)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    _check(_lib.bsa_dense_attn(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _dtype_code(q), heads, d, block, nqb, nkb, qhs, khs,
        vhs, ohs, _ptr(_i32(q_block_len, "q_block_len")), _ptr(_i32(kv_block_len, "kv_block_len")), scale,
        _stream(stream)))
    return out, lse


__all__ = ["gilbert_index", "gilbert_perm", "gilbert_perm_pool", "gilbert_perm_pool_batch", "gilbert_block_window",
           "gilbert_tile_index", "tile_perm", "tile_block_window", "tile_grid", "slab_overlap", "slab_coverage",
           "route_topk", "route_topk_static", "ROUTE_STATIC_SCRATCH_BYTES", "route_workspace_size", "route_capacity", "route_materialize",
           "route_materialize_workspace_size", "materialize_capacity", "MaterializeArgs", "block_sparse_attn",
           "block_sparse_attn_raster", "dense_attn", "version", "library", "BsaError", "RouteArgs", "PermJob",
           "MAX_PERM_JOBS", "EXPORTED", "BSA_OK", "BSA_EINVAL", "BSA_EUNSUPPORTED", "BSA_EWORKSPACE", "BSA_EHIP",
           "BSA_BF16", "BSA_F32"]
