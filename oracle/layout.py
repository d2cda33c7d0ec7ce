"""Raster <-> Gilbert head-major, block-padded layouts, and block lengths.

A chunk's tokens, in curve order, are cut into consecutive ``Bs``-token
blocks; the last block of a chunk is zero-padded.  The KV history is the
concatenation of chunks, each padded on its own, so block ``b`` of every chunk
covers the same footprint of the latent grid ("global-aligned" storage)
[Velox: Spatial Memory Makes World Models Efficient -- Key Contributions 3;
Methodology, Step 6].  Blocks are runs of the token curve, not fixed 3-D
tiles: that is the only reading under which a 3 x 30 x 52 chunk with
128-token blocks pads only its last block.
"""

from __future__ import annotations

import numpy as np


def n_blocks(L: int, bs: int) -> int:
    """Number of ``bs``-token blocks that hold ``L`` tokens."""
    return -(-L // bs)


def chunk_block_lengths(L: int, bs: int, n_chunks: int = 1) -> np.ndarray:
    """Valid tokens of every block of ``n_chunks`` chunks of ``L`` tokens."""
    nb = n_blocks(L, bs)
    one = np.array([min(bs, L - b * bs) for b in range(nb)], dtype=np.int64)
    return np.tile(one, n_chunks)


def permute_forward(src: np.ndarray, perm: np.ndarray, bs: int) -> np.ndarray:
    """Raster token-major ``src[L][heads][d]`` -> Gilbert head-major
    ``dst[heads][nB*bs][d]`` with ``dst[h][i] = src[perm[i]][h]`` for ``i < L``
    and zero rows for ``L <= i < nB*bs``."""
    L, heads, d = src.shape
    assert perm.shape == (L,)
    nb = n_blocks(L, bs)
    dst = np.zeros((heads, nb * bs, d), dtype=src.dtype)
    # row i of every head takes raster token perm[i]
    dst[:, :L, :] = np.transpose(src[perm, :, :], (1, 0, 2))
    return dst


def permute_inverse(src: np.ndarray, perm: np.ndarray, L: int) -> np.ndarray:
    """Gilbert head-major ``src[heads][rows][d]`` -> raster ``dst[L][heads][d]``
    with ``dst[perm[i]][h] = src[h][i]``; padded rows are dropped."""
    heads, rows, d = src.shape
    assert perm.shape == (L,) and rows >= L
    dst = np.zeros((L, heads, d), dtype=src.dtype)
    # raster token perm[i] takes row i of every head
    dst[perm, :, :] = np.transpose(src[:, :L, :], (1, 0, 2))
    return dst
