"""Block router: mean pooling, model-derived importance, soft geometric fusion
with unbiased fallback, and top-K route materialisation.

Pages [Velox: Spatial Memory Makes World Models Efficient]:

* Methodology, Step 4: per layer, the visible KV blocks are scored with
  the block averages of the queries and keys; overlaps above a noise
  threshold tau are rescaled to g_hat, and the distribution is scaled by
  (1 + lambda * g_hat) and normalised again, so full overlap multiplies a
  block's weight by at most 1 + lambda and a block whose overlap was
  discarded keeps its weight.
* Key Contributions 2 and the abstract: where no geometry covers a region,
  its route comes from the model's scores alone (the fallback).
* Methodology, Step 5 / Main Findings: routes take the top-scoring blocks up
  to a budget (50 of 143 in the pages' audit).
* The calibrated constants tau = 0.1, g_ref = 0.2, lambda = 2 close the
  Methodology section; Main Findings motivates rescaling by the median
  positive overlap (0.211).

Readings where the pages are silent (each is listed in the design notes):

* pooling is the arithmetic mean over the valid (unpadded) rows of a block;
* importance is p = softmax_j(qbar_i . kbar_j * scale) with the attention
  scale;
* g_hat = 0 if g <= tau, else min(1, g / g_ref);
* a query-block row whose overlap row is all zero is a fallback row and keeps
  p unchanged; with the rule above the same holds for any row whose overlap
  never exceeds tau, and both counts are reported;
* one overlap matrix [n_qblocks][n_candidates] is shared by all heads;
* top-K ranks by the fused distribution, ties broken towards the lower block
  index; K_eff = min(K, number of candidate blocks with at least one valid
  token); a query block with no valid token gets an empty list;
* lists are written in ascending block order; blocks of the dense tail (the
  current chunk, when the caller asks for it) follow every list.
"""

from __future__ import annotations

import numpy as np

from .numerics import exact_column_sums


def pool_blocks(x: np.ndarray, lengths: np.ndarray, bs: int) -> np.ndarray:
    """Mean of the valid rows of each block of one head: the exact sum of
    each column, rounded once to float64, divided by the row count.

    ``x[rows][d]`` float64 with ``rows = len(lengths) * bs``; block ``b``
    holds rows ``b*bs .. b*bs + lengths[b] - 1``.  Blocks with no valid row
    give NaN."""
    nb = len(lengths)
    d = x.shape[1]
    out = np.full((nb, d), np.nan, dtype=np.float64)
    for b in range(nb):
        n = int(lengths[b])
        if n > 0:
            rows = x[b * bs: b * bs + n, :]
            out[b, :] = exact_column_sums(rows) / n
    return out


def importance(qbar: np.ndarray, kbar: np.ndarray, scale: float, visible: np.ndarray) -> np.ndarray:
    """Model-derived importance p[i][j] = softmax over visible blocks j of
    qbar_i . kbar_j * scale (zero where j is not visible)."""
    nq = qbar.shape[0]
    nk = kbar.shape[0]
    p = np.zeros((nq, nk), dtype=np.float64)
    if not visible.any():
        return p
    s = (qbar @ kbar[visible].T) * scale
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    p[:, visible] = e / e.sum(axis=1, keepdims=True)
    return p


def rescale_overlap(g: np.ndarray, tau: float, g_ref: float) -> np.ndarray:
    """Vetted, rescaled overlap: 0 at or below the noise threshold tau, else
    g / g_ref capped at 1."""
    g = np.asarray(g, dtype=np.float64)
    return np.where(g <= tau, 0.0, np.minimum(1.0, g / g_ref))


def fuse(p: np.ndarray, overlap, lam: float, tau: float, g_ref: float):
    """Soft geometric fusion with unbiased fallback.

    Returns ``(p_fused, zero_rows, unvetted_rows)``.  Rows of ``overlap`` that
    are all zero keep ``p`` (fallback); other rows become
    ``p * (1 + lam * g_hat)`` renormalised over the row."""
    nq = p.shape[0]
    if overlap is None:
        flags = np.ones(nq, dtype=bool)
        return p.copy(), flags, flags.copy()
    g = np.asarray(overlap, dtype=np.float64)
    g_hat = rescale_overlap(g, tau, g_ref)
    zero_rows = ~(g != 0.0).any(axis=1)
    unvetted_rows = ~(g_hat > 0.0).any(axis=1)
    out = p.copy()
    for i in range(nq):
        if zero_rows[i]:
            continue
        w = p[i] * (1.0 + lam * g_hat[i])
        z = w.sum()
        if z > 0:
            out[i] = w / z
    return out, zero_rows, unvetted_rows


def selection_key(qbar, kbar, scale, overlap, lam, tau, g_ref):
    """kappa = s + log1p(lam * g_hat): an order-equivalent form of the fused
    distribution within each row (the renormaliser is a positive per-row
    constant and log is increasing).  Fallback (all-zero) rows use s."""
    s = (qbar @ kbar.T) * scale
    if overlap is None:
        return s
    g = np.asarray(overlap, dtype=np.float64)
    g_hat = rescale_overlap(g, tau, g_ref)
    zero_rows = ~(g != 0.0).any(axis=1)
    bias = np.log1p(lam * g_hat)
    bias[zero_rows, :] = 0.0
    return s + bias


def top_k_ascending(score_row: np.ndarray, visible: np.ndarray, k: int) -> np.ndarray:
    """The ``k`` visible entries with the largest score (ties: lower index
    first), returned in ascending index order."""
    idx = np.nonzero(visible)[0]
    k_eff = min(int(k), idx.size)
    if k_eff <= 0:
        return np.zeros(0, dtype=np.int64)
    vals = score_row[idx]
    # lexsort sorts by the last key first: score descending, then index ascending
    order = np.lexsort((idx, -vals))
    chosen = idx[order[:k_eff]]
    return np.sort(chosen)


def route_head(q, k, q_len, k_len, bs, *, scale, k_per_row, overlap=None,
               lam=2.0, tau=0.1, g_ref=0.2, n_dense_tail=0):
    """Route every query block of one head.

    ``q[nqb*bs][d]``, ``k[nkb*bs][d]`` float64; ``q_len``, ``k_len`` valid
    tokens per block; candidates are KV blocks ``0 .. nkb-n_dense_tail-1``
    with at least one valid token; blocks of the dense tail with at least one
    valid token are appended to every list.  ``k_per_row[i]`` is the budget of
    query block ``i``; ``overlap`` is ``[nqb][n_candidates]`` or None.

    Returns a dict with ``lists`` (one ascending int64 array per query block),
    ``p``, ``p_fused``, ``kappa``, ``zero_rows``, ``unvetted_rows``,
    ``qbar`` and ``kbar``."""
    q_len = np.asarray(q_len)
    k_len = np.asarray(k_len)
    nqb, nkb = len(q_len), len(k_len)
    n_cand = nkb - n_dense_tail
    qbar = pool_blocks(q, q_len, bs)
    kbar = pool_blocks(k[: n_cand * bs], k_len[:n_cand], bs)
    visible = k_len[:n_cand] > 0
    kb = np.where(visible[:, None], kbar, 0.0)
    qb = np.where((q_len > 0)[:, None], qbar, 0.0)
    p = importance(qb, kb, scale, visible)
    p_fused, zero_rows, unvetted_rows = fuse(p, overlap, lam, tau, g_ref)
    kappa = selection_key(qb, kb, scale, overlap, lam, tau, g_ref)
    tail = np.array([j for j in range(n_cand, nkb) if k_len[j] > 0], dtype=np.int64)
    lists = []
    for i in range(nqb):
        if q_len[i] <= 0:
            lists.append(np.zeros(0, dtype=np.int64))
            continue
        sel = top_k_ascending(p_fused[i], visible, int(k_per_row[i]))
        lists.append(np.concatenate([sel, tail]))
    return dict(lists=lists, p=p, p_fused=p_fused, kappa=kappa,
                zero_rows=zero_rows, unvetted_rows=unvetted_rows,
                qbar=qbar, kbar=kbar, visible=visible)


def to_csr(lists_per_row):
    """Concatenate per-row lists into ``(row_ptr, col_idx)`` int64 arrays."""
    row_ptr = np.zeros(len(lists_per_row) + 1, dtype=np.int64)
    for r, lst in enumerate(lists_per_row):
        row_ptr[r + 1] = row_ptr[r] + len(lst)
    col = np.concatenate([np.asarray(l, dtype=np.int64) for l in lists_per_row]) \
        if lists_per_row else np.zeros(0, dtype=np.int64)
    return row_ptr, col
