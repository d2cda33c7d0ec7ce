"""Attention restricted to routed KV blocks, and the dense special case.

Pages [Velox: Spatial Memory Makes World Models Efficient]: the measured path
is an indexed block-sparse attention kernel in which each current query block
looks only at its routed historical KV blocks; skipping a block removes both
its QK^T tile and its KV load (Methodology, Step 6).  The dense baseline
attends to all retained context (Main Findings).

Definition computed here, per head h and query row t of query block i with
routed list S_i:

    U      = valid keys of the blocks in S_i
    z_u    = (q_t . k_u) * scale                  for u in U
    O_t    = sum_u softmax_u(z) v_u,   LSE_t = log sum_u exp(z_u)

with a two-pass softmax (max, then normalised exponentials), in float64.
No causal mask (the chunk attends to all history); padded query rows give
O = 0; an empty list gives O = 0 and LSE = -inf.
"""

from __future__ import annotations

import numpy as np


def _valid_key_rows(blocks, k_len, bs):
    rows = [np.arange(b * bs, b * bs + int(k_len[b]), dtype=np.int64) for b in blocks]
    return np.concatenate(rows) if rows else np.zeros(0, dtype=np.int64)


def attend_rows(q_rows: np.ndarray, k: np.ndarray, v: np.ndarray, key_rows: np.ndarray, scale: float):
    """Softmax attention of the query rows ``q_rows[n][d]`` over the keys
    ``k[key_rows]`` / values ``v[key_rows]``; returns ``(O[n][dv], LSE[n])``."""
    n = q_rows.shape[0]
    dv = v.shape[1]
    if key_rows.size == 0:
        return np.zeros((n, dv)), np.full(n, -np.inf)
    z = (q_rows @ k[key_rows].T) * scale
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    den = e.sum(axis=1, keepdims=True)
    o = (e @ v[key_rows]) / den
    lse = (m + np.log(den))[:, 0]
    return o, lse


def block_sparse_head(q, k, v, q_len, k_len, bs, lists, scale, rows=None):
    """Routed attention for one head.

    ``q[nqb*bs][d]``, ``k``/``v[nkb*bs][d]`` float64; ``lists[i]`` the KV blocks
    of query block ``i``.  ``rows``: optional subset of query rows to compute
    (others are left as NaN), for spot checks at full size.
    Returns ``(O[nqb*bs][dv], LSE[nqb*bs])``."""
    nqb = len(q_len)
    dv = v.shape[1]
    o = np.zeros((nqb * bs, dv))
    lse = np.full(nqb * bs, -np.inf)
    if rows is not None:
        o[:] = np.nan
        lse[:] = np.nan
        wanted = np.zeros(nqb * bs, dtype=bool)
        wanted[np.asarray(rows)] = True
    for i in range(nqb):
        r0 = i * bs
        n_valid = int(q_len[i])
        sel = np.arange(r0, r0 + bs)
        if rows is not None:
            sel = sel[wanted[sel]]
            if sel.size == 0:
                continue
        valid = sel[sel < r0 + n_valid]
        pad = sel[sel >= r0 + n_valid]
        o[pad] = 0.0
        lse[pad] = -np.inf
        if valid.size == 0:
            continue
        keys = _valid_key_rows(lists[i], k_len, bs)
        oi, li = attend_rows(q[valid], k, v, keys, scale)
        o[valid] = oi
        lse[valid] = li
    return o, lse


def dense_head(q, k, v, q_len, k_len, bs, scale, rows=None):
    """Dense attention for one head: every KV block is listed."""
    all_blocks = [b for b in range(len(k_len)) if k_len[b] > 0]
    lists = [all_blocks] * len(q_len)
    return block_sparse_head(q, k, v, q_len, k_len, bs, lists, scale, rows=rows)


def token_mask_head(q, k, v, q_len, k_len, bs, lists, scale):
    """The same result as ``block_sparse_head`` written as one masked
    softmax over the full token-by-token score matrix (brute force for small
    cases): key u is visible to query t when u is a valid row of a block in
    the list of t's block."""
    nq, nk = q.shape[0], k.shape[0]
    allowed = np.zeros((nq, nk), dtype=bool)
    for i, blocks in enumerate(lists):
        for b in blocks:
            allowed[i * bs: i * bs + int(q_len[i]), b * bs: b * bs + int(k_len[b])] = True
    z = (q @ k.T) * scale
    z = np.where(allowed, z, -np.inf)
    o = np.zeros((nq, v.shape[1]))
    lse = np.full(nq, -np.inf)
    live = allowed.any(axis=1)
    zl = z[live]
    m = zl.max(axis=1, keepdims=True)
    e = np.exp(zl - m)
    den = e.sum(axis=1, keepdims=True)
    o[live] = (e @ v) / den
    lse[live] = (m + np.log(den))[:, 0]
    return o, lse
