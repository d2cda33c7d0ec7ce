"""Route materialisation around the top-K: coverage-gated budgets, the
previous chunk's reservation, a cumulative-mass prefix for poorly covered
query blocks, and the local window in Gilbert block order.

Test infrastructure: only tests and the benchmark's CPU baseline use this
module; the library never does.

Pages [Velox: Spatial Memory Makes World Models Efficient]:

* Methodology, Step 3: each query block has a coverage score, the share of
  its tokens that lie in some valid historical slab;
* Methodology, Step 4: the soft geometric fusion applies to well-covered
  query blocks;
* Methodology, Step 5: a well-covered query block first takes every KV
  block of the previous chunk, then fills its budget K_cov with the best of
  the others; a poorly covered one ranks by the unbiased model scores and
  stops at the shortest prefix whose probability mass passes a threshold,
  never more than K_unc blocks; on top of either budget, each route adds the
  block's 26 neighbours in the Gilbert block order and, optionally, blocks
  of reference frames;
* the calibrated constants eta_cov = 0.9, K_cov = 80, K_unc = 150 close the
  Methodology section.

Readings where the pages are silent:

* coverage is given per query block (one vector shared by all heads, like
  the overlap); a block is well covered when coverage >= eta_cov.  The
  coverage reaches the library as float32, so this decision is taken in
  float32 (coverage and eta_cov both rounded to float32): for a coverage
  that is a ratio k/n of token counts (n <= 2^16) that decides exactly as
  the exact ratio against eta_cov does, e.g. 72 of 80 tokens is covered at
  0.9, where a float64 comparison of float32(0.9) with 0.9 would not be;
* the cumulative-mass threshold is not given; it is a parameter (0.9 by
  default) on the unbiased distribution p = softmax(s) of the row, ordered
  by (p descending, block index ascending); the prefix is the shortest one
  whose running sum reaches the threshold;
* the reservation takes every block of the previous chunk that holds a valid
  token (all of them even past K_cov); the top-scoring fill takes
  max(0, K_cov - reserved) more by the fused key of the router;
* the 26-neighbour window of query block i (chunk c) is the set of KV blocks
  holding any cell of the 3 x 3 x 3 neighbourhood (the cell itself included)
  of any valid token of i, with time running across chunk boundaries into
  chunk c - 1 (chunk c + 1 is in the future and not part of the history);
* reference-frame blocks are a caller-given block range;
* only blocks holding a valid token enter a list; lists are ascending and
  duplicate-free; a query block with no valid token gets an empty list.
"""

from __future__ import annotations

import numpy as np

from .route import pool_blocks, selection_key


def block_window(order: np.ndarray, grid, bs: int, q_chunk: int):
    """26-neighbour window of every query block of chunk ``q_chunk``.

    ``order`` is the chunk's curve (``order[i]`` = raster cell of curve
    position i, raster = (t*H + h)*W + w); returns one sorted int64 array of
    absolute KV block indices per query block (blocks of chunks q_chunk - 1
    and q_chunk, ``nbc`` blocks per chunk)."""
    T, H, W = grid
    L = T * H * W
    nbc = -(-L // bs)
    pos = np.empty(L, dtype=np.int64)
    pos[np.asarray(order, dtype=np.int64)] = np.arange(L)
    out = []
    for b in range(nbc):
        found = set()
        for gp in range(b * bs, min(L, (b + 1) * bs)):
            cell = int(order[gp])
            t, rem = divmod(cell, H * W)
            h, w = divmod(rem, W)
            for dt in (-1, 0, 1):
                tt = t + dt
                chunk = q_chunk
                if tt < 0:
                    tt += T
                    chunk -= 1
                elif tt >= T:
                    continue                      # the next chunk is not history
                if chunk < 0:
                    continue
                for dh in (-1, 0, 1):
                    hh = h + dh
                    if hh < 0 or hh >= H:
                        continue
                    for dw in (-1, 0, 1):
                        ww = w + dw
                        if ww < 0 or ww >= W:
                            continue
                        nb_pos = int(pos[(tt * H + hh) * W + ww])
                        found.add(chunk * nbc + nb_pos // bs)
        out.append(np.array(sorted(found), dtype=np.int64))
    return out


def mass_prefix(s_row: np.ndarray, visible: np.ndarray, mass: float, cap: int) -> np.ndarray:
    """Shortest prefix, in (p descending, index ascending) order, of the
    visible blocks whose cumulative p = softmax(s) reaches ``mass``, at most
    ``cap`` blocks; returned ascending."""
    idx = np.nonzero(visible)[0]
    if idx.size == 0 or cap <= 0:
        return np.zeros(0, dtype=np.int64)
    s = s_row[idx]
    e = np.exp(s - s.max())
    p = e / e.sum()
    order = np.lexsort((idx, -s))                # p is increasing in s
    csum = np.cumsum(p[order])
    reach = np.nonzero(csum >= mass)[0]
    m = int(reach[0]) + 1 if reach.size else idx.size
    m = min(m, int(cap), idx.size)
    return np.sort(idx[order[:m]])


def materialize_head(q, k, q_len, k_len, bs, *, scale, coverage, eta_cov=0.9, k_cov=80, k_unc=150,
                     mass=0.9, prev_blocks=(0, 0), windows=None, ref_blocks=(0, 0), overlap=None,
                     lam=2.0, tau=0.1, g_ref=0.2):
    """Materialised routes of every query block of one head.

    ``q[nqb*bs][d]``, ``k[nkb*bs][d]`` float64; ``coverage[nqb]``;
    ``prev_blocks`` and ``ref_blocks`` are [begin, end) block ranges;
    ``windows[i]`` the window of query block i (absolute block indices).
    Every KV block is a candidate.  Returns ``dict(lists, covered, kappa,
    s)`` with one ascending int64 array per query block."""
    q_len = np.asarray(q_len)
    k_len = np.asarray(k_len)
    nqb, nkb = len(q_len), len(k_len)
    qbar = pool_blocks(q, q_len, bs)
    kbar = pool_blocks(k, k_len, bs)
    visible = k_len > 0
    kb = np.where(visible[:, None], kbar, 0.0)
    qb = np.where((q_len > 0)[:, None], qbar, 0.0)
    s = (qb @ kb.T) * scale
    covered = np.asarray(coverage, dtype=np.float64).astype(np.float32) >= np.float32(eta_cov)
    # the geometric fusion applies to the well-covered rows only
    ov = None
    if overlap is not None:
        ov = np.asarray(overlap, dtype=np.float64).copy()
        ov[~covered, :] = 0.0
    kappa = selection_key(qb, kb, scale, ov, lam, tau, g_ref)
    lists = []
    for i in range(nqb):
        if q_len[i] <= 0:
            lists.append(np.zeros(0, dtype=np.int64))
            continue
        members = set()
        if covered[i]:
            reserved = np.zeros(nkb, dtype=bool)
            reserved[prev_blocks[0]:prev_blocks[1]] = True
            reserved &= visible
            members.update(np.nonzero(reserved)[0].tolist())
            rest = visible & ~reserved
            n_fill = max(0, int(k_cov) - int(reserved.sum()))
            idx = np.nonzero(rest)[0]
            if n_fill > 0 and idx.size:
                order = np.lexsort((idx, -kappa[i, idx]))
                members.update(idx[order[:n_fill]].tolist())
        else:
            members.update(mass_prefix(s[i], visible, mass, k_unc).tolist())
        if windows is not None:
            members.update(int(j) for j in windows[i] if 0 <= j < nkb and visible[j])
        for j in range(max(0, ref_blocks[0]), min(nkb, ref_blocks[1])):
            if visible[j]:
                members.add(j)
        lists.append(np.array(sorted(members), dtype=np.int64))
    return dict(lists=lists, covered=covered, kappa=kappa, s=s)
