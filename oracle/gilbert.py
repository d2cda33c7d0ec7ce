"""Generalized-Hilbert ("Gilbert") order of a T x H x W latent grid.

Pages: Velox keeps its KV history in a "global-aligned Gilbert" order so that
neighbouring image regions stay contiguous and a run of consecutive tokens is a
compact 3-D tile [Velox: Spatial Memory Makes World Models Efficient -- Key
Contributions 3; Methodology, Step 6].  Light Interaction speaks of "3D block
sparse attention" [Light Interaction -- abstract].  Neither page defines the
curve, so the construction below is this project's reading: a 3-D
generalized Hilbert curve for an arbitrary cuboid, written as a plain
recursion that emits cells in visit order.

Definition (the GPU kernel implements the same definition as a per-index
descent; the two are written independently).

A call ``fill(p, a, b, c)`` visits every cell of the cuboid with corner ``p``
spanned by the signed axis vectors ``a`` (the travel axis), ``b`` and ``c``.
It starts at ``p`` and, whenever the cuboid's parity allows, ends at
``p + (|a|-1) * unit(a)``.  Halving an axis ``v`` gives ``|v| // 2`` cells,
bumped by one when that is odd and ``|v| > 2`` (even halves keep the parity a
corner-to-corner unit-step path needs).

1. ``|b| == |c| == 1``: a straight run along ``a``.
2. ``|c| == 1`` (or ``|b| == 1``): the 2-D rule in the plane of ``a`` and the
   other axis (below).
3. ``|a| == 1``: the 2-D rule on the ``(b, c)`` face, travelling the longer of
   the two (only reached on parity-infeasible shapes).
4. ``|b| == |c| == 2``: if ``|a| == 2`` the 2x2x2 cube is two 2x2 faces: the
   face at ``a = 0`` by the 2-D rule from ``p`` along ``b``, then the face at
   ``a = 1`` by the 2-D rule from its ``b``-far corner along ``-b``.  Otherwise
   split ``a`` at its even half and fill the two parts in turn.
5. ``2|a| > 3 max(|b|, |c|)``: split ``a`` at its even half; fill both parts
   in turn, each travelling ``a``.
6. otherwise a U-turn in the plane of ``a`` and the longer ``L`` of ``b``,
   ``c`` (``b`` on ties), with ``O`` the remaining axis carried whole:
   ``fill(p, L/2, a/2, O)``, ``fill(p + L/2, a, L - L/2, O)``,
   ``fill(p + (a - unit a) + (L/2 - unit L), -L/2, -(a - a/2), O)``.

2-D rule ``fill2(p, a, b)``: ``|b| == 1`` a run along ``a``; ``|a| == 1`` a run
along ``b``; ``2|a| > 3|b|`` split ``a`` at its even half; otherwise
``fill2(p, b/2, a/2)``, ``fill2(p + b/2, a, b - b/2)``,
``fill2(p + (a - unit a) + (b/2 - unit b), -b/2, -(a - a/2))``.  On
2^k x 2^k squares this is the classic Hilbert curve (up to a transpose).

Top level: the travel axis is the longest of (w, h, t) (ties prefer w, then
h), the second axis the next longest, start (0, 0, 0).  The same curve is used
for every chunk of the history ("global-aligned").

Pins (tests): bijection; unit steps on every shape whose parity allows a
corner-to-corner path (exhaustive sweep) and at the configuration shapes;
the textbook Hilbert ``d2xy`` order on 2^k squares; identity on 1x1xW;
locality of Bs-token runs against raster order.  Sequence parity with any
other program that calls itself "gilbert" is unpinned by design: the pages
fix no construction.
"""

from __future__ import annotations

import sys

import numpy as np

sys.setrecursionlimit(max(10000, sys.getrecursionlimit()))


def _sign(x: int) -> int:
    return (x > 0) - (x < 0)


def _length(v):
    return abs(v[0]) + abs(v[1]) + abs(v[2])


def _unit(v):
    return (_sign(v[0]), _sign(v[1]), _sign(v[2]))


def _plus(*vs):
    return (sum(v[0] for v in vs), sum(v[1] for v in vs), sum(v[2] for v in vs))


def _scale(v, k):
    return (v[0] * k, v[1] * k, v[2] * k)


def _minus(u, v):
    return (u[0] - v[0], u[1] - v[1], u[2] - v[2])


def _even_half(v):
    n = _length(v)
    h = n // 2
    if h % 2 == 1 and n > 2:
        h += 1
    return _scale(_unit(v), h)


def _run(p, v, out):
    u = _unit(v)
    for i in range(_length(v)):
        out.append(_plus(p, _scale(u, i)))


def _fill2(p, a, b, out):
    la, lb = _length(a), _length(b)
    if lb == 1:
        _run(p, a, out)
        return
    if la == 1:
        _run(p, b, out)
        return
    a2, b2 = _even_half(a), _even_half(b)
    if 2 * la > 3 * lb:
        _fill2(p, a2, b, out)
        _fill2(_plus(p, a2), _minus(a, a2), b, out)
        return
    _fill2(p, b2, a2, out)
    _fill2(_plus(p, b2), a, _minus(b, b2), out)
    _fill2(_plus(p, _minus(a, _unit(a)), _minus(b2, _unit(b))),
           _scale(b2, -1), _scale(_minus(a, a2), -1), out)


def _fill3(p, a, b, c, out):
    la, lb, lc = _length(a), _length(b), _length(c)
    if lb == 1 and lc == 1:
        _run(p, a, out)
        return
    if lc == 1:
        _fill2(p, a, b, out)
        return
    if lb == 1:
        _fill2(p, a, c, out)
        return
    if la == 1:
        if lb >= lc:
            _fill2(p, b, c, out)
        else:
            _fill2(p, c, b, out)
        return
    if lb == 2 and lc == 2:
        if la == 2:
            _fill2(p, b, c, out)
            _fill2(_plus(p, _unit(a), _minus(b, _unit(b))), _scale(b, -1), c, out)
            return
        a2 = _even_half(a)
        _fill3(p, a2, b, c, out)
        _fill3(_plus(p, a2), _minus(a, a2), b, c, out)
        return
    if 2 * la > 3 * max(lb, lc):
        a2 = _even_half(a)
        _fill3(p, a2, b, c, out)
        _fill3(_plus(p, a2), _minus(a, a2), b, c, out)
        return
    if lb >= lc:
        big, other = b, c
    else:
        big, other = c, b
    a2, big2 = _even_half(a), _even_half(big)
    _fill3(p, big2, a2, other, out)
    _fill3(_plus(p, big2), a, _minus(big, big2), other, out)
    _fill3(_plus(p, _minus(a, _unit(a)), _minus(big2, _unit(big))),
           _scale(big2, -1), _scale(_minus(a, a2), -1), other, out)


def gilbert_cells(T: int, H: int, W: int):
    """Cells ``(t, h, w)`` of the T x H x W grid in curve order."""
    if T < 1 or H < 1 or W < 1:
        raise ValueError("grid dimensions must be positive")
    # Axis vectors in (t, h, w) coordinates; longest first, ties -> w, h, t.
    axes = [(0, 0, W), (0, H, 0), (T, 0, 0)]
    axes.sort(key=lambda v: -_length(v))  # stable sort keeps the tie order
    out: list = []
    _fill3((0, 0, 0), axes[0], axes[1], axes[2], out)
    return out


def gilbert_order(T: int, H: int, W: int):
    """``perm[i]`` = raster index ``t*H*W + h*W + w`` of the i-th curve cell,
    and ``inv`` with ``inv[perm[i]] == i``.  Both int64 numpy arrays."""
    cells = gilbert_cells(T, H, W)
    perm = np.array([t * H * W + h * W + w for (t, h, w) in cells], dtype=np.int64)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.size, dtype=np.int64)
    return perm, inv
