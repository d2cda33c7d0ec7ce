"""Pins of the oracle's Gilbert order against what the problem fixes:
bijection, unit steps wherever parity allows a corner-to-corner path, the
textbook Hilbert curve on 2^k squares, degenerate shapes, and locality."""

import itertools
import os

import numpy as np
import pytest

from oracle.gilbert import gilbert_cells, gilbert_order


def _l1(a, b):
    return sum(abs(x - y) for x, y in zip(a, b))


def _feasible(T, H, W):
    # corner-to-corner along the longest axis on a bipartite grid graph:
    # an even cell count needs endpoints of opposite colour (travel length
    # even); an odd count needs both on the majority colour (length odd).
    n = T * H * W
    a = max(T, H, W)
    return (n % 2 == 0 and a % 2 == 0) or n % 2 == 1


def _check_bijection(T, H, W, cells):
    assert len(cells) == T * H * W
    assert len(set(cells)) == T * H * W
    for (t, h, w) in cells:
        assert 0 <= t < T and 0 <= h < H and 0 <= w < W


@pytest.mark.parametrize("shape", [(3, 30, 52), (1, 30, 52), (3, 30, 52 * 2), (21, 30, 52), (2, 16, 16)])
def test_config_shapes_unit_steps(shape):
    T, H, W = shape
    cells = gilbert_cells(T, H, W)
    _check_bijection(T, H, W, cells)
    assert cells[0] == (0, 0, 0)
    steps = [_l1(cells[i], cells[i + 1]) for i in range(len(cells) - 1)]
    assert max(steps) == 1
    # ends at the far end of the longest axis
    assert cells[-1] == (0, 0, W - 1) if W >= max(T, H) else True


def test_exhaustive_small_shapes():
    bad_feasible = []
    for T, H, W in itertools.product(range(1, 9), repeat=3):
        cells = gilbert_cells(T, H, W)
        _check_bijection(T, H, W, cells)
        bad = [i for i in range(len(cells) - 1) if _l1(cells[i], cells[i + 1]) != 1]
        if _feasible(T, H, W):
            if bad:
                bad_feasible.append((T, H, W))
        else:
            # parity forbids a corner-to-corner unit path: exactly one jump,
            # and it stays local
            assert len(bad) <= 1, (T, H, W, bad)
            for i in bad:
                assert _l1(cells[i], cells[i + 1]) <= 3
    assert bad_feasible == []


def test_perm_inv_consistent():
    perm, inv = gilbert_order(3, 30, 52)
    assert sorted(perm.tolist()) == list(range(4680))
    assert np.array_equal(inv[perm], np.arange(4680))
    assert np.array_equal(perm[inv], np.arange(4680))


def test_line_is_identity():
    perm, _ = gilbert_order(1, 1, 37)
    assert perm.tolist() == list(range(37))
    perm, _ = gilbert_order(1, 9, 1)
    assert perm.tolist() == list(range(9))


def test_hilbert_order2_golden(golden_dir):
    pts = []
    with open(os.path.join(golden_dir, "hilbert_order2.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                x, y = line.split()
                pts.append((int(x), int(y)))
    cells = gilbert_cells(1, 4, 4)
    # x = w (the travel axis), y = h
    assert [(w, h) for (_t, h, w) in cells] == pts


def _d2xy(n, d):
    """Textbook conversion of a Hilbert index to (x, y) on an n x n grid."""
    x = y = 0
    s = 1
    t = d
    while s < n:
        rx = 1 & (t // 2)
        ry = 1 & (t ^ rx)
        if ry == 0:
            if rx == 1:
                x = s - 1 - x
                y = s - 1 - y
            x, y = y, x
        x += s * rx
        y += s * ry
        t //= 4
        s *= 2
    return x, y


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
def test_classic_hilbert_on_squares(k):
    n = 2 ** k
    cells = gilbert_cells(1, n, n)
    # both end at the far end of their first axis: x = w, y = h
    ref = [_d2xy(n, d) for d in range(n * n)]
    assert [(w, h) for (_t, h, w) in cells] == ref


def _bbox_mean(cells, bs):
    vols = []
    for s in range(0, len(cells), bs):
        run = np.array(cells[s:s + bs])
        vols.append(np.prod(run.max(axis=0) - run.min(axis=0) + 1))
    return float(np.mean(vols))


def test_locality_beats_raster():
    cells = gilbert_cells(3, 30, 52)
    raster = [(t, h, w) for t in range(3) for h in range(30) for w in range(52)]
    for bs in (64, 128):
        g = _bbox_mean(cells, bs)
        r = _bbox_mean(raster, bs)
        assert g < 0.6 * r, (bs, g, r)
        assert g < 1.6 * bs
