"""Pins of the route-materialisation oracle: closed forms of the local window
on single-token blocks, brute-force minimality of the mass prefix, and the
special case that reduces to the plain top-K router."""

import itertools

import numpy as np
import pytest

from oracle import materialize as om
from oracle import route as oroute
from oracle.gilbert import gilbert_order


def test_window_single_token_blocks_is_the_3x3x3_neighbourhood():
    # one-token blocks on the identity curve: block index == raster cell
    T, H, W = 2, 3, 4
    L = T * H * W
    for q_chunk in (0, 1, 3):
        win = om.block_window(np.arange(L), (T, H, W), 1, q_chunk)
        for cell in range(L):
            t, rem = divmod(cell, H * W)
            h, w = divmod(rem, W)
            expect = set()
            for dt, dh, dw in itertools.product((-1, 0, 1), repeat=3):
                tt, hh, ww = t + dt, h + dh, w + dw
                if not (0 <= hh < H and 0 <= ww < W) or tt >= T:
                    continue
                chunk = q_chunk if tt >= 0 else q_chunk - 1
                if chunk < 0:
                    continue
                expect.add(chunk * L + (tt % T) * H * W + hh * W + ww)
            assert set(win[cell].tolist()) == expect, (q_chunk, cell)
        # a cell of the first frame off the spatial border, in a later chunk,
        # sees all 27 cells (one frame back lies in the previous chunk)
        if q_chunk > 0:
            assert len(win[1 * W + 1]) == 27


@pytest.mark.parametrize("bs", [64, 128])
def test_window_properties_on_the_chunk_grid(bs):
    grid = (3, 30, 52)
    order = gilbert_order(*grid)[0]
    nbc = -(-4680 // bs)
    c = 4
    win = om.block_window(order, grid, bs, c)
    assert len(win) == nbc
    for b, wb in enumerate(win):
        assert c * nbc + b in wb                                # its own block
        assert np.all(np.diff(wb) > 0)
        assert np.all((wb >= (c - 1) * nbc) & (wb < (c + 1) * nbc))
        # the neighbourhood relation on cells is symmetric, so is the window
        # among the blocks of the same chunk
        for j in wb[wb >= c * nbc]:
            assert c * nbc + b in win[j - c * nbc]
    # the first chunk has no previous chunk
    win0 = om.block_window(order, grid, bs, 0)
    assert all(np.all(w >= 0) and np.all(w < nbc) for w in win0)


def test_mass_prefix_uniform_closed_form():
    s = np.zeros(8)
    vis = np.ones(8, dtype=bool)
    assert om.mass_prefix(s, vis, 0.5, 150).tolist() == [0, 1, 2, 3]   # 4/8 = 0.5 exactly, ties to low index
    assert om.mass_prefix(s, vis, 1.0, 150).tolist() == list(range(8))
    assert om.mass_prefix(s, vis, 1.0, 3).tolist() == [0, 1, 2]
    vis[2] = False
    assert 2 not in om.mass_prefix(s, vis, 1.0, 150).tolist()


def test_mass_prefix_extremes():
    rng = np.random.default_rng(0)
    s = rng.standard_normal(40)
    vis = np.ones(40, dtype=bool)
    assert om.mass_prefix(s, vis, 1e-12, 150).tolist() == [int(np.argmax(s))]
    assert om.mass_prefix(s, vis, 2.0, 150).size == 40                   # unreachable mass: everything
    assert om.mass_prefix(s, np.zeros(40, dtype=bool), 0.5, 150).size == 0


def test_mass_prefix_is_minimal_by_brute_force():
    rng = np.random.default_rng(1)
    for trial in range(60):
        n = int(rng.integers(2, 10))
        s = rng.standard_normal(n) * 2.0
        vis = rng.random(n) < 0.8
        if not vis.any():
            continue
        mass = float(rng.uniform(0.05, 0.99))
        got = om.mass_prefix(s, vis, mass, 150)
        idx = np.nonzero(vis)[0]
        p = np.zeros(n)
        e = np.exp(s[idx] - s[idx].max())
        p[idx] = e / e.sum()
        assert p[got].sum() >= mass - 1e-12
        # no smaller set of visible blocks reaches the mass
        for m in range(1, got.size):
            for sub in itertools.combinations(idx.tolist(), m):
                assert p[list(sub)].sum() < mass + 1e-12, (trial, sub)


def _tiny(seed=3, nqb=4, nkb=12, bs=8, d=16):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((nqb * bs, d))
    k = rng.standard_normal((nkb * bs, d)) + np.repeat(rng.standard_normal((nkb, d)) * 0.5, bs, axis=0)
    q_len = np.full(nqb, bs)
    k_len = np.full(nkb, bs)
    k_len[5] = 3
    k_len[7] = 0
    return q, k, q_len, k_len, bs


def test_all_covered_without_reservation_is_the_top_k_router():
    q, k, q_len, k_len, bs = _tiny()
    got = om.materialize_head(q, k, q_len, k_len, bs, scale=0.25, coverage=np.ones(4), k_cov=5)
    ref = oroute.route_head(q, k, q_len, k_len, bs, scale=0.25, k_per_row=np.full(4, 5))
    for a, b in zip(got["lists"], ref["lists"]):
        assert np.array_equal(a, b)


def test_routes_of_covered_and_uncovered_rows():
    q, k, q_len, k_len, bs = _tiny(seed=4)
    cov = np.array([0.95, 0.2, 0.9, 0.0])
    ov = np.random.default_rng(9).beta(0.5, 2.0, size=(4, 12))
    win = [np.array([0, 11]), np.array([], dtype=np.int64), np.array([7]), np.array([3, 4])]
    r = om.materialize_head(q, k, q_len, k_len, bs, scale=0.25, coverage=cov, k_cov=6, k_unc=5, mass=0.6,
                            prev_blocks=(8, 11), windows=win, ref_blocks=(0, 2), overlap=ov)
    vis = k_len > 0
    assert r["covered"].tolist() == [True, False, True, False]
    for i, lst in enumerate(r["lists"]):
        assert np.all(np.diff(lst) > 0) and np.all(vis[lst])
        assert {0, 1} <= set(lst.tolist())                           # reference blocks
        assert set(j for j in win[i].tolist() if vis[j]) <= set(lst.tolist())
        if r["covered"][i]:
            assert {8, 9, 10} <= set(lst.tolist())                   # reserved previous chunk
    # an uncovered row ignores the overlap: its route is the plain mass prefix
    for i in (1, 3):
        pre = om.mass_prefix(r["s"][i], vis, 0.6, 5)
        extra = set([0, 1]) | set(j for j in win[i].tolist() if vis[j])
        assert set(r["lists"][i].tolist()) == set(pre.tolist()) | extra
    # a covered row: 3 reserved + the 3 best others by the fused key
    rest = [j for j in range(12) if vis[j] and j not in (8, 9, 10)]
    best = sorted(rest, key=lambda j: (-r["kappa"][0, j], j))[:3]
    assert set(r["lists"][0].tolist()) == {8, 9, 10} | set(best) | {0, 1, 11}


def test_empty_query_block_gets_an_empty_list():
    q, k, q_len, k_len, bs = _tiny(seed=5)
    q_len = q_len.copy()
    q_len[2] = 0
    r = om.materialize_head(q, k, q_len, k_len, bs, scale=0.25, coverage=np.ones(4), k_cov=3,
                            ref_blocks=(0, 3))
    assert r["lists"][2].size == 0 and r["lists"][0].size > 0


def test_float32_coverage_decision_is_exact_for_token_ratios():
    """The well-covered decision is taken in float32 (the coverage's storage
    type): for every ratio k/n of covered tokens (n <= 128) and thresholds
    read as exact fractions, it agrees with the exact rational comparison,
    so a block with exactly 90 % of its tokens covered is well covered."""
    from fractions import Fraction
    for num, den in [(9, 10), (1, 2), (3, 4), (19, 20), (2, 3)]:
        eta = num / den
        for n in range(1, 129):
            for k in range(n + 1):
                f32 = np.float32(k / n) >= np.float32(eta)
                assert f32 == (Fraction(k, n) >= Fraction(num, den)), (k, n, eta)
    # the float64 comparison of a float32-stored 0.9 would call 72/80 poorly covered
    assert float(np.float32(72 / 80)) < 0.9


def test_coverage_at_the_threshold():
    q, k, q_len, k_len, bs = _tiny(seed=6)
    cov = np.array([72 / 80, np.float32(0.9), np.nextafter(np.float32(0.9), np.float32(0)), 71 / 80])
    r = om.materialize_head(q, k, q_len, k_len, bs, scale=0.25, coverage=cov, k_cov=6, k_unc=5, mass=0.6,
                            prev_blocks=(8, 11))
    assert r["covered"].tolist() == [True, True, False, False]
    r32 = om.materialize_head(q, k, q_len, k_len, bs, scale=0.25, coverage=cov.astype(np.float32), k_cov=6,
                              k_unc=5, mass=0.6, prev_blocks=(8, 11))
    assert r32["covered"].tolist() == [True, True, False, False]
    for a, b in zip(r["lists"], r32["lists"]):
        assert np.array_equal(a, b)
