"""Pins of the geometry oracle: closed forms of the camera-facing box, an
exact linear-programming intersection test against the separating-axis
test, a separable count of the grid intersection on camera-aligned boxes,
the self and half-shift IoU, and coverage on configurations whose answer is
known by construction."""

import math

import numpy as np
import pytest
from scipy.optimize import linprog

from oracle import geometry as og
from oracle.gilbert import gilbert_order


def cam(fx=10.0, fy=12.0, cx=0.0, cy=0.0, R=np.eye(3), C=(0.0, 0.0, 0.0)):
    return np.concatenate([[fx, fy, cx, cy], np.asarray(R, dtype=np.float64).reshape(-1), C])


def rot(yaw, pitch=0.0, roll=0.0):
    cy_, sy = math.cos(yaw), math.sin(yaw)
    cp, sp = math.cos(pitch), math.sin(pitch)
    cr, sr = math.cos(roll), math.sin(roll)
    Ry = np.array([[cy_, 0, sy], [0, 1, 0], [-sy, 0, cy_]])
    Rx = np.array([[1, 0, 0], [0, cp, -sp], [0, sp, cp]])
    Rz = np.array([[cr, -sr, 0], [sr, cr, 0], [0, 0, 1]])
    return Ry @ Rx @ Rz


def box(c, R, e):
    return (np.asarray(c, dtype=np.float64), np.asarray(R, dtype=np.float64).T.copy(), np.asarray(e, dtype=np.float64))


def test_slab_box_closed_form():
    c0 = cam(fx=10.0, fy=20.0)
    centre, axes, half = og.slab_box(c0, (-1.0, -2.0, 1.0, 2.0, 4.0, 6.0))
    assert np.allclose(centre, [0.0, 0.0, 5.0], atol=0, rtol=0)
    assert np.array_equal(axes, np.eye(3))
    assert np.allclose(half, [0.5, 0.5, 1.0], rtol=1e-15)
    # a rotated, translated camera: the centre lies on the ray through the
    # rectangle centre at the middle depth, and the axes are the camera's
    R = rot(0.3, -0.2, 0.1)
    c1 = cam(fx=30.0, fy=30.0, cx=26.0, cy=15.0, R=R, C=(1.0, -2.0, 3.0))
    centre, axes, half = og.slab_box(c1, (10.0, 4.0, 18.0, 9.0, 5.0, 9.0))
    x, y, z = R.T @ (centre - np.array([1.0, -2.0, 3.0]))
    assert z == pytest.approx(7.0, rel=1e-14)
    assert 30.0 * x / z + 26.0 == pytest.approx(14.0, rel=1e-14)
    assert 30.0 * y / z + 15.0 == pytest.approx(6.5, rel=1e-14)
    assert np.allclose(axes, R.T, rtol=0, atol=0)
    assert np.allclose(half, [8 * 7 / 60, 5 * 7 / 60, 2.0], rtol=1e-15)


def _intersect_lp(ba, bb):
    """Exact feasibility of a point inside both closed boxes (12 halfspaces)."""
    A_ub, b_ub = [], []
    for c, Ax, e in (ba, bb):
        for k in range(3):
            A_ub.append(Ax[k])
            b_ub.append(e[k] + Ax[k] @ c)
            A_ub.append(-Ax[k])
            b_ub.append(e[k] - Ax[k] @ c)
    r = linprog(np.zeros(3), A_ub=np.array(A_ub), b_ub=np.array(b_ub), bounds=[(None, None)] * 3, method="highs")
    return r.status == 0


def _margin(ba, bb):
    """Largest separation gap over the 15 axes (normalised); near-zero
    margins are too close to call for the LP tolerance."""
    ca, A, ea = ba
    cb, B, eb = bb
    d = cb - ca
    axes = [A[k] for k in range(3)] + [B[k] for k in range(3)]
    axes += [np.cross(A[i], B[j]) for i in range(3) for j in range(3)]
    best = -np.inf
    for L in axes:
        n = np.linalg.norm(L)
        if n < 1e-6:
            continue
        L = L / n
        gap = abs(L @ d) - sum(ea[k] * abs(L @ A[k]) for k in range(3)) - sum(eb[k] * abs(L @ B[k]) for k in range(3))
        best = max(best, gap)
    return best


def test_separating_axis_test_agrees_with_exact_intersection():
    rng = np.random.default_rng(5)
    edge_cases = 0
    checked = 0
    for _ in range(1500):
        ba = box(rng.normal(size=3) * 0.5, rot(*rng.uniform(-math.pi, math.pi, 3)), rng.uniform(0.2, 1.5, 3))
        bb = box(rng.normal(size=3) * 1.5, rot(*rng.uniform(-math.pi, math.pi, 3)), rng.uniform(0.2, 1.5, 3))
        if abs(_margin(ba, bb)) < 1e-6:
            continue
        sep = og.separated(ba, bb)
        assert sep == (not _intersect_lp(ba, bb))
        checked += 1
        # separated by an edge-edge axis only: the face normals alone miss it
        if sep:
            faces = [ba[1][k] for k in range(3)] + [bb[1][k] for k in range(3)]
            d = bb[0] - ba[0]
            by_face = any(abs(L @ d) > sum(ba[2][k] * abs(L @ ba[1][k]) for k in range(3))
                          + sum(bb[2][k] * abs(L @ bb[1][k]) for k in range(3)) for L in faces)
            edge_cases += not by_face
    assert checked > 1400 and edge_cases > 5


def _count_1d(ca, ea, cb, eb, n):
    s = (2.0 * np.arange(n) + 1.0) / n - 1.0
    return int(np.sum(np.abs(ca + s * ea - cb) <= eb))


@pytest.mark.parametrize("n", [4, 8, 13])
def test_grid_iou_on_aligned_boxes_is_the_separable_count(n):
    rng = np.random.default_rng(n)
    R = rot(0.4, 0.2, -0.3)
    for _ in range(200):
        ca, cb = rng.normal(size=3), rng.normal(size=3) * 0.7
        ea, eb = rng.uniform(0.3, 1.5, 3), rng.uniform(0.3, 1.5, 3)
        # coordinates in the shared frame: the count factorises by axis
        cnt = 1
        for k in range(3):
            cnt *= _count_1d(ca[k], ea[k], cb[k], eb[k], n)
        va, vb = 8 * np.prod(ea), 8 * np.prod(eb)
        inter = va * cnt / n ** 3
        sep = any(abs(ca[k] - cb[k]) > ea[k] + eb[k] for k in range(3))
        expect = 0.0 if sep else inter / (va + vb - inter)
        got = og.grid_iou(box(R @ ca, R, ea), box(R @ cb, R, eb), n)
        assert got == pytest.approx(expect, rel=1e-12, abs=1e-15)


def test_grid_iou_self_half_shift_and_disjoint():
    R = rot(0.7, -0.1, 0.2)
    e = np.array([0.5, 1.0, 2.0])
    a = box(np.zeros(3), R, e)
    assert og.grid_iou(a, a, 8) == 1.0
    # shifted by one half extent along the second axis: half the points
    shifted = box(R @ np.array([0.0, 1.0, 0.0]), R, e)
    assert og.grid_iou(a, shifted, 8) == pytest.approx(1.0 / 3.0, rel=1e-15)
    far = box(R @ np.array([0.0, 0.0, 4.5]), R, e)
    assert og.grid_iou(a, far, 8) == 0.0
    # containment: a small box inside a large one -> vol_small / vol_large
    small = box(np.zeros(3), R, e / 2)
    assert og.grid_iou(small, a, 8) == pytest.approx(1.0 / 8.0, rel=1e-15)


def test_overlap_matrix_takes_the_best_pair():
    c0 = cam(fx=20.0, fy=20.0)
    cams = np.stack([c0, cam(fx=20.0, fy=20.0, C=(0.0, 0.0, 0.5))])
    q_geom = np.array([[0, 0, 4, 4, 5, 7], [-6, -6, -2, -2, 5, 7.0]])
    h_geom = np.array([[-6, -6, -2, -2, 5, 7.0], [20, 20, 24, 24, 5, 7.0], [0, 0, 4, 4, 4.5, 6.5]])
    ov = og.overlap_matrix(cams, [0, 2, 2], [0, 0], q_geom, [0, 2, 3, 3], [0, 0, 1], h_geom, n=8)
    assert ov.shape == (2, 3)
    assert ov[0, 0] == 1.0                              # second query slab equals the first historical one
    assert ov[1].tolist() == [0.0, 0.0, 0.0]            # a block without slabs
    # same frustum seen from a camera half a unit further forward: the
    # slab at camera depth [4.5, 6.5] is the world box of depth [5, 7]
    assert ov[0, 1] == og.grid_iou(og.slab_box(c0, q_geom[0]), og.slab_box(cams[1], h_geom[2]), 8)
    assert 0.0 < ov[0, 1] < 1.0
    assert ov[0, 2] == 0.0                              # historical block 2 has no slab


def test_projection_round_trip_and_coverage_by_construction():
    R = rot(0.2, 0.1, 0.0)
    c0 = cam(fx=8.0, fy=8.0, cx=4.0, cy=3.0, R=R, C=(0.5, 0.0, -1.0))
    # unproject a token centre and test it against slabs around it
    u, v, z = 2.5, 1.5, 5.0
    p = R @ np.array([(u - 4.0) * z / 8.0, (v - 3.0) * z / 8.0, z]) + np.array([0.5, 0.0, -1.0])
    assert og.in_slab(p, c0, (2, 1, 3, 2, 4.0, 6.0))
    assert not og.in_slab(p, c0, (2, 1, 3, 2, 5.5, 6.0))          # in front of the depth interval
    assert not og.in_slab(p, c0, (3, 1, 4, 2, 4.0, 6.0))          # the next column
    # frame 0's camera sits far off, frame 1's is the slab's; depth 5
    # everywhere except a NaN row; one slab over the left half of frame 1 at
    # depth [4, 6]: a block's coverage is the share of its tokens in frame 1,
    # left half, not in the NaN row
    grid = (2, 4, 6)
    T, H, W = grid
    order = gilbert_order(*grid)[0]
    cams = np.stack([cam(fx=8.0, fy=8.0, cx=4.0, cy=3.0, R=R, C=(100.0, 0.0, -1.0)), c0])
    depth = np.full(grid, 5.0)
    depth[:, 2, :] = np.nan
    bs = 5
    cov = og.coverage_scores(cams, [0, 1], depth, order, grid, bs, [1], np.array([[0, 0, 3, 4, 4.0, 6.0]]))
    assert 0.0 < cov.max() < 1.0 and cov.min() == 0.0
    for i in range(len(cov)):
        cells = order[i * bs:(i + 1) * bs]
        t, h, w = cells // (H * W), (cells % (H * W)) // W, cells % W
        expect = np.mean((t == 1) & (w < 3) & (h != 2))
        assert cov[i] == expect, (i, cov[i], expect)
    # a subset of blocks, in the order asked
    sub = og.coverage_scores(cams, [0, 1], depth, order, grid, bs, [1], np.array([[0, 0, 3, 4, 4.0, 6.0]]),
                             blocks=[4, 0])
    assert sub.tolist() == [cov[4], cov[0]]
