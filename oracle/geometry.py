"""Geometric overlap and coverage of query blocks against the historical
frustum slabs: camera-facing oriented boxes, a separating-axis test, a
deterministic grid intersection-over-union, and the coverage score.

Test infrastructure: only tests and the benchmark's CPU baseline use this
module; the library never does.

Pages [Velox: Spatial Memory Makes World Models Efficient]:

* Methodology, Step 1: the geometry of a historical block is a set of
  frustum slabs (each a rectangle of tokens in the camera that saw it, with
  a range of depths) that the validity gates let through;
* Methodology, Step 3: every slab, query or historical, is replaced by an
  oriented box facing its camera; a query block scores a historical block
  by the largest intersection-over-union of its box with one of that
  block's boxes, measured on a fixed grid, a separating-axis test first
  discarding pairs that cannot meet; coverage, a second score, is the share
  of the query block's tokens lying in some valid historical slab (inside
  its rectangle and within its depth range).

Readings where the pages are silent:

* camera: pinhole in token units, ``cam = (fx, fy, cx, cy, R (row-major
  3 x 3, world-from-camera: its columns are the camera's right, down and
  forward axes in world space), C (camera centre))``; a camera-space point
  (x, y, z), z > 0, sits at token coordinates u = fx x / z + cx (column),
  v = fy y / z + cy (row); token (h, w) covers [w, w+1) x [h, h+1);
* slab: camera index, rectangle [u0, u1) x [v0, v1) in token units and a
  depth interval [z_lo, z_hi] in camera z; only valid slabs are given;
* camera-facing box of a slab: axes = the camera's axes; centre on the ray
  through the rectangle's centre at the middle depth z_m = (z_lo + z_hi)/2;
  half extents = the rectangle's half width and half height at z_m,
  (u1 - u0) z_m / (2 fx) and (v1 - v0) z_m / (2 fy), and half the depth
  interval;
* separating-axis test over the 15 axes of two boxes (3 + 3 face normals,
  9 edge cross products; a cross product with squared length below 1e-12
  is skipped, its edges being parallel); the boxes are separated when some
  axis has |L . (c_B - c_A)| > r_A + r_B (touching is not separated);
* grid: n x n x n points at the cell centres of the query box; the
  intersection volume is vol_A * (points inside the historical box) / n^3;
  IoU = inter / (vol_A + vol_B - inter), 0 when separated or when the union
  has no volume;
* a query block's overlap with a historical block is the largest IoU over
  every (query slab, historical slab) pair of the two blocks, 0 if either
  has none;
* coverage: the token's point is its centre (w + 1/2, h + 1/2) at its query
  depth in its frame's camera; it is covered when, for some historical slab,
  the point projects (z > 0) inside the slab's rectangle and its camera z
  lies in [z_lo, z_hi]; tokens without a depth (NaN or <= 0) are not
  covered; coverage = covered tokens / tokens of the block (0 for a block
  without tokens).

Arithmetic is float64 throughout.
"""

from __future__ import annotations

import numpy as np

AXIS_EPS2 = 1e-12


def camera_parts(cam):
    cam = np.asarray(cam, dtype=np.float64)
    return cam[0], cam[1], cam[2], cam[3], cam[4:13].reshape(3, 3), cam[13:16]


def slab_box(cam, geom):
    """Camera-facing box of a slab: ``(centre[3], axes[3][3] (rows = unit
    axes), half[3])``."""
    fx, fy, cx, cy, R, C = camera_parts(cam)
    u0, v0, u1, v1, zlo, zhi = (float(g) for g in geom)
    zm = (zlo + zhi) / 2.0
    uc, vc = (u0 + u1) / 2.0, (v0 + v1) / 2.0
    pc = np.array([(uc - cx) * zm / fx, (vc - cy) * zm / fy, zm])
    centre = R @ pc + C
    axes = R.T.copy()                    # row k = camera axis k in world space
    half = np.array([(u1 - u0) * zm / (2.0 * fx), (v1 - v0) * zm / (2.0 * fy), (zhi - zlo) / 2.0])
    return centre, axes, half


def separated(box_a, box_b) -> bool:
    """Separating-axis test of two oriented boxes."""
    ca, A, ea = box_a
    cb, B, eb = box_b
    d = cb - ca
    axes = [A[k] for k in range(3)] + [B[k] for k in range(3)]
    for i in range(3):
        for j in range(3):
            L = np.cross(A[i], B[j])
            if L @ L >= AXIS_EPS2:
                axes.append(L)
    for L in axes:
        ra = sum(ea[k] * abs(L @ A[k]) for k in range(3))
        rb = sum(eb[k] * abs(L @ B[k]) for k in range(3))
        if abs(L @ d) > ra + rb:
            return True
    return False


def grid_points(box, n: int) -> np.ndarray:
    """The n^3 cell centres of a box, [n^3][3]."""
    c, A, e = box
    s = (2.0 * np.arange(n) + 1.0) / n - 1.0
    si, sj, sl = np.meshgrid(s, s, s, indexing="ij")
    off = (si.reshape(-1, 1) * e[0]) * A[0] + (sj.reshape(-1, 1) * e[1]) * A[1] + (sl.reshape(-1, 1) * e[2]) * A[2]
    return c + off


def inside_box(points: np.ndarray, box) -> np.ndarray:
    c, B, e = box
    rel = (points - c) @ B.T             # coordinates along B's axes
    return np.all(np.abs(rel) <= e, axis=1)


def grid_iou(box_a, box_b, n: int = 8) -> float:
    """IoU of the query box ``box_a`` and the historical box ``box_b`` on an
    n^3 grid over ``box_a``; 0 when the separating-axis test separates them."""
    if separated(box_a, box_b):
        return 0.0
    cnt = int(inside_box(grid_points(box_a, n), box_b).sum())
    va = 8.0 * box_a[2][0] * box_a[2][1] * box_a[2][2]
    vb = 8.0 * box_b[2][0] * box_b[2][1] * box_b[2][2]
    inter = va * cnt / float(n * n * n)
    union = va + vb - inter
    return inter / union if union > 0.0 else 0.0


def overlap_matrix(cams, q_ptr, q_cam, q_geom, h_ptr, h_cam, h_geom, n: int = 8) -> np.ndarray:
    """overlap[i][j] = max IoU over the slabs of query block i and historical
    block j (slabs of block b are entries ptr[b] .. ptr[b+1]-1)."""
    nqb, nkb = len(q_ptr) - 1, len(h_ptr) - 1
    qbox = [slab_box(cams[int(q_cam[s])], q_geom[s]) for s in range(int(q_ptr[-1]))]
    hbox = [slab_box(cams[int(h_cam[s])], h_geom[s]) for s in range(int(h_ptr[-1]))]
    out = np.zeros((nqb, nkb))
    for i in range(nqb):
        for j in range(nkb):
            best = 0.0
            for a in range(int(q_ptr[i]), int(q_ptr[i + 1])):
                for b in range(int(h_ptr[j]), int(h_ptr[j + 1])):
                    best = max(best, grid_iou(qbox[a], hbox[b], n))
            out[i, j] = best
    return out


def token_points(cams, frame_cam, depth, order, grid, bs):
    """World points of the query chunk's tokens in curve order, and their
    block index: ``(points[L][3] (NaN where no depth), block[L])``."""
    T, H, W = grid
    L = T * H * W
    cells = np.asarray(order, dtype=np.int64)
    t, rem = cells // (H * W), cells % (H * W)
    h, w = rem // W, rem % W
    z = np.asarray(depth, dtype=np.float64).reshape(-1)[cells]
    pts = np.full((L, 3), np.nan)
    for g in range(L):
        if not (z[g] > 0.0):
            continue
        fx, fy, cx, cy, R, C = camera_parts(cams[int(frame_cam[t[g]])])
        u, v = w[g] + 0.5, h[g] + 0.5
        pc = np.array([(u - cx) * z[g] / fx, (v - cy) * z[g] / fy, z[g]])
        pts[g] = R @ pc + C
    return pts, np.arange(L) // bs


def in_slab(p, cam, geom) -> bool:
    """Whether world point p falls inside a slab spatially and in depth."""
    fx, fy, cx, cy, R, C = camera_parts(cam)
    u0, v0, u1, v1, zlo, zhi = (float(g) for g in geom)
    x, y, z = R.T @ (p - C)
    if not (z > 0.0):
        return False
    u, v = fx * x / z + cx, fy * y / z + cy
    return u0 <= u < u1 and v0 <= v < v1 and zlo <= z <= zhi


def coverage_scores(cams, frame_cam, depth, order, grid, bs, h_cam, h_geom, blocks=None) -> np.ndarray:
    """Coverage of the query blocks of the chunk by the historical slabs
    (all blocks, or those listed in ``blocks``, in that order)."""
    T, H, W = grid
    L = T * H * W
    nqb = -(-L // bs)
    pts, blk = token_points(cams, frame_cam, depth, order, grid, bs)
    which = range(nqb) if blocks is None else [int(b) for b in blocks]
    out = []
    for i in which:
        g0, g1 = i * bs, min(L, (i + 1) * bs)
        covered = 0
        for g in range(g0, g1):
            if np.isnan(pts[g, 0]):
                continue
            for s in range(len(h_cam)):
                if in_slab(pts[g], cams[int(h_cam[s])], h_geom[s]):
                    covered += 1
                    break
        out.append(covered / (g1 - g0) if g1 > g0 else 0.0)
    return np.array(out)
