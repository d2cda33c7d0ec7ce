"""Seeded synthetic workloads for routed block-sparse attention.

This module only draws inputs.  It holds none of the method's arithmetic (no
curve, no pooling, no routing, no attention): the oracle and the HIP path
both take what it returns, and each computes everything else on its own.

The workloads stand in for per-layer attention shapes of a chunked, Wan-style
video DiT with a 3 x 30 x 52 latent chunk (4680 tokens) and 48-chunk
rollouts, as in Velox's runtime traces [Velox: Spatial Memory Makes World
Models Efficient -- Main Findings; Methodology, closing paragraph].  No
dataset is used or reproduced.

Every random piece is drawn from its own PCG64 stream keyed by
``(seed, tag, head, chunk)``, so a piece (one head of one chunk) can be
regenerated on its own and is identical to the same piece of a full draw.
Normal draws are float32; sums with offsets are formed in float32 and then
rounded to bf16 (round to nearest even) for bf16 workloads.  Padded rows
(past a chunk's last valid token) are exact zeros.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

# stream tags
(T_QNOISE, T_KNOISE, T_V, T_QOFF, T_KOFF, T_OVERLAP, T_ZROWS, T_KROW, T_FIELD, T_MIXQ, T_MIXK, T_COVER, T_SLAB,
 T_DEPTH) = range(14)

CHUNK_GRID = (3, 30, 52)           # latent frames x height x width of one chunk
CHUNK_TOKENS = 3 * 30 * 52         # 4680


def _rng(*key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _parallel(fn, items):
    items = list(items)
    if len(items) <= 1:
        return [fn(x) for x in items]
    with ThreadPoolExecutor(_threads()) as ex:
        return list(ex.map(fn, items))


def block_lengths(tokens: int, bs: int) -> np.ndarray:
    """Valid tokens of each ``bs``-token block holding ``tokens`` tokens
    (input structure: the last block of a chunk is partly padding)."""
    nb = -(-tokens // bs)
    return np.array([min(bs, tokens - b * bs) for b in range(nb)], dtype=np.int32)


@dataclass
class Workload:
    """Inputs of one configuration.

    Blocked tensors are head-major ``[heads][n_blocks*bs][d]`` (``torch``, CPU,
    ``dtype``).  For raster workloads ``q``/``k``/``v`` are None and
    ``q_raster[L][heads][d]``, ``k_raster``/``v_raster[n_chunks][L][heads][d]``
    are given instead, with ``grid`` the chunk's latent grid."""
    name: str
    dtype: torch.dtype
    heads: int
    d: int
    bs: int
    q_len: np.ndarray
    k_len: np.ndarray
    k_per_row: np.ndarray                 # [heads*nqb] int32 budgets
    scale: float
    q: Optional[torch.Tensor] = None
    k: Optional[torch.Tensor] = None
    v: Optional[torch.Tensor] = None
    overlap: Optional[np.ndarray] = None  # [nqb][n_candidates] float32
    coverage: Optional[np.ndarray] = None  # [nqb] float32
    lam: float = 2.0
    g_ref: float = 0.2
    tau: float = 0.1
    n_dense_tail: int = 0
    grid: Optional[tuple] = None
    q_raster: Optional[torch.Tensor] = None
    k_raster: Optional[torch.Tensor] = None
    v_raster: Optional[torch.Tensor] = None
    head_ids: list = field(default_factory=list)
    notes: str = ""

    @property
    def nqb(self) -> int:
        return len(self.q_len)

    @property
    def nkb(self) -> int:
        return len(self.k_len)

    @property
    def n_candidates(self) -> int:
        return self.nkb - self.n_dense_tail


def _to_dtype(x32: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    return t.to(dtype) if dtype != torch.float32 else t.clone()


def _blocked_tensor(seed, noise_tag, off_tag, heads, head_ids, n_chunks, lens, bs, d,
                    dtype, offset_sd):
    """``[len(head_ids)][n_chunks*len(lens)*bs][d]`` with N(0,1) noise plus a
    per-(head, block) N(0, offset_sd^2) offset vector, zero padded rows."""
    nbc = len(lens)
    rows_c = nbc * bs
    out = torch.zeros((len(head_ids), n_chunks * rows_c, d), dtype=dtype)
    valid = np.zeros(rows_c, dtype=bool)
    for b, n in enumerate(lens):
        valid[b * bs: b * bs + n] = True

    def piece(job):
        hi, c = job
        h = head_ids[hi]
        x = np.zeros((rows_c, d), dtype=np.float32)
        noise = _rng(seed, noise_tag, h, c).standard_normal((int(valid.sum()), d), dtype=np.float32)
        x[valid] = noise
        if off_tag is not None and offset_sd > 0:
            off = _rng(seed, off_tag, h, c).standard_normal((nbc, d), dtype=np.float32) * np.float32(offset_sd)
            x += np.repeat(off, bs, axis=0) * valid[:, None]
        out[hi, c * rows_c:(c + 1) * rows_c, :] = _to_dtype(x, dtype)
        return None

    _parallel(piece, [(hi, c) for hi in range(len(head_ids)) for c in range(n_chunks)])
    return out


def c1() -> Workload:
    """Tiny fp32 routed attention: 1 head, d 64, 4 query blocks and 16 KV
    blocks of 64 tokens, top-K 4, no bias, N(0,1) plus N(0, 0.5^2) per-block
    offsets on Q and K, scale 1/8."""
    seed, H, d, bs = 1001, 1, 64, 64
    qlen = np.full(4, 64, dtype=np.int32)
    klen = np.full(16, 64, dtype=np.int32)
    heads = [0]
    q = _blocked_tensor(seed, T_QNOISE, T_QOFF, H, heads, 1, qlen, bs, d, torch.float32, 0.5)
    k = _blocked_tensor(seed, T_KNOISE, T_KOFF, H, heads, 1, klen, bs, d, torch.float32, 0.5)
    v = _blocked_tensor(seed, T_V, None, H, heads, 1, klen, bs, d, torch.float32, 0.0)
    return Workload("C1-tiny-fp32", torch.float32, H, d, bs, qlen, klen,
                    np.full(H * 4, 4, dtype=np.int32), 1.0 / math.sqrt(d), q, k, v,
                    head_ids=heads)


def c2(heads=None) -> Workload:
    """Wan-1.3B-like layer, bf16: 12 heads, d 128, a 4680-token query chunk in
    37 blocks of 128 (the last holds 72 tokens), 143 full history blocks,
    top-K 50, N(0,1) plus N(0, 0.5^2) per-block offsets, no bias."""
    seed, H, d, bs = 1002, 12, 128, 128
    head_ids = list(range(H)) if heads is None else list(heads)
    qlen = block_lengths(CHUNK_TOKENS, bs)
    klen = np.full(143, bs, dtype=np.int32)
    q = _blocked_tensor(seed, T_QNOISE, T_QOFF, H, head_ids, 1, qlen, bs, d, torch.bfloat16, 0.5)
    k = _blocked_tensor(seed, T_KNOISE, T_KOFF, H, head_ids, 1, klen, bs, d, torch.bfloat16, 0.5)
    v = _blocked_tensor(seed, T_V, None, H, head_ids, 1, klen, bs, d, torch.bfloat16, 0.0)
    return Workload("C2-wan1.3b-bf16", torch.bfloat16, len(head_ids), d, bs, qlen, klen,
                    np.full(len(head_ids) * len(qlen), 50, dtype=np.int32), 1.0 / math.sqrt(d),
                    q, k, v, head_ids=head_ids)


def c3(heads=None) -> Workload:
    """C2's tensors plus a per-(query block, KV block) overlap ~ Beta(0.5, 2)
    drawn in float64 and stored as float32, with 11 of the 37 query-block
    rows set to zero (forcing the unbiased fallback); lambda 2, g_ref 0.2,
    tau 0.1, top-K 50."""
    w = c2(heads)
    rng = _rng(1003, T_OVERLAP, 0, 0)
    g = rng.beta(0.5, 2.0, size=(w.nqb, w.nkb)).astype(np.float32)
    zero_rows = _rng(1003, T_ZROWS, 0, 0).choice(w.nqb, 11, replace=False)
    g[zero_rows, :] = 0.0
    w.name = "C3-geometric-bias-bf16"
    w.overlap = g
    w.notes = "zero rows: " + ",".join(str(int(i)) for i in sorted(zero_rows))
    return w


def c4(c: int = 48, heads=None, n_store_chunks: Optional[int] = None, chunk_lens=None) -> Workload:
    """Growing-context 14B-like layer, bf16: 40 heads, d 128, a 4680-token
    query chunk (37 blocks of 128), KV history of ``c`` chunks of 4680 tokens
    (37 blocks each, the last of each chunk holds 72 tokens); N(0,1) plus
    N(0, 0.5^2) per-block offsets on Q and K; fixed top-K 50.

    The KV store is drawn chunk by chunk, so the history at ``c`` is the
    prefix of the history at any larger ``c`` (the store grows by appending).
    ``n_store_chunks`` (default ``c``) sets how many chunks are allocated.
    ``chunk_lens`` replaces the per-chunk block lengths (e.g. those of a
    fixed-tile layout: the same draws, blocks of other valid lengths)."""
    seed, H, d, bs = 1004, 40, 128, 128
    head_ids = list(range(H)) if heads is None else list(heads)
    n_store = c if n_store_chunks is None else max(c, n_store_chunks)
    qlen = block_lengths(CHUNK_TOKENS, bs) if chunk_lens is None else np.asarray(chunk_lens, dtype=np.int32)
    klen_chunk = qlen.copy()
    q = _blocked_tensor(seed, T_QNOISE, T_QOFF, H, head_ids, 1, qlen, bs, d, torch.bfloat16, 0.5)
    k = _blocked_tensor(seed, T_KNOISE, T_KOFF, H, head_ids, n_store, klen_chunk, bs, d, torch.bfloat16, 0.5)
    v = _blocked_tensor(seed, T_V, None, H, head_ids, n_store, klen_chunk, bs, d, torch.bfloat16, 0.0)
    klen = np.tile(klen_chunk, c).astype(np.int32)
    rows = c * len(klen_chunk) * bs
    return Workload(f"C4-growing-context-c{c}-bf16", torch.bfloat16, len(head_ids), d, bs, qlen, klen,
                    np.full(len(head_ids) * len(qlen), 50, dtype=np.int32), 1.0 / math.sqrt(d),
                    q, k[:, :rows, :], v[:, :rows, :], head_ids=head_ids,
                    notes=f"store chunks allocated: {n_store}")


def route_inputs(q_len: np.ndarray, nkb: int):
    """Inputs of route materialisation for one query chunk: a coverage per
    query block and an overlap with every KV block of the history.

    Coverage is a share of a block's valid tokens, n / q_len with n =
    round(u * q_len), u ~ Beta(4, 0.7) (P(u >= 0.9) is about 0.5); three
    blocks are set to exactly 0.9 in float32 (just below 0.9 in float64) and
    two to 1.  Overlap ~ Beta(0.5, 2) in float64, stored as float32.
    Returns ``(coverage[nqb], overlap[nqb][nkb])``, both float32."""
    q_len = np.asarray(q_len)
    nqb = len(q_len)
    rng = _rng(1005, T_COVER, 0, 0)
    u = rng.beta(4.0, 0.7, size=nqb)
    cov = np.round(u * q_len) / np.maximum(q_len, 1)
    pick = rng.choice(nqb, min(nqb, 5), replace=False)
    cov[pick[:3]] = np.float32(0.9)
    cov[pick[3:]] = 1.0
    overlap = _rng(1005, T_OVERLAP, nkb, 0).beta(0.5, 2.0, size=(nqb, nkb)).astype(np.float32)
    return cov.astype(np.float32), overlap


def _rotation(yaw: float, pitch: float) -> np.ndarray:
    cy_, sy = math.cos(yaw), math.sin(yaw)
    cp, sp = math.cos(pitch), math.sin(pitch)
    ry = np.array([[cy_, 0.0, sy], [0.0, 1.0, 0.0], [-sy, 0.0, cy_]])
    rx = np.array([[1.0, 0.0, 0.0], [0.0, cp, -sp], [0.0, sp, cp]])
    return ry @ rx


# A synthetic scene for the slab geometry: a corridor 12 units wide along
# +z (walls x = -6 and x = +6, from the floor y = +1.5 up to y = -3; the
# camera's y axis points down), a floor, and an end wall at z = 40; rays
# that leave over the walls see sky (no depth).
_ROOM_X, _FLOOR_Y, _TOP_Y, _END_Z = 6.0, 1.5, -3.0, 40.0


def _camera(g: int, grid) -> np.ndarray:
    T, H, W = grid
    cam = np.zeros(16)
    R = _rotation(0.3 * math.sin(0.07 * g), 0.05 * math.sin(0.11 * g))
    cam[:4] = (36.0, 36.0, W / 2.0, H / 2.0)
    cam[4:13] = R.reshape(-1)
    cam[13:16] = (1.5 * math.sin(0.02 * g), 0.0, 0.12 * g)
    return cam


def _raycast(cam: np.ndarray, u: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Camera depth of the scene along the rays through token coordinates
    (u, v); NaN where the ray sees sky."""
    fx, fy, cx, cy = cam[:4]
    R, C = cam[4:13].reshape(3, 3), cam[13:16]
    dc = np.stack([(u - cx) / fx, (v - cy) / fy, np.ones_like(u)], axis=-1)
    dw = dc @ R.T
    best = np.full(u.shape, np.inf)
    with np.errstate(divide="ignore", invalid="ignore"):
        for axis, plane in ((0, -_ROOM_X), (0, _ROOM_X), (1, _FLOOR_Y), (2, _END_Z)):
            t = (plane - C[axis]) / dw[..., axis]
            hit = C + t[..., None] * dw
            ok = (t > 0) & np.isfinite(t)
            ok &= (hit[..., 0] >= -_ROOM_X - 1e-9) & (hit[..., 0] <= _ROOM_X + 1e-9)
            ok &= (hit[..., 1] >= _TOP_Y) & (hit[..., 1] <= _FLOOR_Y + 1e-9) & (hit[..., 2] <= _END_Z + 1e-9)
            best = np.where(ok & (t < best), t, best)
    return np.where(np.isfinite(best), best, np.nan)   # dc has unit camera z, so t is the camera depth


def _slabs(rng, n_blocks, cam_of_frame, cams, grid):
    """Slabs of ``n_blocks`` blocks, standing in for the reconstruction of
    the pages' Step 1: per block 1-3 distinct frames, each a token rectangle
    (2-7 rows, 4-13 columns, at most the grid) whose depth interval is the
    10th-90th percentile of the scene depth at its token centres, widened
    to a thickness of at least 0.1; a rectangle with fewer than 4 depth
    samples or a spread above 60 % of its median depth gives no slab."""
    T, H, W = grid
    ptr, cam, geom = [0], [], []
    for b in range(n_blocks):
        k = int(rng.integers(1, 4))
        for f in sorted(rng.choice(T, size=min(k, T), replace=False)):
            hh = int(rng.integers(min(2, H), min(8, H + 1)))
            ww = int(rng.integers(min(4, W), min(14, W + 1)))
            v0, u0 = int(rng.integers(0, H - hh + 1)), int(rng.integers(0, W - ww + 1))
            ci = cam_of_frame(b, int(f))
            vv, uu = np.meshgrid(np.arange(v0, v0 + hh) + 0.5, np.arange(u0, u0 + ww) + 0.5, indexing="ij")
            z = _raycast(cams[ci], uu.reshape(-1), vv.reshape(-1))
            z = z[np.isfinite(z)]
            if z.size < 4:
                continue
            lo, hi, med = np.percentile(z, 10), np.percentile(z, 90), np.median(z)
            if hi - lo > 0.6 * med:
                continue
            if hi - lo < 0.1:
                mid = (lo + hi) / 2.0
                lo, hi = mid - 0.05, mid + 0.05
            cam.append(ci)
            geom.append((u0, v0, u0 + ww, v0 + hh, lo, hi))
        ptr.append(len(cam))
    return (np.asarray(ptr, dtype=np.int32), np.asarray(cam, dtype=np.int32),
            np.asarray(geom, dtype=np.float64).reshape(-1, 6))


def geometry_inputs(q_chunk: int, nbc: int, grid=CHUNK_GRID):
    """Inputs of the geometric overlap and coverage for query chunk
    ``q_chunk`` of a rollout: cameras of every frame so far, frustum slabs
    of the historical blocks (chunks 0 .. q_chunk-1; the query chunk's own
    blocks have none), slabs of the query blocks, and a depth per query
    token.

    A camera moves through a synthetic corridor (``_raycast``): at latent
    frame g it sits at (1.5 sin(0.02 g), 0, 0.12 g) with yaw 0.3 sin(0.07 g)
    and pitch 0.05 sin(0.11 g); fx = fy = 36,
    principal point at the grid centre, token units; cameras are float64
    [frames][16] (fx, fy, cx, cy, world-from-camera R row-major, centre).
    Slabs: ``_slabs``.  Query depth: the scene depth at each token centre of
    the query chunk times (1 + N(0, 0.01)), NaN over sky, float32 raster
    [T][H][W]."""
    T, H, W = grid
    n_frames = T * (q_chunk + 1)
    cams = np.stack([_camera(g, grid) for g in range(n_frames)])
    rng = _rng(1006, T_SLAB, q_chunk, 0)
    h_ptr, h_cam, h_geom = _slabs(rng, q_chunk * nbc, lambda b, f: T * (b // nbc) + f, cams, grid)
    # the query chunk's own blocks carry no historical slab
    h_ptr = np.concatenate([h_ptr, np.full(nbc, h_ptr[-1], dtype=np.int32)])
    q_ptr, q_cam, q_geom = _slabs(_rng(1006, T_SLAB, q_chunk, 1), nbc, lambda b, f: T * q_chunk + f, cams, grid)
    vv, uu = np.meshgrid(np.arange(H) + 0.5, np.arange(W) + 0.5, indexing="ij")
    noise = _rng(1006, T_DEPTH, q_chunk, 0).normal(0.0, 0.01, size=(T, H, W))
    depth = np.stack([_raycast(cams[T * q_chunk + t], uu, vv) for t in range(T)]) * (1.0 + noise)
    return dict(cams=cams, h_ptr=h_ptr, h_cam=h_cam, h_geom=h_geom, q_ptr=q_ptr, q_cam=q_cam, q_geom=q_geom,
                frame_cam=np.arange(T * q_chunk, T * (q_chunk + 1), dtype=np.int32),
                depth=depth.astype(np.float32), grid=tuple(grid))


def c4_routes(c: int = 48, heads=None, n_store_chunks: Optional[int] = None) -> Workload:
    """C4 plus the inputs of route materialisation (``route_inputs``)."""
    w = c4(c, heads, n_store_chunks)
    w.coverage, w.overlap = route_inputs(w.q_len, w.nkb)
    w.name = f"C4R-materialised-routes-c{c}-bf16"
    return w


def _field_params(seed):
    """Rank-8 smooth field: each component is a sum of 4 cosines with integer
    wave numbers in {0,1,2}^3 (not all zero) over (frame/144, y/30, x/52)
    and uniform random phases."""
    rng = _rng(seed, T_FIELD, 0, 0)
    waves = []
    for _r in range(8):
        comps = []
        for _m in range(4):
            while True:
                kk = rng.integers(0, 3, size=3)
                if kk.any():
                    break
            phase = rng.uniform(0.0, 2.0 * math.pi)
            comps.append((int(kk[0]), int(kk[1]), int(kk[2]), float(phase)))
        waves.append(comps)
    return waves


def _field_values(waves, frames, n_frames_total, Hh, Ww):
    """Field components ``[len(frames)*Hh*Ww][8]`` (float64, raster order)
    at the given global frame indices, normalised to unit variance over the
    whole rollout grid."""
    tt = np.asarray(frames, dtype=np.float64)[:, None, None] / n_frames_total
    yy = np.arange(Hh, dtype=np.float64)[None, :, None] / Hh
    xx = np.arange(Ww, dtype=np.float64)[None, None, :] / Ww
    out = np.zeros((len(frames), Hh, Ww, 8))
    for r, comps in enumerate(waves):
        f = np.zeros((len(frames), Hh, Ww))
        for (kt, ky, kx, ph) in comps:
            f = f + np.cos(2.0 * math.pi * (kt * tt + ky * yy + kx * xx) + ph)
        out[..., r] = f
    return out.reshape(-1, 8)


def c5(heads=None, n_chunks: int = 48) -> Workload:
    """Ragged routes, bf16: 40 heads, d 128, 64-token blocks, 48 chunks of a
    3 x 30 x 52 grid (47 history chunks + the current one).  Q and K are a
    rank-8 spatially smooth field over the rollout's latent grid mixed per
    head (mixing ~ N(0, 1/8)) plus N(0, 0.3^2) noise; V ~ N(0,1).  Tensors are
    raster token-major per chunk.  Budgets K ~ uniform integer in [8, 143]
    per (head, query block) over the history; the current chunk's 74 blocks
    are attended densely."""
    seed, H, d, bs = 1005, 40, 128, 64
    head_ids = list(range(H)) if heads is None else list(heads)
    T, Hh, Ww = CHUNK_GRID
    L = CHUNK_TOKENS
    n_frames_total = T * 48
    waves = _field_params(seed)
    # normalisation over the whole 48-chunk rollout grid
    all_f = _field_values(waves, range(n_frames_total), n_frames_total, Hh, Ww)
    norm = all_f.std(axis=0)
    mix_q = np.stack([_rng(seed, T_MIXQ, h, 0).standard_normal((8, d)) / math.sqrt(8.0) for h in range(H)])
    mix_k = np.stack([_rng(seed, T_MIXK, h, 0).standard_normal((8, d)) / math.sqrt(8.0) for h in range(H)])
    mix_q = mix_q[head_ids]
    mix_k = mix_k[head_ids]
    nh = len(head_ids)

    def field_chunk(c):
        f = _field_values(waves, range(T * c, T * c + T), n_frames_total, Hh, Ww) / norm
        return f.astype(np.float32)

    def make(mix, noise_tag, chunks, noise_sd):
        out = torch.empty((len(chunks), L, nh, d), dtype=torch.bfloat16)

        def piece(job):
            ci, hi = job
            c = chunks[ci]
            base = field_chunk(c) @ mix[hi].astype(np.float32) if mix is not None else 0.0
            noise = _rng(seed, noise_tag, head_ids[hi], c).standard_normal((L, d), dtype=np.float32)
            x = base + noise * np.float32(noise_sd)
            out[ci, :, hi, :] = _to_dtype(x, torch.bfloat16)
            return None

        _parallel(piece, [(ci, hi) for ci in range(len(chunks)) for hi in range(nh)])
        return out

    cur = n_chunks - 1
    q_r = make(mix_q, T_QNOISE, [cur], 0.3)[0]
    k_r = make(mix_k, T_KNOISE, list(range(n_chunks)), 0.3)
    v_r = make(None, T_V, list(range(n_chunks)), 1.0)
    nbc = -(-L // bs)
    qlen = block_lengths(L, bs)
    klen = np.tile(block_lengths(L, bs), n_chunks).astype(np.int32)
    kr = _rng(seed, T_KROW, 0, 0).integers(8, 144, size=(H, nbc)).astype(np.int32)[head_ids]
    return Workload("C5-ragged-structured-bf16", torch.bfloat16, nh, d, bs, qlen, klen,
                    kr.reshape(-1), 1.0 / math.sqrt(d), n_dense_tail=nbc, grid=CHUNK_GRID,
                    q_raster=q_r, k_raster=k_r, v_raster=v_r, head_ids=head_ids)


REGISTRY = {"C1": c1, "C2": c2, "C3": c3, "C4": c4, "C5": c5, "C4R": c4_routes}


def get(name: str, **kw) -> Workload:
    return REGISTRY[name](**kw)
