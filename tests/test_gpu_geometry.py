"""GPU parity of the slab geometry against the oracle: overlap (float32 of
the float64 IoU) and coverage on the seeded camera path, at a short history
and at chunk 48 (sampled rows), grid sizes, skipped cameras, clamped ranges,
ragged blocks; then the chain slabs -> overlap and coverage -> materialised
routes."""

import numpy as np
import pytest
import torch

import workloads
from oracle import geometry as og
from oracle import materialize as om
from oracle.gilbert import gilbert_order

from helpers import assert_lists_equal, csr_lists, f64, need_gpu

pytestmark = pytest.mark.gpu


def _dev(g, dev):
    out = {}
    for k, v in g.items():
        out[k] = torch.from_numpy(np.ascontiguousarray(v)).to(dev) if isinstance(v, np.ndarray) else v
    return out


def _ulp_equal(got, ref64):
    """float32 results against the float64 oracle rounded to float32: equal,
    or one float32 ulp apart where the float64 values straddle a rounding
    boundary (the two sides sum in different orders)."""
    ref = ref64.astype(np.float32)
    diff = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    tol = np.spacing(np.maximum(np.abs(ref), np.float32(1e-30))).astype(np.float64)
    assert np.all(diff <= tol), (np.max(diff), np.argmax(diff))
    assert np.array_equal(got > 0, ref > 0)
    return int(np.sum(diff > 0))


@pytest.mark.parametrize("grid_n", [8, 4, 13])
def test_slab_overlap_matches_oracle(grid_n):
    dev = need_gpu()
    import block_sparse_attention_gilbert_amd as bsa
    g = workloads.geometry_inputs(3, 37)
    d = _dev(g, dev)
    ov = bsa.slab_overlap(d["cams"], d["q_ptr"], d["q_cam"], d["q_geom"], d["h_ptr"], d["h_cam"], d["h_geom"],
                          grid_n=grid_n)
    torch.cuda.synchronize()
    rows = range(37) if grid_n == 8 else range(0, 37, 6)
    q_ptr = g["q_ptr"]
    ref = np.stack([og.overlap_matrix(g["cams"], q_ptr[i:i + 2] - q_ptr[i], g["q_cam"][q_ptr[i]:],
                                      g["q_geom"][q_ptr[i]:], g["h_ptr"], g["h_cam"], g["h_geom"], n=grid_n)[0]
                    for i in rows])
    got = ov.cpu().numpy()[list(rows)]
    n_ulp = _ulp_equal(got, ref)
    print("grid %d: %d of %d pairs positive, %d one ulp apart" % (grid_n, int((got > 0).sum()), got.size, n_ulp))
    assert (got > 0).sum() > 10
    assert np.all(ov.cpu().numpy()[:, 3 * 37:] == 0.0)       # the query chunk's own blocks carry no slab


def test_slab_overlap_and_coverage_at_chunk_48_sampled():
    dev = need_gpu()
    import block_sparse_attention_gilbert_amd as bsa
    g = workloads.geometry_inputs(47, 37)
    d = _dev(g, dev)
    ov = bsa.slab_overlap(d["cams"], d["q_ptr"], d["q_cam"], d["q_geom"], d["h_ptr"], d["h_cam"], d["h_geom"])
    perm, _ = bsa.gilbert_index(*g["grid"], device=dev)
    cov = bsa.slab_coverage(d["cams"], perm, g["grid"], d["frame_cam"], d["depth"], d["h_cam"], d["h_geom"],
                            block=128)
    torch.cuda.synchronize()
    assert ov.shape == (37, 1776)
    q_ptr = g["q_ptr"]
    for i in (0, 17, 36):
        ref = og.overlap_matrix(g["cams"], q_ptr[i:i + 2] - q_ptr[i], g["q_cam"][q_ptr[i]:], g["q_geom"][q_ptr[i]:],
                                g["h_ptr"], g["h_cam"], g["h_geom"])[0]
        _ulp_equal(ov[i].cpu().numpy(), ref)
    order = gilbert_order(*g["grid"])[0]
    blocks = [5, 30]
    ref_cov = og.coverage_scores(g["cams"], g["frame_cam"], g["depth"], order, g["grid"], 128, g["h_cam"],
                                 g["h_geom"], blocks=blocks)
    assert np.array_equal(cov.cpu().numpy()[blocks], ref_cov.astype(np.float32))


@pytest.mark.parametrize("block", [128, 64, 1, 200, 300])
def test_slab_coverage_matches_oracle(block):
    dev = need_gpu()
    import block_sparse_attention_gilbert_amd as bsa
    grid = (3, 30, 52) if block in (128, 64, 300) else (2, 6, 9)
    g = workloads.geometry_inputs(3, 37, grid=grid)
    d = _dev(g, dev)
    perm, _ = bsa.gilbert_index(*grid, device=dev)
    cov = bsa.slab_coverage(d["cams"], perm, grid, d["frame_cam"], d["depth"], d["h_cam"], d["h_geom"], block=block)
    torch.cuda.synchronize()
    order = gilbert_order(*grid)[0]
    ref = og.coverage_scores(g["cams"], g["frame_cam"], g["depth"], order, grid, block, g["h_cam"], g["h_geom"])
    assert np.array_equal(cov.cpu().numpy(), ref.astype(np.float32))
    if grid == (3, 30, 52):
        assert 0.0 < ref.max() and ref.min() == 0.0          # the top rows have no depth


def test_slab_edge_cases():
    """Cameras outside [0, n_cams) are skipped, ranges past the slab count
    are clamped, blocks without slabs give 0, grid_n = 1, no historical slab
    at all gives zero coverage."""
    dev = need_gpu()
    import block_sparse_attention_gilbert_amd as bsa
    g = workloads.geometry_inputs(2, 37)
    h_cam = g["h_cam"].copy()
    bad = [0, 3, 7]
    h_cam[bad] = [-1, 99, len(g["cams"])]
    h_ptr = g["h_ptr"].copy()
    n_h = len(h_cam)
    h_ptr_long = h_ptr.copy()
    h_ptr_long[-1] = n_h + 50                                # past the end: clamped
    d = _dev(dict(g, h_cam=h_cam, h_ptr=h_ptr_long), dev)
    for n in (8, 1):
        ov = bsa.slab_overlap(d["cams"], d["q_ptr"], d["q_cam"], d["q_geom"], d["h_ptr"], d["h_cam"], d["h_geom"],
                              grid_n=n)
        torch.cuda.synchronize()
        # the oracle over the same slabs with the skipped ones removed
        keep = np.ones(n_h, dtype=bool)
        keep[bad] = False
        new_ptr = np.array([keep[:p].sum() for p in h_ptr], dtype=np.int32)
        q_ptr = g["q_ptr"]
        for i in (0, 9, 36):
            ref = og.overlap_matrix(g["cams"], q_ptr[i:i + 2] - q_ptr[i], g["q_cam"][q_ptr[i]:],
                                    g["q_geom"][q_ptr[i]:], new_ptr, g["h_cam"][keep], g["h_geom"][keep], n=n)[0]
            _ulp_equal(ov[i].cpu().numpy(), ref)
    perm, _ = bsa.gilbert_index(*g["grid"], device=dev)
    empty_cam = torch.zeros(0, dtype=torch.int32, device=dev)
    empty_geom = torch.zeros((0, 6), dtype=torch.float64, device=dev)
    cov = bsa.slab_coverage(d["cams"], perm, g["grid"], d["frame_cam"], d["depth"], empty_cam, empty_geom, block=128)
    torch.cuda.synchronize()
    assert torch.all(cov == 0)


def test_slabs_to_materialised_routes():
    """The chain of the pages' Steps 3-5 on one chunk: overlap and coverage
    from the slabs on the GPU, then the materialised routes; lists equal the
    oracle chain's."""
    dev = need_gpu()
    import block_sparse_attention_gilbert_amd as bsa
    c = 4
    w = workloads.c4(c=c, heads=[3, 30])
    g = workloads.geometry_inputs(c - 1, w.nqb)
    d = _dev(g, dev)
    perm, inv = bsa.gilbert_index(*g["grid"], device=dev)
    ov = bsa.slab_overlap(d["cams"], d["q_ptr"], d["q_cam"], d["q_geom"], d["h_ptr"], d["h_cam"], d["h_geom"])
    cov = bsa.slab_coverage(d["cams"], perm, g["grid"], d["frame_cam"], d["depth"], d["h_cam"], d["h_geom"],
                            block=w.bs)
    window, wlen = bsa.gilbert_block_window(perm, inv, g["grid"], block=w.bs, q_chunk=c - 1)
    prev = ((c - 2) * w.nqb, (c - 1) * w.nqb)
    r = bsa.route_materialize(w.q.to(dev), w.k.to(dev), block=w.bs, nqb=w.nqb, nkb=w.nkb, scale=w.scale,
                              q_block_len=torch.from_numpy(w.q_len).to(dev),
                              kv_block_len=torch.from_numpy(w.k_len).to(dev), overlap=ov, coverage=cov,
                              prev_blocks=prev, window=window, window_len=wlen, k_cov=80, k_unc=150, mass=0.9)
    torch.cuda.synchronize()
    got = csr_lists(r["row_ptr"], r["col_idx"], w.heads, w.nqb)
    order = gilbert_order(*g["grid"])[0]
    ref_ov = og.overlap_matrix(g["cams"], g["q_ptr"], g["q_cam"], g["q_geom"], g["h_ptr"], g["h_cam"], g["h_geom"])
    ref_cov = og.coverage_scores(g["cams"], g["frame_cam"], g["depth"], order, g["grid"], w.bs, g["h_cam"],
                                 g["h_geom"])
    _ulp_equal(ov.cpu().numpy(), ref_ov)
    assert np.array_equal(cov.cpu().numpy(), ref_cov.astype(np.float32))
    win = om.block_window(order, g["grid"], w.bs, c - 1)
    print("covered query blocks: %d of %d" % (int((ref_cov.astype(np.float32) >= np.float32(0.9)).sum()), w.nqb))
    for hi in range(w.heads):
        # the oracle's own float64 coverage (it takes the decision in float32)
        ref = om.materialize_head(f64(w.q[hi]), f64(w.k[hi]), w.q_len, w.k_len, w.bs, scale=w.scale,
                                  coverage=ref_cov, k_cov=80, k_unc=150, mass=0.9,
                                  prev_blocks=prev, windows=win, overlap=ref_ov.astype(np.float32),
                                  lam=w.lam, tau=w.tau, g_ref=w.g_ref)
        assert_lists_equal(got[hi], ref["lists"], "head %d" % hi)
