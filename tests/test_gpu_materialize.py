"""GPU parity of the local-window builder and of route materialisation
against the oracle: windows and lists bit-exact, on the chunk grid and on
small ragged cases (empty query blocks, empty KV blocks, out-of-range window
entries, clipped ranges, every budget and mass extreme)."""

import numpy as np
import pytest
import torch

import workloads
from oracle import materialize as om
from oracle import route as oroute
from oracle.gilbert import gilbert_order

from helpers import assert_lists_equal, csr_lists, f64, need_gpu

pytestmark = pytest.mark.gpu


def _window_rows(win, stride):
    """Padded int32 rows + lengths of a list of window arrays (inputs)."""
    rows = np.full((len(win), stride), -7, dtype=np.int32)
    lens = np.zeros(len(win), dtype=np.int32)
    for b, wb in enumerate(win):
        rows[b, :len(wb)] = wb
        lens[b] = len(wb)
    return rows, lens


@pytest.mark.parametrize("grid,block,q_chunk", [((3, 30, 52), 128, 0), ((3, 30, 52), 128, 3),
                                                ((3, 30, 52), 64, 1), ((2, 5, 7), 3, 2), ((4, 3, 5), 1, 1)])
def test_block_window_matches_oracle(grid, block, q_chunk):
    dev = need_gpu()
    import block_sparse_attention_gilbert_amd as bsa
    T, H, W = grid
    order = gilbert_order(T, H, W)[0]
    perm, inv = bsa.gilbert_index(T, H, W, device=dev)
    assert np.array_equal(perm.cpu().numpy(), order)
    window, wlen = bsa.gilbert_block_window(perm, inv, grid, block=block, q_chunk=q_chunk)
    torch.cuda.synchronize()
    ref = om.block_window(order, grid, block, q_chunk)
    win, wl = window.cpu().numpy(), wlen.cpu().numpy()
    assert len(wl) == len(ref)
    for b, rb in enumerate(ref):
        assert np.array_equal(win[b, :wl[b]], rb), (b, win[b, :wl[b]], rb)


def _materialize_gpu(bsa, w, dev, q, k, ql, kl, **kw):
    cov = None if w.coverage is None else torch.from_numpy(w.coverage).to(dev)
    ov = None if w.overlap is None else torch.from_numpy(w.overlap).to(dev)
    return bsa.route_materialize(q, k, block=w.bs, nqb=w.nqb, nkb=w.nkb, scale=w.scale, q_block_len=ql,
                                 kv_block_len=kl, overlap=ov, lam=w.lam, g_ref=w.g_ref, tau=w.tau, coverage=cov,
                                 **kw)


@pytest.mark.parametrize("c,heads", [(4, [0, 21, 39]), (16, [7])])
def test_materialize_parity_growing_history(c, heads):
    """Query chunk c-1 over a c-chunk history: reservation of chunk c-2,
    fill to K_cov = 80, mass prefix (0.9) capped at K_unc = 150, the window
    of the chunk grid, reference blocks 0..3."""
    dev = need_gpu()
    import block_sparse_attention_gilbert_amd as bsa
    w = workloads.c4_routes(c=c, heads=heads)
    nbc = w.nqb
    qc = c - 1
    win = om.block_window(gilbert_order(*workloads.CHUNK_GRID)[0], workloads.CHUNK_GRID, w.bs, qc)
    rows, lens = _window_rows(win, 2 * nbc)
    q, k = w.q.to(dev), w.k.to(dev)
    ql = torch.from_numpy(w.q_len).to(dev)
    kl = torch.from_numpy(w.k_len).to(dev)
    prev, ref = ((qc - 1) * nbc, qc * nbc), (0, 4)
    r = _materialize_gpu(bsa, w, dev, q, k, ql, kl, k_cov=80, k_unc=150, mass=0.9, prev_blocks=prev,
                         window=torch.from_numpy(rows).to(dev), window_len=torch.from_numpy(lens).to(dev),
                         ref_blocks=ref, want_keys=True)
    torch.cuda.synchronize()
    got = csr_lists(r["row_ptr"], r["col_idx"], w.heads, w.nqb)
    sizes = []
    for hi in range(w.heads):
        ref_h = om.materialize_head(f64(w.q[hi]), f64(w.k[hi]), w.q_len, w.k_len, w.bs, scale=w.scale,
                                    coverage=w.coverage, k_cov=80, k_unc=150, mass=0.9, prev_blocks=prev,
                                    windows=win, ref_blocks=ref, overlap=w.overlap, lam=w.lam, tau=w.tau,
                                    g_ref=w.g_ref)
        assert_lists_equal(got[hi], ref_h["lists"], "head %d" % heads[hi])
        keys = r["sel_keys"][hi].cpu().numpy()
        assert np.allclose(keys, ref_h["kappa"], rtol=1e-12, atol=1e-12)
        sizes += [len(x) for x in ref_h["lists"]]
    print("c=%d list sizes min/mean/max %d/%.1f/%d" % (c, min(sizes), np.mean(sizes), max(sizes)))


def _small(seed, dtype, block=64, d=64):
    rng = np.random.default_rng(seed)
    heads, nqb, nkb = 2, 4, 20
    q = torch.from_numpy(rng.standard_normal((heads, nqb * block, d)).astype(np.float32)).to(dtype)
    base = rng.standard_normal((heads, nkb, 1, d)).astype(np.float32) * 1.5
    k = torch.from_numpy((rng.standard_normal((heads, nkb, block, d)).astype(np.float32) + base)
                         .reshape(heads, nkb * block, d)).to(dtype)
    q_len = np.array([block, 0, 17, block], dtype=np.int32)
    k_len = np.full(nkb, block, dtype=np.int32)
    k_len[[3, 9, 15]] = 0
    k_len[[5, 12]] = [1, 40]
    return heads, nqb, nkb, q, k, q_len, k_len


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_materialize_small_edge_cases(dtype):
    dev = need_gpu()
    import block_sparse_attention_gilbert_amd as bsa
    heads, nqb, nkb, q, k, q_len, k_len = _small(11, dtype)
    block, scale = 64, 0.125
    cov = np.array([1.0, 0.95, 0.2, 0.0], dtype=np.float32)
    ov = np.random.default_rng(12).beta(0.5, 2.0, size=(nqb, nkb)).astype(np.float32)
    stride = 6
    raw = [[0, 19, -1, 25, 0, 3], [7], [2, 2, 8, 30], [11, 12, 13, 14, 15, 16, 17, 18, 19]]
    rows = np.full((nqb, stride), -1, dtype=np.int32)
    lens = np.array([6, 1, 4, 9], dtype=np.int32)          # the last is clamped to the stride
    for i, x in enumerate(raw):
        rows[i, :min(stride, len(x))] = x[:stride]
    win_eff = [np.array(x[:stride]) for x in raw]
    dq, dk = q.to(dev), k.to(dev)
    ql, kl = torch.from_numpy(q_len).to(dev), torch.from_numpy(k_len).to(dev)
    cases = [dict(k_cov=6, k_unc=5, mass=0.5), dict(k_cov=6, k_unc=5, mass=1e-9), dict(k_cov=6, k_unc=256, mass=1.0),
             dict(k_cov=6, k_unc=256, mass=2.0), dict(k_cov=0, k_unc=0, mass=0.5), dict(k_cov=40, k_unc=3, mass=0.9),
             dict(k_cov=2, k_unc=7, mass=0.99)]
    for case in cases:
        for prev, ref in [((4, 8), (18, 100)), ((0, 0), (0, 0)), ((16, 40), (2, 2))]:
            r = bsa.route_materialize(dq, dk, block=block, nqb=nqb, nkb=nkb, scale=scale, q_block_len=ql,
                                      kv_block_len=kl, overlap=torch.from_numpy(ov).to(dev),
                                      coverage=torch.from_numpy(cov).to(dev), prev_blocks=prev,
                                      window=torch.from_numpy(rows).to(dev), window_len=torch.from_numpy(lens).to(dev),
                                      ref_blocks=ref, **case)
            torch.cuda.synchronize()
            got = csr_lists(r["row_ptr"], r["col_idx"], heads, nqb)
            for h in range(heads):
                ref_h = om.materialize_head(f64(q[h]), f64(k[h]), q_len, k_len, block, scale=scale, coverage=cov,
                                            prev_blocks=prev, windows=win_eff, ref_blocks=ref, overlap=ov, **case)
                assert_lists_equal(got[h], ref_h["lists"], "%s prev %s ref %s head %d" % (case, prev, ref, h))
                assert got[h][1].size == 0                        # query block without a valid token


def test_materialize_all_covered_is_the_top_k_router():
    """No coverage, no reservation, no window, no reference blocks: the
    plain top-K router's lists, and the same lists from the pooled-key
    cache on a second call."""
    dev = need_gpu()
    import block_sparse_attention_gilbert_amd as bsa
    w = workloads.c3(heads=[2, 9])
    q, k = w.q.to(dev), w.k.to(dev)
    ql = torch.from_numpy(w.q_len.astype(np.int32)).to(dev)
    kl = torch.from_numpy(w.k_len.astype(np.int32)).to(dev)
    ov = torch.from_numpy(w.overlap).to(dev)
    kpool = torch.full((w.heads, w.nkb + 5, w.d), float("nan"), dtype=torch.float64, device=dev)
    args = dict(block=w.bs, nqb=w.nqb, nkb=w.nkb, scale=w.scale, q_block_len=ql, kv_block_len=kl, overlap=ov,
                lam=w.lam, g_ref=w.g_ref, tau=w.tau, k_cov=50, k_unc=150, kpool=kpool)
    r1 = bsa.route_materialize(q, k, kpool_valid_blocks=0, **args)
    l1 = csr_lists(r1["row_ptr"], r1["col_idx"], w.heads, w.nqb)
    r2 = bsa.route_materialize(q, k, kpool_valid_blocks=w.nkb, **args)
    l2 = csr_lists(r2["row_ptr"], r2["col_idx"], w.heads, w.nqb)
    torch.cuda.synchronize()
    for h in range(w.heads):
        ref = oroute.route_head(f64(w.q[h]), f64(w.k[h]), w.q_len, w.k_len, w.bs, scale=w.scale,
                                k_per_row=np.full(w.nqb, 50), overlap=w.overlap, lam=w.lam, tau=w.tau,
                                g_ref=w.g_ref)
        assert_lists_equal(l1[h], ref["lists"], "head %d" % h)
        assert_lists_equal(l2[h], ref["lists"], "cached head %d" % h)


def test_pipeline_step_with_materialised_routes():
    """One call of the chunked pipeline with the materialised route (window
    rebuilt on the GPU inside the step): lists equal the oracle's, and the
    attention over them matches the oracle within the bf16 bounds."""
    dev = need_gpu()
    import block_sparse_attention_gilbert_amd as bsa
    from block_sparse_attention_gilbert_amd.pipeline import RoutedAttention
    from oracle import attention as oatt

    from helpers import BF16_MAX_ABS, BF16_MEAN_ABS, err_summary, valid_rows

    c = 3
    w = workloads.c4_routes(c=c, heads=[0, 5])
    ra = RoutedAttention(workloads.CHUNK_GRID, w.heads, w.d, w.bs, c, device=dev, k_store=w.k.contiguous().to(dev),
                         v_store=w.v.contiguous().to(dev))
    ks, vs = ra.slot(c - 1)
    q_r = bsa.gilbert_perm(w.q.to(dev), ra.perm, block=w.bs, inverse=True)
    k_r = bsa.gilbert_perm(ks, ra.perm, block=w.bs, inverse=True)
    v_r = bsa.gilbert_perm(vs, ra.perm, block=w.bs, inverse=True)
    mat = dict(coverage=torch.from_numpy(w.coverage).to(dev), k_cov=80, k_unc=150, mass=0.9, ref_blocks=(0, 3))
    o_r, r = ra.step(q_r, k_r, v_r, c - 1, overlap=torch.from_numpy(w.overlap).to(dev), materialize=mat)
    torch.cuda.synchronize()
    # the step writes O in raster order: Gilbert row g is token perm[g]
    perm = ra.perm.cpu().numpy()
    L = len(perm)
    got = csr_lists(r["row_ptr"], r["col_idx"], w.heads, w.nqb)
    win = om.block_window(gilbert_order(*workloads.CHUNK_GRID)[0], workloads.CHUNK_GRID, w.bs, c - 1)
    vmask = valid_rows(w.q_len, w.bs)
    for hi in range(w.heads):
        q, k, v = f64(w.q[hi]), f64(w.k[hi]), f64(w.v[hi])
        ref = om.materialize_head(q, k, w.q_len, w.k_len, w.bs, scale=w.scale, coverage=w.coverage, k_cov=80,
                                  k_unc=150, mass=0.9, prev_blocks=((c - 2) * w.nqb, (c - 1) * w.nqb), windows=win,
                                  ref_blocks=(0, 3), overlap=w.overlap, lam=w.lam, tau=w.tau, g_ref=w.g_ref)
        assert_lists_equal(got[hi], ref["lists"], "head %d" % hi)
        o_ref, _ = oatt.block_sparse_head(q, k, v, w.q_len, w.k_len, w.bs, ref["lists"], w.scale)
        o_g = np.zeros_like(o_ref)
        o_g[:L] = f64(o_r[:, hi, :])[perm]
        mx, mean = err_summary(o_g, o_ref, vmask)
        assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, (hi, mx, mean)


def test_materialize_coverage_at_the_threshold():
    """Query blocks of 80 valid tokens with 72 and 71 of them covered, and
    float32 0.9 and the float32 just below it: the first two are well
    covered (reservation + top-K fill), the others take the mass prefix, on
    the GPU as in the oracle (both decide in float32)."""
    dev = need_gpu()
    import block_sparse_attention_gilbert_amd as bsa
    rng = np.random.default_rng(21)
    heads, nqb, nkb, block, d = 2, 4, 24, 128, 128
    q_len = np.array([80, 80, 80, 80], dtype=np.int32)
    k_len = np.full(nkb, block, dtype=np.int32)
    q = torch.zeros((heads, nqb * block, d), dtype=torch.bfloat16)
    k = torch.from_numpy(rng.standard_normal((heads, nkb * block, d)).astype(np.float32)).to(torch.bfloat16)
    for i in range(nqb):
        q[:, i * block: i * block + 80] = torch.from_numpy(
            rng.standard_normal((heads, 80, d)).astype(np.float32)).to(torch.bfloat16)
    cov = np.array([72 / 80, 0.9, np.nextafter(np.float32(0.9), np.float32(0)), 71 / 80], dtype=np.float32)
    ov = rng.beta(0.5, 2.0, size=(nqb, nkb)).astype(np.float32)
    r = bsa.route_materialize(q.to(dev), k.to(dev), block=block, nqb=nqb, nkb=nkb, scale=d ** -0.5,
                              q_block_len=torch.from_numpy(q_len).to(dev), kv_block_len=torch.from_numpy(k_len).to(dev),
                              overlap=torch.from_numpy(ov).to(dev), coverage=torch.from_numpy(cov).to(dev),
                              prev_blocks=(16, 20), k_cov=8, k_unc=6, mass=0.5)
    torch.cuda.synchronize()
    got = csr_lists(r["row_ptr"], r["col_idx"], heads, nqb)
    for h in range(heads):
        ref = om.materialize_head(f64(q[h]), f64(k[h]), q_len, k_len, block, scale=d ** -0.5, coverage=cov,
                                  k_cov=8, k_unc=6, mass=0.5, prev_blocks=(16, 20), overlap=ov)
        assert ref["covered"].tolist() == [True, True, False, False]
        assert_lists_equal(got[h], ref["lists"], "head %d" % h)
        for i in (0, 1):
            assert {16, 17, 18, 19} <= set(got[h][i].tolist())
