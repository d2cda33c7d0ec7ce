"""GPU parity of the router: CSR lists bit-exact against the oracle on the
configurations (C1-C5 at sizes the oracle finishes in seconds), fallback
counts, selection keys, the pooled-key cache, and edge cases."""

import numpy as np
import pytest
import torch

import workloads
from oracle import layout as olay
from oracle import route as oroute
from oracle.gilbert import gilbert_order

from helpers import assert_lists_equal, csr_lists, f64, need_gpu

pytestmark = pytest.mark.gpu


def _gpu_route(w, dev, **kw):
    import block_sparse_attention_gilbert_amd as bsa
    q, k = w.q.to(dev), w.k.to(dev)
    ql = torch.from_numpy(w.q_len.astype(np.int32)).to(dev)
    kl = torch.from_numpy(w.k_len.astype(np.int32)).to(dev)
    ov = None if w.overlap is None else torch.from_numpy(w.overlap).to(dev)
    r = bsa.route_topk(q, k, block=w.bs, nqb=w.nqb, nkb=w.nkb, scale=w.scale, q_block_len=ql, kv_block_len=kl,
                       overlap=ov, lam=w.lam, g_ref=w.g_ref, tau=w.tau, k_fixed=int(w.k_per_row[0]),
                       n_dense_tail_blocks=w.n_dense_tail, **kw)
    torch.cuda.synchronize()
    return r


def _oracle_head(w, h, **kw):
    q, k = f64(w.q[h]), f64(w.k[h])
    return oroute.route_head(q, k, w.q_len, w.k_len, w.bs, scale=w.scale,
                             k_per_row=w.k_per_row[h * w.nqb:(h + 1) * w.nqb], overlap=w.overlap,
                             lam=w.lam, tau=w.tau, g_ref=w.g_ref, n_dense_tail=w.n_dense_tail, **kw)


@pytest.mark.parametrize("name", ["C1", "C2", "C3"])
def test_routes_bit_exact(name):
    dev = need_gpu()
    w = workloads.get(name)
    r = _gpu_route(w, dev, want_keys=True)
    got = csr_lists(r["row_ptr"], r["col_idx"], w.heads, w.nqb)
    keys = r["sel_keys"].cpu().numpy()
    for h in range(w.heads):
        ref = _oracle_head(w, h)
        assert_lists_equal(got[h], ref["lists"], "%s head %d" % (name, h))
        # selection keys agree with the oracle's kappa to rounding
        kap = ref["kappa"]
        assert np.max(np.abs(keys[h] - kap)) <= 1e-12 * max(1.0, np.max(np.abs(kap)))
    fb = r["fallback_counts"].cpu().numpy()
    if w.overlap is None:
        assert fb.tolist() == [0, 0]
    else:
        ref = _oracle_head(w, 0)
        assert fb[0] == int(ref["zero_rows"].sum()) == 11
        assert fb[1] == int(ref["unvetted_rows"].sum())


@pytest.mark.parametrize("c", [1, 2, 5])
def test_routes_growing_context(c):
    dev = need_gpu()
    w = workloads.c4(c=c, heads=[0, 7, 21, 39])
    r = _gpu_route(w, dev)
    got = csr_lists(r["row_ptr"], r["col_idx"], w.heads, w.nqb)
    for h in range(w.heads):
        ref = _oracle_head(w, h)
        assert_lists_equal(got[h], ref["lists"], "C4 c=%d head %d" % (c, h))
        if c == 1:  # K >= candidates: every block, i.e. dense
            assert all(len(l) == 37 for l in got[h])


def _c5_blocked(w, n_chunks):
    """Gilbert-permuted C5 tensors (oracle's own permutation), per head."""
    T, H, W = w.grid
    L = T * H * W
    perm, _ = gilbert_order(T, H, W)
    q = olay.permute_forward(f64(w.q_raster), perm, w.bs)
    k = np.concatenate([olay.permute_forward(f64(w.k_raster[c]), perm, w.bs) for c in range(n_chunks)], axis=1)
    v = np.concatenate([olay.permute_forward(f64(w.v_raster[c]), perm, w.bs) for c in range(n_chunks)], axis=1)
    return q, k, v, olay.chunk_block_lengths(L, w.bs), olay.chunk_block_lengths(L, w.bs, n_chunks)


def test_routes_ragged_dense_tail():
    dev = need_gpu()
    import block_sparse_attention_gilbert_amd as bsa
    from block_sparse_attention_gilbert_amd.pipeline import RoutedAttention
    n_chunks = 4
    w = workloads.c5(heads=[0, 1, 2], n_chunks=n_chunks)
    ra = RoutedAttention(w.grid, w.heads, w.d, w.bs, n_chunks, device=dev, k_cap=143, n_dense_tail_chunks=1)
    for c in range(n_chunks - 1):
        ra.append(w.k_raster[c].to(dev), w.v_raster[c].to(dev), c)
    kpr = torch.from_numpy(w.k_per_row).to(dev)
    _, r = ra.step(w.q_raster.to(dev), w.k_raster[-1].to(dev), w.v_raster[-1].to(dev), n_chunks - 1,
                   k_per_row=kpr)
    torch.cuda.synchronize()
    q, k, _v, ql, kl = _c5_blocked(w, n_chunks)
    nbc = len(ql)
    got = csr_lists(r["row_ptr"], r["col_idx"], w.heads, nbc)
    for h in range(w.heads):
        ref = oroute.route_head(q[h], k[h], ql, kl, w.bs, scale=w.scale,
                                k_per_row=w.k_per_row[h * nbc:(h + 1) * nbc], n_dense_tail=nbc)
        assert_lists_equal(got[h], ref["lists"], "C5 head %d" % h)
    assert bsa is not None


def test_pooled_key_cache_incremental():
    dev = need_gpu()
    import block_sparse_attention_gilbert_amd as bsa
    w = workloads.c4(c=3, heads=[0, 1])
    ql = torch.from_numpy(w.q_len).to(dev)
    kl = torch.from_numpy(w.k_len).to(dev)
    q, k = w.q.to(dev), w.k.to(dev)
    cache = torch.zeros((w.heads, w.nkb, w.d), dtype=torch.float64, device=dev)
    kw = dict(block=128, nqb=37, nkb=w.nkb, scale=w.scale, q_block_len=ql, kv_block_len=kl, k_fixed=50)
    r_full = bsa.route_topk(q, k, kpool=cache, kpool_valid_blocks=0, **kw)   # pools every block
    lists_full = csr_lists(r_full["row_ptr"], r_full["col_idx"], w.heads, 37)
    cache[:, 74:] = float("nan")            # forget the newest chunk's means ...
    r_inc = bsa.route_topk(q, k, kpool=cache, kpool_valid_blocks=74, **kw)  # ... and pool only it
    lists_inc = csr_lists(r_inc["row_ptr"], r_inc["col_idx"], w.heads, 37)
    for h in range(w.heads):
        assert_lists_equal(lists_inc[h], lists_full[h], "incremental head %d" % h)
        ref = _oracle_head(w, h)
        assert_lists_equal(lists_inc[h], ref["lists"], "cache head %d" % h)
        assert np.array_equal(cache[h].cpu().numpy(), ref["kbar"])   # exact block means


def test_routes_from_pooled_queries():
    """Routing from the pooled queries of the fused permutation (q not
    read) gives the lists of routing from the permuted queries."""
    dev = need_gpu()
    import block_sparse_attention_gilbert_amd as bsa
    w = workloads.c4(c=3, heads=[0, 1])
    perm, _ = bsa.gilbert_index(3, 30, 52, device=dev)
    q_raster = bsa.gilbert_perm(w.q.to(dev), perm, block=128, inverse=True)
    q_blk, qbar = bsa.gilbert_perm_pool(q_raster, perm, block=128)
    ql = torch.from_numpy(w.q_len).to(dev)
    kl = torch.from_numpy(w.k_len).to(dev)
    kw = dict(block=128, nqb=37, nkb=w.nkb, scale=w.scale, q_block_len=ql, kv_block_len=kl, k_fixed=50)
    r_q = bsa.route_topk(q_blk, w.k.to(dev), **kw)
    lists_q = csr_lists(r_q["row_ptr"], r_q["col_idx"], w.heads, 37)
    garbage = torch.full_like(q_blk, float("nan"))          # must not be read
    r_p = bsa.route_topk(garbage, w.k.to(dev), qpool=qbar, **kw)
    lists_p = csr_lists(r_p["row_ptr"], r_p["col_idx"], w.heads, 37)
    for h in range(w.heads):
        assert_lists_equal(lists_p[h], lists_q[h], "pooled queries head %d" % h)
        assert_lists_equal(lists_p[h], _oracle_head(w, h)["lists"], "oracle head %d" % h)


def test_pooled_key_cache_grows_with_history():
    """One cache with a fixed head stride serves a history that grows by a
    chunk per call: each call pools only the appended chunk."""
    dev = need_gpu()
    import block_sparse_attention_gilbert_amd as bsa
    w = workloads.c4(c=3, heads=[0, 1, 2])
    ql = torch.from_numpy(w.q_len).to(dev)
    kl = torch.from_numpy(w.k_len).to(dev)
    q, k = w.q.to(dev), w.k.to(dev)
    cache = torch.full((w.heads, 5 * 37, w.d), float("nan"), dtype=torch.float64, device=dev)  # room for 5 chunks
    valid = 0
    for c in (1, 2, 3):
        nkb = 37 * c
        r = bsa.route_topk(q, k, block=128, nqb=37, nkb=nkb, scale=w.scale, q_block_len=ql, kv_block_len=kl[:nkb],
                           k_fixed=50, kpool=cache, kpool_valid_blocks=valid)
        valid = nkb
        lists = csr_lists(r["row_ptr"], r["col_idx"], w.heads, 37)
        for h in range(w.heads):
            ref = oroute.route_head(f64(w.q[h]), f64(w.k[h])[: nkb * 128], w.q_len, w.k_len[:nkb], w.bs,
                                    scale=w.scale, k_per_row=w.k_per_row[:37])
            assert_lists_equal(lists[h], ref["lists"], "growing cache c=%d head %d" % (c, h))
            assert np.array_equal(cache[h, :nkb].cpu().numpy(), ref["kbar"])
    assert torch.isnan(cache[:, 111:]).all()   # nothing written past the history


def test_route_edge_cases():
    dev = need_gpu()
    import block_sparse_attention_gilbert_amd as bsa
    rng = np.random.default_rng(5)
    heads, d, bs, nqb, nkb = 2, 64, 64, 3, 12
    q = torch.from_numpy(rng.standard_normal((heads, nqb * bs, d)).astype(np.float32)).to(torch.bfloat16)
    k = torch.from_numpy(rng.standard_normal((heads, nkb * bs, d)).astype(np.float32)).to(torch.bfloat16)
    k[:, 9 * bs:10 * bs] = k[:, 4 * bs:5 * bs]            # duplicate block -> exact tie
    q_len = np.array([bs, 0, 17], dtype=np.int32)         # an empty query block, a ragged one
    k_len = np.array([bs] * 6 + [0] + [bs] * 3 + [5, bs], dtype=np.int32)  # an empty KV block
    k[:, 6 * bs:7 * bs] = 1.0e4                           # junk in the empty block's rows
    for K, tail in [(0, 0), (3, 0), (4, 2), (50, 0), (5, 2)]:
        r = bsa.route_topk(q.to(dev), k.to(dev), block=bs, nqb=nqb, nkb=nkb, scale=0.125,
                           q_block_len=torch.from_numpy(q_len).to(dev), kv_block_len=torch.from_numpy(k_len).to(dev),
                           k_fixed=K, n_dense_tail_blocks=tail)
        got = csr_lists(r["row_ptr"], r["col_idx"], heads, nqb)
        for h in range(heads):
            ref = oroute.route_head(f64(q[h]), f64(k[h]), q_len, k_len, bs, scale=0.125,
                                    k_per_row=[K] * nqb, n_dense_tail=tail)
            assert_lists_equal(got[h], ref["lists"], "K=%d tail=%d head %d" % (K, tail, h))
            assert len(got[h][1]) == 0
            assert all(6 not in l.tolist() for l in got[h])


def test_route_maximum_candidates():
    """4096 candidates (the most one wave selects over) with per-row budgets
    up to 143 and a dense tail, and 4097 (a second segment of one
    candidate), against the oracle."""
    dev = need_gpu()
    import block_sparse_attention_gilbert_amd as bsa
    rng = np.random.default_rng(4096)
    heads, d, bs, nqb, n_cand, tail = 2, 64, 64, 3, 4096, 3
    nkb = n_cand + tail
    q = torch.from_numpy(rng.standard_normal((heads, nqb * bs, d)).astype(np.float32)).to(torch.bfloat16)
    k = torch.from_numpy(rng.standard_normal((heads, nkb * bs, d)).astype(np.float32)).to(torch.bfloat16)
    kpr = rng.integers(0, 144, size=heads * nqb).astype(np.int32)
    kpr[0] = 143
    r = bsa.route_topk(q.to(dev), k.to(dev), block=bs, nqb=nqb, nkb=nkb, scale=0.125,
                       k_per_row=torch.from_numpy(kpr).to(dev), k_max=143, n_dense_tail_blocks=tail)
    got = csr_lists(r["row_ptr"], r["col_idx"], heads, nqb)
    for h in range(heads):
        ref = oroute.route_head(f64(q[h]), f64(k[h]), [bs] * nqb, [bs] * nkb, bs, scale=0.125,
                                k_per_row=kpr[h * nqb:(h + 1) * nqb], n_dense_tail=tail)
        assert_lists_equal(got[h], ref["lists"], "max candidates head %d" % h)
    # one candidate more: two segments, the second holding a single block
    # that is the best of every row
    k2 = torch.cat([k, torch.zeros((heads, bs, d), dtype=torch.bfloat16)], dim=1)
    k2[:, n_cand * bs:] = q[:, :bs].float().mean(dim=1, keepdim=True).mul(50).to(torch.bfloat16)
    r2 = bsa.route_topk(q.to(dev), k2.to(dev), block=bs, nqb=nqb, nkb=n_cand + 1, scale=0.125, k_fixed=5)
    got2 = csr_lists(r2["row_ptr"], r2["col_idx"], heads, nqb)
    for h in range(heads):
        ref = oroute.route_head(f64(q[h]), f64(k2[h]), [bs] * nqb, [bs] * (n_cand + 1), bs, scale=0.125,
                                k_per_row=np.full(nqb, 5))
        assert_lists_equal(got2[h], ref["lists"], "4097 candidates head %d" % h)
    assert n_cand in got2[0][0].tolist()


def test_route_selection_paths():
    """Every path of the threshold select against the oracle: budgets of up
    to 64, 128 and 256 (the three fast-path widths), above 256 (the radix
    select), and a query block whose keys all tie (all-zero queries: every
    score is 0, so the fast path's candidate gather overflows and the radix
    select takes the lowest indices)."""
    dev = need_gpu()
    import block_sparse_attention_gilbert_amd as bsa
    rng = np.random.default_rng(77)
    heads, d, bs, nqb, nkb = 2, 64, 64, 4, 1000
    q = torch.from_numpy(rng.standard_normal((heads, nqb * bs, d)).astype(np.float32)).to(torch.bfloat16)
    k = torch.from_numpy(rng.standard_normal((heads, nkb * bs, d)).astype(np.float32)).to(torch.bfloat16)
    q[:, 2 * bs:3 * bs] = 0                                # query block 2: every score ties
    for K in (50, 100, 200, 300):
        r = bsa.route_topk(q.to(dev), k.to(dev), block=bs, nqb=nqb, nkb=nkb, scale=0.125, k_fixed=K)
        got = csr_lists(r["row_ptr"], r["col_idx"], heads, nqb)
        for h in range(heads):
            ref = oroute.route_head(f64(q[h]), f64(k[h]), [bs] * nqb, [bs] * nkb, bs, scale=0.125,
                                    k_per_row=[K] * nqb)
            assert_lists_equal(got[h], ref["lists"], "K=%d head %d" % (K, h))
            assert np.array_equal(got[h][2], np.arange(K))  # ties: the lowest indices


def _long_history(seed, heads, d, bs, n_chunks, nbc_tokens=4680):
    """Q of one chunk and K of a long history (per-chunk padded blocks), N(0,1)
    plus N(0, 0.5^2) per-block offsets, bf16 (input recipe of the growing
    context, without its V)."""
    rng = np.random.default_rng(seed)
    q_len = workloads.block_lengths(nbc_tokens, bs)
    k_len = np.tile(q_len, n_chunks).astype(np.int32)

    def blocked(lens):
        x = rng.standard_normal((heads, len(lens), bs, d), dtype=np.float32)
        x += rng.standard_normal((heads, len(lens), 1, d), dtype=np.float32) * np.float32(0.5)
        x[:, np.arange(bs)[None, :] >= lens[:, None]] = 0.0
        return torch.from_numpy(x.reshape(heads, len(lens) * bs, d)).to(torch.bfloat16)

    return blocked(q_len), blocked(k_len), q_len, k_len


@pytest.mark.parametrize("d,bs,n_chunks,heads", [(128, 128, 170, 1), (64, 64, 90, 2)])
def test_routes_beyond_one_wave_of_candidates(d, bs, n_chunks, heads):
    """More than 4096 candidates (6290 and 6660): selected in segments of 4096
    whose top-K are merged; lists bit-exact against the oracle for a fixed
    budget and for per-row budgets up to 256."""
    dev = need_gpu()
    import block_sparse_attention_gilbert_amd as bsa
    q, k, q_len, k_len = _long_history(31 + d, heads, d, bs, n_chunks)
    nqb, nkb = len(q_len), len(k_len)
    assert nkb > 6000
    scale = d ** -0.5
    kpr = np.random.default_rng(5).integers(1, 257, size=heads * nqb).astype(np.int32)
    kw = dict(block=bs, nqb=nqb, nkb=nkb, scale=scale, q_block_len=torch.from_numpy(q_len).to(dev),
              kv_block_len=torch.from_numpy(k_len).to(dev))
    print("routing %d candidates" % nkb, flush=True)
    r_fix = bsa.route_topk(q.to(dev), k.to(dev), k_fixed=50, **kw)
    r_var = bsa.route_topk(q.to(dev), k.to(dev), k_per_row=torch.from_numpy(kpr).to(dev), k_max=256, **kw)
    torch.cuda.synchronize()
    g_fix = csr_lists(r_fix["row_ptr"], r_fix["col_idx"], heads, nqb)
    g_var = csr_lists(r_var["row_ptr"], r_var["col_idx"], heads, nqb)
    for h in range(heads):
        qh, kh = f64(q[h]), f64(k[h])
        ref = oroute.route_head(qh, kh, q_len, k_len, bs, scale=scale, k_per_row=np.full(nqb, 50))
        assert_lists_equal(g_fix[h], ref["lists"], "fixed budget head %d" % h)
        ref = oroute.route_head(qh, kh, q_len, k_len, bs, scale=scale, k_per_row=kpr[h * nqb:(h + 1) * nqb])
        assert_lists_equal(g_var[h], ref["lists"], "per-row budgets head %d" % h)


def test_routes_beyond_one_wave_ties_across_segments():
    """Exact ties between blocks of different segments (the same K rows copied
    into a block of a later segment): the lower index wins, as in the
    oracle, also when the budget cuts between the copies."""
    dev = need_gpu()
    import block_sparse_attention_gilbert_amd as bsa
    q, k, q_len, k_len = _long_history(47, 1, 64, 64, 70)
    nqb, nkb = len(q_len), len(k_len)
    assert 4240 < nkb     # two segments: 4096 + the rest
    k = k.clone()
    # copy the 40 blocks a row likes best into blocks past the first segment
    qh, kh = f64(q[0]), f64(k[0])
    best = np.argsort(-oroute.route_head(qh, kh, q_len, k_len, 64, scale=0.125,
                                         k_per_row=np.full(nqb, 40))["kappa"][3])[:40]
    dst = np.arange(4200, 4200 + 40)
    for a, b in zip(best, dst):
        k[0, b * 64:(b + 1) * 64] = k[0, a * 64:(a + 1) * 64]
        k_len[b] = k_len[a]
    for kf in (20, 40, 60):
        r = bsa.route_topk(q.to(dev), k.to(dev), block=64, nqb=nqb, nkb=nkb, scale=0.125, k_fixed=kf,
                           q_block_len=torch.from_numpy(q_len).to(dev), kv_block_len=torch.from_numpy(k_len).to(dev))
        torch.cuda.synchronize()
        got = csr_lists(r["row_ptr"], r["col_idx"], 1, nqb)
        ref = oroute.route_head(qh, f64(k[0]), q_len, k_len, 64, scale=0.125, k_per_row=np.full(nqb, kf))
        assert_lists_equal(got[0], ref["lists"], "ties, budget %d" % kf)


@pytest.mark.parametrize("dtype,span", [(torch.float32, 60), (torch.bfloat16, 36)])
def test_router_pools_exact_means_mixed_magnitudes(dtype, span):
    """The router's own pooling (every K block into an empty pooled-key
    cache) gives the oracle's exact block means bit for bit on rows whose
    magnitudes span 2^60 (float32, summed as exact pairs) or 2^36 (bf16, a
    plain float64 sum, exact below 2^39)."""
    dev = need_gpu()
    import block_sparse_attention_gilbert_amd as bsa
    rng = np.random.default_rng(41)
    heads, nqb, nkb, block, d = 2, 3, 9, 64, 64
    def mixed(rows):
        x = 2.0 ** rng.uniform(-span / 2, span / 2, (heads, rows, d)) * rng.choice([-1.0, 1.0], (heads, rows, d))
        x[:, 1::2, ::3] = -x[:, 0::2, ::3]
        return torch.from_numpy(x.astype(np.float32)).to(dtype)
    q, k = mixed(nqb * block), mixed(nkb * block)
    kl = np.full(nkb, block, dtype=np.int32)
    kl[4], kl[8] = 37, 1
    ql = np.full(nqb, block, dtype=np.int32)
    cache = torch.zeros((heads, nkb, d), dtype=torch.float64, device=dev)
    bsa.route_topk(q.to(dev), k.to(dev), block=block, nqb=nqb, nkb=nkb, scale=0.125,
                   q_block_len=torch.from_numpy(ql).to(dev), kv_block_len=torch.from_numpy(kl).to(dev), k_fixed=3,
                   kpool=cache, kpool_valid_blocks=0)
    torch.cuda.synchronize()
    for h in range(heads):
        want = oroute.pool_blocks(f64(k[h]), kl, block)
        assert np.array_equal(cache[h].cpu().numpy(), want), h
