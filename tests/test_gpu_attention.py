"""GPU parity of block-sparse and dense attention against the oracle, plus
the properties the kernel must keep: select-all equals dense bitwise,
determinism, every valid output written, padding inert, and the edge cases
(empty lists, ignored indices, empty KV blocks, ragged query blocks)."""

import numpy as np
import pytest
import torch

import workloads
from oracle import attention as oatt
from oracle import route as oroute

from helpers import (BF16_MAX_ABS, BF16_MEAN_ABS, F32_MAX_ABS, LSE_BF16, LSE_F32, csr_lists, err_summary, f64,
                     need_gpu, valid_rows)

pytestmark = pytest.mark.gpu


def _tensors(w, dev):
    return (w.q.to(dev), w.k.to(dev), w.v.to(dev), torch.from_numpy(w.q_len.astype(np.int32)).to(dev),
            torch.from_numpy(w.k_len.astype(np.int32)).to(dev))


def _route(w, dev, q, k, ql, kl):
    import block_sparse_attention_gilbert_amd as bsa
    ov = None if w.overlap is None else torch.from_numpy(w.overlap).to(dev)
    return bsa.route_topk(q, k, block=w.bs, nqb=w.nqb, nkb=w.nkb, scale=w.scale, q_block_len=ql, kv_block_len=kl,
                          overlap=ov, lam=w.lam, g_ref=w.g_ref, tau=w.tau, k_fixed=int(w.k_per_row[0]))


def _check_against_oracle(w, o, lse, lists_all, heads=None, dense=False):
    bf = w.dtype == torch.bfloat16
    vmask = valid_rows(w.q_len, w.bs)
    worst = (0.0, 0.0)
    for h in (range(w.heads) if heads is None else heads):
        q, k, v = f64(w.q[h]), f64(w.k[h]), f64(w.v[h])
        if dense:
            o_ref, l_ref = oatt.dense_head(q, k, v, w.q_len, w.k_len, w.bs, w.scale)
        else:
            o_ref, l_ref = oatt.block_sparse_head(q, k, v, w.q_len, w.k_len, w.bs, lists_all[h], w.scale)
        og = f64(o[h])
        mx, mean = err_summary(og, o_ref, vmask)
        if bf:
            assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, (h, mx, mean)
        else:
            assert mx <= F32_MAX_ABS, (h, mx)
        assert np.all(og[~vmask] == 0.0)
        lg = lse[h].cpu().numpy().astype(np.float64)
        assert np.max(np.abs(lg[vmask] - l_ref[vmask])) <= (LSE_BF16 if bf else LSE_F32)
        assert np.all(np.isneginf(lg[~vmask]))
        worst = (max(worst[0], mx), max(worst[1], mean))
    return worst


@pytest.mark.parametrize("name", ["C1", "C2", "C3"])
def test_block_sparse_parity(name):
    dev = need_gpu()
    import block_sparse_attention_gilbert_amd as bsa
    w = workloads.get(name)
    q, k, v, ql, kl = _tensors(w, dev)
    r = _route(w, dev, q, k, ql, kl)
    o = torch.full_like(q, float("nan"))        # every element must be written
    o, lse = bsa.block_sparse_attn(q, k, v, r["row_ptr"], r["col_idx"], block=w.bs, scale=w.scale,
                                   q_block_len=ql, kv_block_len=kl, out=o, lse=True)
    torch.cuda.synchronize()
    lists = csr_lists(r["row_ptr"], r["col_idx"], w.heads, w.nqb)
    for h in range(w.heads):  # the lists themselves are pinned in the router tests
        ref = oroute.route_head(f64(w.q[h]), f64(w.k[h]), w.q_len, w.k_len, w.bs, scale=w.scale,
                                k_per_row=w.k_per_row[h * w.nqb:(h + 1) * w.nqb], overlap=w.overlap,
                                lam=w.lam, tau=w.tau, g_ref=w.g_ref)
        assert all(np.array_equal(a, b) for a, b in zip(lists[h], ref["lists"]))
    print(name, "max/mean abs err", _check_against_oracle(w, o, lse, lists))


def test_growing_context_parity():
    dev = need_gpu()
    import block_sparse_attention_gilbert_amd as bsa
    w = workloads.c4(c=3, heads=[0, 19, 39])
    q, k, v, ql, kl = _tensors(w, dev)
    r = _route(w, dev, q, k, ql, kl)
    o, lse = bsa.block_sparse_attn(q, k, v, r["row_ptr"], r["col_idx"], block=128, scale=w.scale, q_block_len=ql,
                                   kv_block_len=kl, lse=True)
    torch.cuda.synchronize()
    lists = csr_lists(r["row_ptr"], r["col_idx"], w.heads, w.nqb)
    print("C4 c=3 max/mean abs err", _check_against_oracle(w, o, lse, lists))


def test_dense_parity_and_select_all_equals_dense():
    dev = need_gpu()
    import block_sparse_attention_gilbert_amd as bsa
    w = workloads.c2(heads=[0, 6, 11])
    q, k, v, ql, kl = _tensors(w, dev)
    o_d, l_d = bsa.dense_attn(q, k, v, block=128, scale=w.scale, q_block_len=ql, kv_block_len=kl, lse=True)
    all_rows = torch.arange(w.nkb, dtype=torch.int32, device=dev).repeat(w.heads * w.nqb)
    row_ptr = torch.arange(0, w.heads * w.nqb + 1, dtype=torch.int32, device=dev) * w.nkb
    o_s, l_s = bsa.block_sparse_attn(q, k, v, row_ptr, all_rows, block=128, scale=w.scale, q_block_len=ql,
                                     kv_block_len=kl, lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o_s, o_d) and torch.equal(l_s, l_d)
    print("C2 dense max/mean abs err", _check_against_oracle(w, o_d, l_d, None, dense=True))


def test_fp32_dense_parity():
    dev = need_gpu()
    import block_sparse_attention_gilbert_amd as bsa
    w = workloads.c1()
    q, k, v, ql, kl = _tensors(w, dev)
    o, lse = bsa.dense_attn(q, k, v, block=64, scale=w.scale, q_block_len=ql, kv_block_len=kl, lse=True)
    torch.cuda.synchronize()
    _check_against_oracle(w, o, lse, None, dense=True)


def test_deterministic_and_padding_inert():
    dev = need_gpu()
    import block_sparse_attention_gilbert_amd as bsa
    w = workloads.c4(c=2, heads=[3, 4])
    q, k, v, ql, kl = _tensors(w, dev)
    r = _route(w, dev, q, k, ql, kl)
    args = dict(block=128, scale=w.scale, q_block_len=ql, kv_block_len=kl, lse=True)
    o1, l1 = bsa.block_sparse_attn(q, k, v, r["row_ptr"], r["col_idx"], **args)
    o2, l2 = bsa.block_sparse_attn(q, k, v, r["row_ptr"], r["col_idx"], **args)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # large finite junk in every padded row of Q, K and V changes nothing
    q2, k2, v2 = q.clone(), k.clone(), v.clone()
    q2[:, 36 * 128 + 72:] = 1.0e4
    for c in range(2):
        k2[:, (c * 37 + 36) * 128 + 72:(c * 37 + 37) * 128] = -1.0e4
        v2[:, (c * 37 + 36) * 128 + 72:(c * 37 + 37) * 128] = 1.0e4
    o3, l3 = bsa.block_sparse_attn(q2, k2, v2, r["row_ptr"], r["col_idx"], **args)
    torch.cuda.synchronize()
    assert torch.equal(o1, o3) and torch.equal(l1, l3)
    # padded rows are never fetched: NaN there changes nothing either
    q2[:, 36 * 128 + 72:] = float("nan")
    for c in range(2):
        k2[:, (c * 37 + 36) * 128 + 72:(c * 37 + 37) * 128] = float("nan")
        v2[:, (c * 37 + 36) * 128 + 72:(c * 37 + 37) * 128] = float("nan")
    o4, l4 = bsa.block_sparse_attn(q2, k2, v2, r["row_ptr"], r["col_idx"], **args)
    torch.cuda.synchronize()
    assert torch.equal(o1, o4) and torch.equal(l1, l4)


def _raster_case(name):
    """(workload, row map, token count): the Gilbert curve for the C4 layout
    (ragged last block), a seeded shuffle for C1 (fp32), and a map with
    padding rows (-1, as in the tile layout) over C2's rows."""
    import block_sparse_attention_gilbert_amd as bsa
    g = torch.Generator().manual_seed(31)
    if name == "curve":
        w = workloads.c4(c=2, heads=[3, 4])
        perm, _ = bsa.gilbert_index(3, 30, 52, device="cuda")
        return w, perm, 4680
    if name == "shuffle":
        w = workloads.c1()
        n = int(w.q_len.sum())
        return w, torch.randperm(n, generator=g).to(torch.int32), n
    w = workloads.c2(heads=[0, 5])
    rows = w.nqb * w.bs
    m = torch.randperm(rows, generator=g).to(torch.int32)
    m[torch.randperm(rows, generator=g)[: rows // 10]] = -1        # padding rows: not written
    return w, m, rows


@pytest.mark.parametrize("name", ["curve", "shuffle", "padding"])
def test_raster_output_is_the_blocked_output_permuted(name):
    """The raster-output launch writes row g's bits at token row_map[g]:
    equal, bit for bit, to the blocked launch followed by the inverse
    permutation; every mapped token is written, the others are untouched,
    and the LSE is the blocked launch's."""
    dev = need_gpu()
    import block_sparse_attention_gilbert_amd as bsa
    w, row_map, tokens = _raster_case(name)
    row_map = row_map.to(dev)
    q, k, v, ql, kl = _tensors(w, dev)
    r = _route(w, dev, q, k, ql, kl)
    args = dict(block=w.bs, scale=w.scale, q_block_len=ql, kv_block_len=kl, lse=True)
    o_blk, l_blk = bsa.block_sparse_attn(q, k, v, r["row_ptr"], r["col_idx"], **args)
    out = torch.full((tokens + 3, w.heads, w.d), 7.0, dtype=q.dtype, device=dev)
    o_r, l_r = bsa.block_sparse_attn_raster(q, k, v, r["row_ptr"], r["col_idx"], row_map, out=out, **args)
    torch.cuda.synchronize()
    assert torch.equal(l_r, l_blk)
    m = row_map.cpu().numpy()
    g = np.nonzero(m >= 0)[0]
    got = o_r.cpu()
    ref = o_blk.cpu().transpose(0, 1)                     # [rows][heads][d]
    assert torch.equal(got[torch.from_numpy(m[g]).long()], ref[torch.from_numpy(g).long()])
    written = np.zeros(tokens + 3, dtype=bool)
    written[m[g]] = True
    assert torch.all(got[torch.from_numpy(~written)] == 7.0)
    # the queries read in raster order through the same map: the same bits
    # (rows the map leaves out read as zeros, as the blocked padding rows)
    q_r = torch.full((tokens + 3, w.heads, w.d), 5.0, dtype=q.dtype, device=dev)
    qb = q.transpose(0, 1)                                  # [rows][heads][d] view of the blocked queries
    idx = torch.from_numpy(g).long().to(dev)
    q_r[torch.from_numpy(m[g]).long().to(dev)] = qb[idx]
    pad = torch.ones(q.shape[1], dtype=torch.bool, device=dev)
    pad[idx] = False
    q_zero = q.clone()
    q_zero[:, pad] = 0                                      # unmapped rows read as zeros
    o_z, l_z = bsa.block_sparse_attn_raster(q_zero, k, v, r["row_ptr"], r["col_idx"], row_map,
                                            out=torch.full_like(out, 7.0), **args)
    o_q, l_q = bsa.block_sparse_attn_raster(q_r, k, v, r["row_ptr"], r["col_idx"], row_map, q_raster=True,
                                            nqb=w.nqb, out=torch.full_like(out, 7.0), **args)
    torch.cuda.synchronize()
    assert torch.equal(o_q, o_z) and torch.equal(l_q, l_z)
    print(name, "rows mapped", len(g), "of", len(m))


@pytest.mark.parametrize("block,d", [(64, 64), (64, 128), (128, 64)])
def test_edge_cases_small(block, d):
    """Empty lists, out-of-range and negative indices (ignored), an empty KV
    block, ragged query blocks, strided heads -- bf16 and fp32."""
    dev = need_gpu()
    import block_sparse_attention_gilbert_amd as bsa
    rng = np.random.default_rng(block + d)
    heads, nqb, nkb = 2, 3, 6
    for dtype in (torch.bfloat16, torch.float32):
        q = torch.from_numpy(rng.standard_normal((heads, nqb * block, d)).astype(np.float32)).to(dtype)
        store = torch.from_numpy(rng.standard_normal((heads, 2 * nkb * block, d)).astype(np.float32)).to(dtype)
        v = torch.from_numpy(rng.standard_normal((heads, nkb * block, d)).astype(np.float32)).to(dtype)
        k_view = store.to(dev)[:, : nkb * block]              # head stride 2*nkb*block*d
        q_len = np.array([block, 1, 33], dtype=np.int32)
        k_len = np.array([block, 0, 7, block, block, 1], dtype=np.int32)
        raw = [[0, 2, 5], [], [3, -1, 1, 99, 4],                 # head 0
               [1], [0, 1, 2, 3, 4, 5], [5, 2]]                   # head 1
        row_ptr = np.cumsum([0] + [len(x) for x in raw]).astype(np.int32)
        col = np.concatenate([np.asarray(x, dtype=np.int32) for x in raw if x])
        o, lse = bsa.block_sparse_attn(q.to(dev), k_view, v.to(dev), torch.from_numpy(row_ptr).to(dev),
                                       torch.from_numpy(col).to(dev), block=block, scale=0.1,
                                       q_block_len=torch.from_numpy(q_len).to(dev),
                                       kv_block_len=torch.from_numpy(k_len).to(dev), lse=True, nkb=nkb)
        torch.cuda.synchronize()
        vmask = valid_rows(q_len, block)
        kk = f64(store[:, : nkb * block])
        for h in range(heads):
            lists = [[j for j in raw[h * nqb + i] if 0 <= j < nkb] for i in range(nqb)]
            o_ref, l_ref = oatt.block_sparse_head(f64(q[h]), kk[h], f64(v[h]), q_len, k_len, block, lists, 0.1)
            og = f64(o[h])
            mx, _ = err_summary(og, o_ref, vmask)
            assert mx <= (BF16_MAX_ABS if dtype == torch.bfloat16 else F32_MAX_ABS), (dtype, h, mx)
            assert np.all(og[~vmask] == 0.0)
            lg = lse[h].cpu().numpy().astype(np.float64)
            both_inf = np.isneginf(lg) & np.isneginf(l_ref)
            assert np.all(both_inf | (np.abs(lg - l_ref) <= (LSE_BF16 if dtype == torch.bfloat16 else 1e-4)))
        # head 0 block 1 has an empty list: zeros and -inf
        assert torch.all(o[0, block: 2 * block] == 0) and torch.all(torch.isneginf(lse[0, block:2 * block]))


@pytest.mark.parametrize("block", [64, 128])
def test_ragged_lengths_every_item_once(block):
    """Lists of widely different lengths (0 to nkb) over more than 128 query
    blocks per head and 3 heads (450 items: the per-XCD runs of 56 items cut
    heads apart, two items fall outside the runs, windows of 128 split a
    head): the workgroups take the items longest list first, and every
    (head, query block) must still be computed exactly once."""
    dev = need_gpu()
    import block_sparse_attention_gilbert_amd as bsa
    rng = np.random.default_rng(7 + block)
    heads, nqb, nkb, d = 3, 150, 10, 128
    q = torch.from_numpy(rng.standard_normal((heads, nqb * block, d)).astype(np.float32)).to(torch.bfloat16)
    k = torch.from_numpy(rng.standard_normal((heads, nkb * block, d)).astype(np.float32)).to(torch.bfloat16)
    v = torch.from_numpy(rng.standard_normal((heads, nkb * block, d)).astype(np.float32)).to(torch.bfloat16)
    q_len = np.full(nqb, block, dtype=np.int32)
    q_len[-1] = 5
    k_len = np.full(nkb, block, dtype=np.int32)
    k_len[3] = 17
    raw = [sorted(rng.choice(nkb, size=int(rng.integers(0, nkb + 1)), replace=False).tolist())
           for _ in range(heads * nqb)]
    row_ptr = np.cumsum([0] + [len(x) for x in raw]).astype(np.int32)
    col = np.concatenate([np.asarray(x, dtype=np.int32) for x in raw if x])
    o = torch.full((heads, nqb * block, d), float("nan"), dtype=torch.bfloat16, device=dev)
    o, lse = bsa.block_sparse_attn(q.to(dev), k.to(dev), v.to(dev), torch.from_numpy(row_ptr).to(dev),
                                   torch.from_numpy(col).to(dev), block=block, scale=0.09,
                                   q_block_len=torch.from_numpy(q_len).to(dev),
                                   kv_block_len=torch.from_numpy(k_len).to(dev), out=o, lse=True)
    torch.cuda.synchronize()
    vmask = valid_rows(q_len, block)
    for h in range(heads):
        lists = raw[h * nqb:(h + 1) * nqb]
        o_ref, l_ref = oatt.block_sparse_head(f64(q[h]), f64(k[h]), f64(v[h]), q_len, k_len, block, lists, 0.09)
        og = f64(o[h])
        mx, mean = err_summary(og, o_ref, vmask)
        assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, (h, mx, mean)
        assert np.all(og[~vmask] == 0.0)
        lg = lse[h].cpu().numpy().astype(np.float64)
        both_inf = np.isneginf(lg) & np.isneginf(l_ref)
        assert np.all(both_inf | (np.abs(lg - l_ref) <= LSE_BF16)), h


def test_wrapper_rejects_short_or_mistyped_arrays():
    """The binding checks what the C ABI cannot see (device array lengths,
    operand dtypes, nkb against the KV rows) and raises ValueError before
    anything is launched."""
    dev = need_gpu()
    import block_sparse_attention_gilbert_amd as bsa
    heads, nqb, nkb, bs, d = 2, 3, 5, 64, 64
    q = torch.zeros((heads, nqb * bs, d), dtype=torch.bfloat16, device=dev)
    k = torch.zeros((heads, nkb * bs, d), dtype=torch.bfloat16, device=dev)
    v = torch.zeros_like(k)
    rp = torch.zeros(heads * nqb + 1, dtype=torch.int32, device=dev)
    ci = torch.zeros(1, dtype=torch.int32, device=dev)
    i32 = lambda n: torch.full((n,), bs, dtype=torch.int32, device=dev)
    cases = [
        dict(lse=torch.empty(heads * nqb * bs - 1, dtype=torch.float32, device=dev)),
        dict(q_block_len=i32(nqb - 1)),
        dict(kv_block_len=i32(nkb - 1)),
        dict(nkb=nkb + 1),
        dict(nkb=0),
        dict(out=torch.empty((heads, nqb * bs, d), dtype=torch.float32, device=dev)),
        dict(out=torch.empty((heads, nqb * bs - bs, d), dtype=torch.bfloat16, device=dev)),
    ]
    for kw in cases:
        with pytest.raises(ValueError):
            bsa.block_sparse_attn(q, k, v, rp, ci, block=bs, **kw)
    with pytest.raises(ValueError):
        bsa.block_sparse_attn(q, k, v, rp[:-1], ci, block=bs)
    with pytest.raises(ValueError):
        bsa.block_sparse_attn(q, k.float(), v, rp, ci, block=bs)
    with pytest.raises(ValueError):
        bsa.block_sparse_attn(q, k, v.float(), rp, ci, block=bs)
    with pytest.raises(ValueError):
        bsa.dense_attn(q, k, v, block=bs, kv_block_len=i32(nkb - 1))
    with pytest.raises(ValueError):
        bsa.dense_attn(q, k, v, block=bs, lse=torch.empty(7, dtype=torch.float32, device=dev))
    row_map = torch.arange(nqb * bs, dtype=torch.int32, device=dev)
    with pytest.raises(ValueError):
        bsa.block_sparse_attn_raster(q, k, v, rp, ci, row_map, block=bs, q_block_len=i32(nqb - 1))
    q_r = torch.zeros((nqb * bs, heads, d), dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError):
        bsa.block_sparse_attn_raster(q_r, k.float(), v, rp, ci, row_map, block=bs, q_raster=True, nqb=nqb)
    with pytest.raises(ValueError):
        bsa.block_sparse_attn_raster(q_r, k, v, rp, ci, row_map, block=bs, q_raster=True, nqb=nqb,
                                     lse=torch.empty(5, dtype=torch.float32, device=dev))
    with pytest.raises(ValueError):
        bsa.block_sparse_attn_raster(q_r, k, v, rp, ci, row_map, block=bs, q_raster=True, nqb=nqb,
                                     out=torch.empty((nqb * bs, heads, d), dtype=torch.float32, device=dev))
    torch.cuda.synchronize()
