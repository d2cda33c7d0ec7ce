"""The router's no-allocation entry point (bsa_route_topk_static, for
callers that cannot allocate) against the workspace entry point
(bsa_route_topk) on the same inputs: bitwise equal row pointers, lists and
fallback counts, over two calls in a row, the second on a smaller problem,
so the shared scratch holds the first call's contents when the second
starts."""

import numpy as np
import pytest
import torch

import workloads

from helpers import need_gpu

pytestmark = pytest.mark.gpu


def _i32(a, dev):
    return torch.from_numpy(np.asarray(a, dtype=np.int32)).to(dev)


def _compare(bsa, dev, q, k, *, nqb, nkb, q_len, kv_len, scale, k_fixed, overlap=None, kpool=None):
    kw = dict(block=128, nqb=nqb, nkb=nkb, scale=scale, q_block_len=q_len, kv_block_len=kv_len, k_fixed=k_fixed,
              overlap=overlap)
    ref = bsa.route_topk(q, k, **kw)
    heads = q.shape[0]
    cap = bsa.route_capacity(heads, nqb, nkb, k_fixed)
    out = {"row_ptr": torch.full((heads * nqb + 1,), -7, dtype=torch.int32, device=dev),
           "col_idx": torch.full((cap,), -7, dtype=torch.int32, device=dev),
           "fallback_counts": torch.full((2,), -7, dtype=torch.int32, device=dev)}
    if kpool is not None:
        kw["kpool"], kw["kpool_valid_blocks"] = kpool, 0
    got = bsa.route_topk_static(q, k, out=out, **kw)
    torch.cuda.synchronize()
    rp = ref["row_ptr"].cpu().numpy()
    assert np.array_equal(got["row_ptr"].cpu().numpy(), rp)
    n = int(rp[-1])
    assert n == heads * nqb * min(k_fixed, nkb)
    assert np.array_equal(got["col_idx"][:n].cpu().numpy(), ref["col_idx"][:n].cpu().numpy())
    assert np.array_equal(got["fallback_counts"].cpu().numpy(), ref["fallback_counts"].cpu().numpy())


def test_static_router_matches_workspace_router_twice():
    dev = need_gpu()
    import block_sparse_attention_gilbert_amd as bsa
    # 1st call: growing-context layer at chunk 12 (40 heads, 444 candidates),
    # pooled keys in the scratch (about 25 MB of it)
    w = workloads.c4(12)
    print("static router: C4 chunk 12", flush=True)
    _compare(bsa, dev, w.q.to(dev), w.k.to(dev), nqb=w.nqb, nkb=w.nkb, q_len=_i32(w.q_len, dev),
             kv_len=_i32(w.k_len, dev), scale=w.scale, k_fixed=int(w.k_per_row[0]))
    # 2nd call: the smaller biased layer (12 heads, 143 candidates, overlap
    # with all-zero rows), pooled keys in a caller cache
    w2 = workloads.c3()
    print("static router: C3", flush=True)
    kpool = torch.empty((w2.heads, w2.nkb, w2.d), dtype=torch.float64, device=dev)
    _compare(bsa, dev, w2.q.to(dev), w2.k.to(dev), nqb=w2.nqb, nkb=w2.nkb, q_len=_i32(w2.q_len, dev),
             kv_len=_i32(w2.k_len, dev), scale=w2.scale, k_fixed=int(w2.k_per_row[0]),
             overlap=torch.from_numpy(w2.overlap).to(dev), kpool=kpool)
