"""One routed-attention call captured into a HIP graph: every replay, with
eager calls and synchronisations between the replays, must equal the eager
call bitwise (the library records no memset node and allocates nothing
during the call).  And the call, with its fused passes, equals the plain
chain of separate passes bit for bit."""

import pytest
import torch

import workloads

from helpers import need_gpu

pytestmark = pytest.mark.gpu


def test_step_graph_replays_match_eager():
    dev = need_gpu()
    from block_sparse_attention_gilbert_amd import gilbert_perm
    from block_sparse_attention_gilbert_amd.pipeline import RoutedAttention
    w = workloads.c4(c=3, heads=[0, 1, 2])
    ra = RoutedAttention((3, 30, 52), w.heads, w.d, w.bs, 3, device=dev, k_cap=50,
                         k_store=w.k.contiguous().to(dev), v_store=w.v.contiguous().to(dev))
    ks, vs = ra.slot(2)
    q_r = gilbert_perm(w.q.to(dev), ra.perm, block=128, inverse=True)
    k_r = gilbert_perm(ks, ra.perm, block=128, inverse=True).clone()
    v_r = gilbert_perm(vs, ra.perm, block=128, inverse=True).clone()
    o_eager = ra.step(q_r, k_r, v_r, 2)[0].clone()
    lse_eager = ra.lse.clone()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ra.step(q_r, k_r, v_r, 2)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        ra.step(q_r, k_r, v_r, 2)
    torch.cuda.synchronize()
    for rep in range(4):
        ra.o_raster.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ra.o_raster, o_eager), rep
        assert torch.equal(ra.lse, lse_eager), rep
        ra.step(q_r, k_r, v_r, 2)            # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(ra.o_raster, o_eager), rep


def test_step_equals_the_stage_by_stage_chain():
    """The step (K block means inside its permutation, Q only pooled and
    read in raster order by the attention, O written through the curve)
    gives the same bits as the plain chain of separate passes: permute Q,
    K and V, route (pooling Q and K itself), attend into blocked rows,
    permute O back."""
    dev = need_gpu()
    from block_sparse_attention_gilbert_amd import gilbert_perm
    from block_sparse_attention_gilbert_amd.pipeline import RoutedAttention
    w = workloads.c4(c=4, heads=[2, 9, 33])
    mk = lambda: RoutedAttention((3, 30, 52), w.heads, w.d, w.bs, 4, device=dev, k_cap=50,
                                 k_store=w.k.contiguous().to(dev), v_store=w.v.contiguous().to(dev))
    ra, rb = mk(), mk()
    ks, vs = ra.slot(3)
    q_r = gilbert_perm(w.q.to(dev), ra.perm, block=128, inverse=True)
    k_r = gilbert_perm(ks, ra.perm, block=128, inverse=True).clone()
    v_r = gilbert_perm(vs, ra.perm, block=128, inverse=True).clone()
    o_step, r_step = ra.step(q_r, k_r, v_r, 3)
    rb.use_kpool = False
    rb.to_blocks(k_r, rb.slot(3)[0])
    rb.to_blocks(v_r, rb.slot(3)[1])
    rb.to_blocks(q_r, rb.q_blk)
    r_chain = rb.route_and_attend(3)
    o_chain = rb.to_raster(rb.o_blk, torch.empty_like(q_r))
    torch.cuda.synchronize()
    n = int(r_step["row_ptr"][-1])
    assert torch.equal(r_step["row_ptr"], r_chain["row_ptr"])
    assert torch.equal(r_step["col_idx"][:n], r_chain["col_idx"][:n])
    assert torch.equal(o_step, o_chain)
    assert torch.equal(ra.lse, rb.lse)
    # the step without the pooled-key cache (separate passes over Q, K and V,
    # the router pooling the whole history): the same bits again
    rc = mk()
    rc.use_kpool = False
    o_nc, r_nc = rc.step(q_r, k_r, v_r, 3)
    torch.cuda.synchronize()
    assert torch.equal(r_nc["col_idx"][:n], r_chain["col_idx"][:n])
    assert torch.equal(o_nc, o_step) and torch.equal(rc.lse, ra.lse)
