"""GPU parity of the Gilbert order (bit-exact against the oracle's
enumeration) and of the raster <-> Gilbert permutation (bitwise)."""

import itertools

import numpy as np
import pytest
import torch

from oracle import layout as olay
from oracle.gilbert import gilbert_order

from helpers import f64, need_gpu

pytestmark = pytest.mark.gpu


def test_index_config_shapes():
    dev = need_gpu()
    import block_sparse_attention_gilbert_amd as bsa
    for shape in [(3, 30, 52), (1, 30, 52), (21, 30, 52), (3, 60, 104), (1, 1, 1), (1, 1, 37), (2, 2, 2)]:
        perm, inv = bsa.gilbert_index(*shape, device=dev)
        ref, ref_inv = gilbert_order(*shape)
        assert np.array_equal(perm.cpu().numpy(), ref), shape
        assert np.array_equal(inv.cpu().numpy(), ref_inv), shape


def test_index_small_shape_sweep():
    dev = need_gpu()
    import block_sparse_attention_gilbert_amd as bsa
    for shape in itertools.product(range(1, 7), repeat=3):
        perm, _ = bsa.gilbert_index(*shape, device=dev, with_inverse=False)
        assert np.array_equal(perm.cpu().numpy(), gilbert_order(*shape)[0]), shape


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("block,d", [(128, 128), (64, 128), (64, 64), (128, 64)])
def test_permute_bitwise(dtype, block, d):
    dev = need_gpu()
    import block_sparse_attention_gilbert_amd as bsa
    T, H, W = 3, 30, 52
    L, heads = T * H * W, 3
    g = torch.Generator().manual_seed(11)
    src = torch.randn((L, heads, d), generator=g).to(dtype)
    perm, _ = bsa.gilbert_index(T, H, W, device=dev)
    dst = bsa.gilbert_perm(src.to(dev), perm, block=block)
    ref = olay.permute_forward(f64(src), gilbert_order(T, H, W)[0], block)
    assert np.array_equal(f64(dst), ref)              # bitwise (values exact in float64)
    assert torch.all(dst[:, L:, :] == 0)
    back = bsa.gilbert_perm(dst, perm, block=block, inverse=True)
    assert torch.equal(back.cpu(), src)


def test_permute_into_store_slot_and_token_stride():
    dev = need_gpu()
    import block_sparse_attention_gilbert_amd as bsa
    T, H, W = 3, 30, 52
    L, heads, d, block = T * H * W, 4, 128, 128
    nbc = -(-L // block)
    # raster rows carry q, k, v side by side: token stride 3*heads*d
    fused = torch.randn((L, 3, heads, d), generator=torch.Generator().manual_seed(3)).to(torch.bfloat16).to(dev)
    k_raster = fused[:, 1]
    store = torch.full((heads, 3 * nbc * block, d), 7.0, dtype=torch.bfloat16, device=dev)
    perm, _ = bsa.gilbert_index(T, H, W, device=dev)
    slot = store[:, nbc * block: 2 * nbc * block]
    bsa.gilbert_perm(k_raster, perm, block=block, dst=slot)
    ref = olay.permute_forward(f64(k_raster), gilbert_order(T, H, W)[0], block)
    assert np.array_equal(f64(slot), ref)
    assert torch.all(store[:, : nbc * block] == 7.0) and torch.all(store[:, 2 * nbc * block:] == 7.0)
    out = torch.zeros((L, 2, heads, d), dtype=torch.bfloat16, device=dev)
    bsa.gilbert_perm(slot, perm, block=block, inverse=True, dst=out[:, 1])
    assert torch.equal(out[:, 1], k_raster) and torch.all(out[:, 0] == 0)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("block,d", [(128, 128), (64, 128), (64, 64), (128, 64)])
def test_permute_pool_bitwise_and_exact_means(dtype, block, d):
    """The fused pass writes the same bits as the plain permutation and the
    oracle's block means of the permuted rows, exactly (ragged last block)."""
    dev = need_gpu()
    import block_sparse_attention_gilbert_amd as bsa
    from oracle import route as oroute
    T, H, W = 3, 30, 52
    L, heads = T * H * W, 3
    src = torch.randn((L, heads, d), generator=torch.Generator().manual_seed(12)).to(dtype)
    perm, _ = bsa.gilbert_index(T, H, W, device=dev)
    dst, pool = bsa.gilbert_perm_pool(src.to(dev), perm, block=block)
    plain = bsa.gilbert_perm(src.to(dev), perm, block=block)
    torch.cuda.synchronize()
    assert torch.equal(dst, plain)
    ref = olay.permute_forward(f64(src), gilbert_order(T, H, W)[0], block)
    lens = olay.chunk_block_lengths(L, block)
    assert lens[-1] < block
    for h in range(heads):
        assert np.array_equal(pool[h].cpu().numpy(), oroute.pool_blocks(ref[h], lens, block)), h
    # the block means alone (nothing permuted): the same values
    none, pool2 = bsa.gilbert_perm_pool(src.to(dev), perm, block=block, pool_only=True)
    torch.cuda.synchronize()
    assert none is None and torch.equal(pool2, pool)


def test_permute_pool_into_cache_slice():
    """K of one chunk into a store slot and its means into the matching
    slice of a pooled-key cache (both head-strided views); the rest of the
    store and of the cache is untouched, and a raster tensor with a wider
    token stride is read correctly."""
    dev = need_gpu()
    import block_sparse_attention_gilbert_amd as bsa
    from oracle import route as oroute
    T, H, W = 3, 30, 52
    L, heads, d, block = T * H * W, 4, 128, 128
    nbc = -(-L // block)
    fused = torch.randn((L, 3, heads, d), generator=torch.Generator().manual_seed(5)).to(torch.bfloat16).to(dev)
    k_raster = fused[:, 1]
    store = torch.full((heads, 3 * nbc * block, d), 7.0, dtype=torch.bfloat16, device=dev)
    cache = torch.full((heads, 3 * nbc, d), -1.0, dtype=torch.float64, device=dev)
    perm, _ = bsa.gilbert_index(T, H, W, device=dev)
    slot = store[:, nbc * block: 2 * nbc * block]
    bsa.gilbert_perm_pool(k_raster, perm, block=block, dst=slot, pool=cache[:, nbc: 2 * nbc])
    torch.cuda.synchronize()
    ref = olay.permute_forward(f64(k_raster), gilbert_order(T, H, W)[0], block)
    assert np.array_equal(f64(slot), ref)
    lens = olay.chunk_block_lengths(L, block)
    for h in range(heads):
        assert np.array_equal(cache[h, nbc: 2 * nbc].cpu().numpy(), oroute.pool_blocks(ref[h], lens, block))
    assert torch.all(store[:, : nbc * block] == 7.0) and torch.all(store[:, 2 * nbc * block:] == 7.0)
    assert torch.all(cache[:, :nbc] == -1.0) and torch.all(cache[:, 2 * nbc:] == -1.0)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("block,d", [(128, 128), (64, 64)])
def test_permute_pool_batch(dtype, block, d):
    """Q (block means only), K (store slot + cache slice) and V (store slot,
    no means) of one chunk through one launch: every output equals the
    oracle's, bitwise, and the stores and cache outside the slots are
    untouched."""
    dev = need_gpu()
    import block_sparse_attention_gilbert_amd as bsa
    from oracle import route as oroute
    T, H, W = 3, 30, 52
    L, heads = T * H * W, 5
    nbc = -(-L // block)
    fused = torch.randn((L, 3, heads, d), generator=torch.Generator().manual_seed(21)).to(dtype).to(dev)
    q, k, v = fused[:, 0], fused[:, 1], fused[:, 2]
    k_store = torch.full((heads, 3 * nbc * block, d), 7.0, dtype=dtype, device=dev)
    v_store = torch.full((heads, 3 * nbc * block, d), 5.0, dtype=dtype, device=dev)
    cache = torch.full((heads, 3 * nbc, d), -1.0, dtype=torch.float64, device=dev)
    qbar = torch.full((heads, nbc, d), -2.0, dtype=torch.float64, device=dev)
    perm, _ = bsa.gilbert_index(T, H, W, device=dev)
    ks, vs = k_store[:, nbc * block: 2 * nbc * block], v_store[:, nbc * block: 2 * nbc * block]
    bsa.gilbert_perm_pool_batch([(q, None, qbar), (k, ks, cache[:, nbc: 2 * nbc]), (v, vs, None)], perm,
                                block=block)
    torch.cuda.synchronize()
    order = gilbert_order(T, H, W)[0]
    lens = olay.chunk_block_lengths(L, block)
    refs = [olay.permute_forward(f64(x), order, block) for x in (q, k, v)]
    assert np.array_equal(f64(ks), refs[1]) and np.array_equal(f64(vs), refs[2])
    for h in range(heads):
        assert np.array_equal(qbar[h].cpu().numpy(), oroute.pool_blocks(refs[0][h], lens, block)), h
        assert np.array_equal(cache[h, nbc: 2 * nbc].cpu().numpy(), oroute.pool_blocks(refs[1][h], lens, block)), h
    for store, fill in ((k_store, 7.0), (v_store, 5.0)):
        assert torch.all(store[:, : nbc * block] == fill) and torch.all(store[:, 2 * nbc * block:] == fill)
    assert torch.all(cache[:, :nbc] == -1.0) and torch.all(cache[:, 2 * nbc:] == -1.0)
    # one job alone, and the single-tensor entry on the same input: the same bits
    dst1, pool1 = bsa.gilbert_perm_pool(k, perm, block=block)
    ks2 = torch.empty_like(dst1)
    pool2 = torch.empty_like(pool1)
    bsa.gilbert_perm_pool_batch([(k, ks2, pool2)], perm, block=block)
    torch.cuda.synchronize()
    assert torch.equal(ks2, dst1) and torch.equal(pool2, pool1)


def test_index_large_grid():
    dev = need_gpu()
    import block_sparse_attention_gilbert_amd as bsa
    shape = (21, 60, 104)   # 131,040 cells: a 21-frame, 2x-resolution chunk
    perm, inv = bsa.gilbert_index(*shape, device=dev)
    ref, ref_inv = gilbert_order(*shape)
    assert np.array_equal(perm.cpu().numpy(), ref)
    assert np.array_equal(inv.cpu().numpy(), ref_inv)


def _mixed_magnitudes(shape, span_log2, seed, dtype):
    """Values of random sign and magnitude 2^U(-span/2, span/2), with every
    second row of a block cancelling the row before it in some columns: sums
    that a plain float64 accumulation rounds, in an order-dependent way."""
    rng = np.random.default_rng(seed)
    x = 2.0 ** rng.uniform(-span_log2 / 2, span_log2 / 2, shape) * rng.choice([-1.0, 1.0], shape)
    x[1::2, :, ::3] = -x[0::2, :, ::3][: x[1::2].shape[0]]
    return torch.from_numpy(x.astype(np.float32)).to(dtype)


@pytest.mark.parametrize("dtype,span", [(torch.float32, 60), (torch.bfloat16, 36)])
def test_permute_pool_exact_means_mixed_magnitudes(dtype, span):
    """Block means of rows whose magnitudes span 2^60 (float32: summed as
    exact pairs) or 2^36 (bf16: a plain float64 sum, exact below 2^39) equal
    the oracle's exact means bit for bit (its exact sum, rounded once): the
    fused pass's summation order does not show."""
    dev = need_gpu()
    import block_sparse_attention_gilbert_amd as bsa
    from oracle import route as oroute
    T, H, W = 2, 12, 20
    L, heads, d, block = T * H * W, 2, 64, 64
    src = _mixed_magnitudes((L, heads, d), span, 31, dtype)
    perm, _ = bsa.gilbert_index(T, H, W, device=dev)
    _, pool = bsa.gilbert_perm_pool(src.to(dev), perm, block=block)
    torch.cuda.synchronize()
    ref = olay.permute_forward(f64(src), gilbert_order(T, H, W)[0], block)
    lens = olay.chunk_block_lengths(L, block)
    plain_differs = 0
    for h in range(heads):
        want = oroute.pool_blocks(ref[h], lens, block)
        assert np.array_equal(pool[h].cpu().numpy(), want), h
        for b, n in enumerate(lens):
            plain_differs += int(np.sum(ref[h][b * block: b * block + n].sum(axis=0) / n != want[b]))
    if dtype == torch.float32:
        assert plain_differs > 0   # the inputs do reach sums a plain accumulation rounds
