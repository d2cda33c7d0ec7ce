"""Pins of the oracle layouts: a hand-worked permutation, round trip,
padding, block lengths of the 3 x 30 x 52 chunk."""

import numpy as np

from oracle import layout
from oracle.gilbert import gilbert_order


def test_hand_worked_forward_and_inverse():
    # L = 5 tokens, 1 head, d = 1, blocks of 2: perm = [3, 0, 4, 1, 2]
    src = np.array([10.0, 11.0, 12.0, 13.0, 14.0]).reshape(5, 1, 1)
    perm = np.array([3, 0, 4, 1, 2])
    dst = layout.permute_forward(src, perm, 2)
    assert dst.shape == (1, 6, 1)
    assert dst[0, :, 0].tolist() == [13.0, 10.0, 14.0, 11.0, 12.0, 0.0]
    back = layout.permute_inverse(dst, perm, 5)
    assert np.array_equal(back, src)


def test_round_trip_and_padding_chunk():
    perm, _ = gilbert_order(3, 30, 52)
    rng = np.random.default_rng(1)
    src = rng.standard_normal((4680, 3, 8))
    for bs in (64, 128):
        dst = layout.permute_forward(src, perm, bs)
        assert dst.shape[1] == layout.n_blocks(4680, bs) * bs
        assert np.all(dst[:, 4680:, :] == 0)
        assert np.array_equal(layout.permute_inverse(dst, perm, 4680), src)
        # per-head multiset of rows is preserved
        for h in range(3):
            assert np.isclose(dst[h].sum(), src[:, h, :].sum(), rtol=0, atol=1e-9)


def test_chunk_block_lengths():
    assert layout.n_blocks(4680, 128) == 37 and layout.n_blocks(4680, 64) == 74
    l128 = layout.chunk_block_lengths(4680, 128, 2)
    assert len(l128) == 74 and l128[36] == 72 and l128[73] == 72 and l128[:36].min() == 128
    l64 = layout.chunk_block_lengths(4680, 64)
    assert l64[-1] == 8 and l64.sum() == 4680
