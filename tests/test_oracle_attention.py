"""Pins of the oracle attention: select-all equals dense equals the textbook
formula and torch's SDPA in float64; brute force over a token mask; closed
forms (Q = 0, one key, V = 1); list-order invariance; padding and empty
lists."""

import math

import numpy as np
import pytest
import torch

from oracle import attention, route
from oracle.numerics import bf16_bits_to_f64

import workloads


def _f64(t):
    if t.dtype == torch.bfloat16:
        return bf16_bits_to_f64(t.contiguous().view(torch.int16).numpy())
    return t.double().numpy()


@pytest.fixture(scope="module")
def c1():
    w = workloads.c1()
    return w, _f64(w.q[0]), _f64(w.k[0]), _f64(w.v[0])


def test_select_all_equals_dense_equals_sdpa(c1):
    w, q, k, v = c1
    lists = [list(range(w.nkb))] * w.nqb
    o_sel, l_sel = attention.block_sparse_head(q, k, v, w.q_len, w.k_len, w.bs, lists, w.scale)
    o_den, l_den = attention.dense_head(q, k, v, w.q_len, w.k_len, w.bs, w.scale)
    assert np.array_equal(o_sel, o_den) and np.array_equal(l_sel, l_den)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, None], torch.from_numpy(k)[None, None],
        torch.from_numpy(v)[None, None], scale=w.scale)[0, 0].numpy()
    assert np.max(np.abs(o_den - ref)) < 1e-12
    z = q @ k.T * w.scale
    lse = np.log(np.exp(z - z.max(1, keepdims=True)).sum(1)) + z.max(1)
    assert np.max(np.abs(l_den - lse)) < 1e-12


def test_brute_force_token_mask(c1):
    w, q, k, v = c1
    r = route.route_head(q, k, w.q_len, w.k_len, w.bs, scale=w.scale, k_per_row=w.k_per_row)
    o, l = attention.block_sparse_head(q, k, v, w.q_len, w.k_len, w.bs, r["lists"], w.scale)
    o2, l2 = attention.token_mask_head(q, k, v, w.q_len, w.k_len, w.bs, r["lists"], w.scale)
    assert np.max(np.abs(o - o2)) < 1e-12 and np.max(np.abs(l - l2)) < 1e-12


def test_list_order_invariance(c1):
    w, q, k, v = c1
    rng = np.random.default_rng(5)
    lists = [sorted(rng.choice(w.nkb, 4, replace=False).tolist()) for _ in range(w.nqb)]
    shuffled = [list(rng.permutation(l)) for l in lists]
    o1, _ = attention.block_sparse_head(q, k, v, w.q_len, w.k_len, w.bs, lists, w.scale)
    o2, _ = attention.block_sparse_head(q, k, v, w.q_len, w.k_len, w.bs, shuffled, w.scale)
    assert np.max(np.abs(o1 - o2)) < 1e-12


def test_values_of_ones_give_ones(c1):
    """Each softmax row sums to one: with V = 1 every valid output is 1."""
    w, q, k, _v = c1
    ones = np.ones_like(_v)
    lists = [[0, 3, 5, 15]] * w.nqb
    o, _ = attention.block_sparse_head(q, k, ones, w.q_len, w.k_len, w.bs, lists, w.scale)
    assert np.max(np.abs(o - 1.0)) < 1e-13


def test_zero_query_gives_mean_of_values(c1):
    w, _q, k, v = c1
    q0 = np.zeros((w.nqb * w.bs, k.shape[1]))
    lists = [[1, 2], [7], [0, 15], [4, 5, 6]]
    o, lse = attention.block_sparse_head(q0, k, v, w.q_len, w.k_len, w.bs, lists, w.scale)
    for i, blocks in enumerate(lists):
        rows = np.concatenate([np.arange(b * 64, b * 64 + 64) for b in blocks])
        assert np.max(np.abs(o[i * 64:(i + 1) * 64] - v[rows].mean(0))) < 1e-13
        assert np.allclose(lse[i * 64:(i + 1) * 64], math.log(len(rows)), atol=1e-13)


def test_single_valid_key_returns_its_value():
    rng = np.random.default_rng(2)
    bs, d = 8, 16
    q = rng.standard_normal((bs, d))
    k = rng.standard_normal((3 * bs, d))
    v = rng.standard_normal((3 * bs, d))
    o, lse = attention.block_sparse_head(q, k, v, [bs], [bs, 1, bs], bs, [[1]], 0.25)
    assert np.array_equal(o, np.repeat(v[bs:bs + 1], bs, axis=0))
    assert np.allclose(lse, q @ k[bs] * 0.25, atol=1e-14)


def test_padding_rows_and_empty_lists():
    rng = np.random.default_rng(4)
    bs, d = 8, 4
    q = rng.standard_normal((2 * bs, d))
    q[bs + 3:] = 1e4  # padded rows of block 1 hold junk
    k = rng.standard_normal((2 * bs, d))
    v = rng.standard_normal((2 * bs, d))
    o, lse = attention.block_sparse_head(q, k, v, [bs, 3], [bs, bs], bs, [[0, 1], []], 0.5)
    assert np.all(o[bs:] == 0.0) and np.all(np.isneginf(lse[bs:]))
    o2, _ = attention.block_sparse_head(q, k, v, [bs, 3], [bs, bs], bs, [[0, 1], [0]], 0.5)
    assert np.all(o2[bs + 3:] == 0.0) and np.all(np.isfinite(o2[bs:bs + 3]))


def test_padded_keys_do_not_leak():
    rng = np.random.default_rng(6)
    bs, d = 8, 4
    q = rng.standard_normal((bs, d))
    k = rng.standard_normal((2 * bs, d))
    v = rng.standard_normal((2 * bs, d))
    o1, _ = attention.block_sparse_head(q, k, v, [bs], [bs, 5], bs, [[0, 1]], 0.5)
    k[bs + 5:] = 50.0
    v[bs + 5:] = 1e6
    o2, _ = attention.block_sparse_head(q, k, v, [bs], [bs, 5], bs, [[0, 1]], 0.5)
    assert np.array_equal(o1, o2)


def test_row_subset_matches_full(c1):
    w, q, k, v = c1
    lists = [[0, 1, 2, 3]] * w.nqb
    o, l = attention.block_sparse_head(q, k, v, w.q_len, w.k_len, w.bs, lists, w.scale)
    rows = [0, 5, 130, 255]
    o2, l2 = attention.block_sparse_head(q, k, v, w.q_len, w.k_len, w.bs, lists, w.scale, rows=rows)
    # BLAS may sum in another order for a different row count
    assert np.max(np.abs(o[rows] - o2[rows])) < 1e-13 and np.max(np.abs(l[rows] - l2[rows])) < 1e-13
