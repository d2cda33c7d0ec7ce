"""Pins of the oracle router: pooling closed forms, the hand-worked fusion
example, special cases that reduce to the unbiased route, the selection
predicate and tie rule, and the pages' random-expectation figure."""

import json
import math
import os

import numpy as np
import pytest

from oracle import route
from oracle.numerics import bf16_bits_to_f64

import workloads


def _f64(t):
    import torch
    if t.dtype == torch.bfloat16:
        return bf16_bits_to_f64(t.contiguous().view(torch.int16).numpy())
    return t.double().numpy()


# ---------------------------------------------------------------- pooling

def test_pool_constant_block_exact():
    x = np.full((3 * 8, 4), 0.375)
    lens = np.array([8, 8, 5])
    x[2 * 8 + 5:, :] = 1.0e4  # padding must not leak in
    m = route.pool_blocks(x, lens, 8)
    assert np.array_equal(m, np.full((3, 4), 0.375))


def test_pool_sum_exact_for_bf16_values():
    rng = np.random.default_rng(0)
    vals = rng.standard_normal((128 * 4, 16)).astype(np.float32)
    bits = (vals.view(np.uint32) >> 16).astype(np.uint16)
    x = bf16_bits_to_f64(bits)
    lens = np.array([128, 128, 128, 72])
    m = route.pool_blocks(x, lens, 128)
    for b, n in enumerate(lens):
        for c in range(16):
            # the mean is the correctly rounded quotient of the exact sum
            exact = math.fsum(x[b * 128: b * 128 + n, c].tolist())
            assert m[b, c] == exact / n


def test_pool_empty_block_is_nan_and_not_visible():
    x = np.ones((2 * 4, 2))
    m = route.pool_blocks(x, np.array([4, 0]), 4)
    assert np.all(np.isnan(m[1]))


# ---------------------------------------------------------------- fusion

def test_fusion_worked_example(golden_dir):
    ex = json.load(open(os.path.join(golden_dir, "fusion_worked_example.json")))
    c = ex["constants"]
    qbar = np.array([[1.0]])
    kbar = np.array([[0.0], [math.log(2.0)], [math.log(3.0)], [0.0]])
    vis = np.ones(4, dtype=bool)
    p = route.importance(qbar, kbar, 1.0, vis)
    assert np.allclose(p[0], ex["p"], rtol=0, atol=1e-15)
    assert np.allclose(route.rescale_overlap(np.array(ex["overlap"]), c["tau"], c["g_ref"]), ex["g_hat"], atol=1e-15)
    pf, zero, unvetted = route.fuse(p, np.array([ex["overlap"]]), c["lambda"], c["tau"], c["g_ref"])
    assert np.allclose(pf[0], ex["p_fused"], rtol=0, atol=1e-15)
    assert not zero[0] and not unvetted[0]
    assert route.top_k_ascending(pf[0], vis, 2).tolist() == ex["top2_fused"]
    assert route.top_k_ascending(p[0], vis, 2).tolist() == ex["top2_unbiased"]


def test_fusion_threshold_is_inclusive():
    g = np.array([0.1, 0.1000001, 0.2, 0.5])
    gh = route.rescale_overlap(g, 0.1, 0.2)
    assert gh[0] == 0.0 and gh[1] > 0.5 and gh[2] == 1.0 and gh[3] == 1.0


def _c3_head(h=0):
    w = workloads.c3(heads=[h])
    q, k = _f64(w.q[0]), _f64(w.k[0])
    return w, q, k


def test_lambda_zero_and_zero_rows_reduce_to_unbiased():
    w, q, k = _c3_head()
    kr = w.k_per_row[: w.nqb]
    base = route.route_head(q, k, w.q_len, w.k_len, w.bs, scale=w.scale, k_per_row=kr)
    lam0 = route.route_head(q, k, w.q_len, w.k_len, w.bs, scale=w.scale, k_per_row=kr,
                            overlap=w.overlap, lam=0.0)
    biased = route.route_head(q, k, w.q_len, w.k_len, w.bs, scale=w.scale, k_per_row=kr,
                              overlap=w.overlap, lam=w.lam, tau=w.tau, g_ref=w.g_ref)
    for i in range(w.nqb):
        assert np.array_equal(lam0["lists"][i], base["lists"][i])
    zero = biased["zero_rows"]
    assert zero.sum() == 11
    changed = 0
    for i in range(w.nqb):
        if zero[i]:
            assert np.array_equal(biased["lists"][i], base["lists"][i])
        else:
            changed += int(not np.array_equal(biased["lists"][i], base["lists"][i]))
    assert changed > 0  # the bias does act on covered rows


def test_uniform_full_overlap_preserves_order():
    w, q, k = _c3_head()
    kr = w.k_per_row[: w.nqb]
    g = np.full_like(w.overlap, 0.9)
    base = route.route_head(q, k, w.q_len, w.k_len, w.bs, scale=w.scale, k_per_row=kr)
    full = route.route_head(q, k, w.q_len, w.k_len, w.bs, scale=w.scale, k_per_row=kr, overlap=g)
    for i in range(w.nqb):
        assert np.array_equal(full["lists"][i], base["lists"][i])
        assert np.allclose(full["p_fused"][i], base["p"][i], atol=1e-15)


def test_fused_rows_normalised_and_boost_bounded():
    w, q, k = _c3_head()
    kr = w.k_per_row[: w.nqb]
    r = route.route_head(q, k, w.q_len, w.k_len, w.bs, scale=w.scale, k_per_row=kr,
                         overlap=w.overlap, lam=w.lam, tau=w.tau, g_ref=w.g_ref)
    assert np.allclose(r["p_fused"].sum(axis=1), 1.0, atol=1e-12)
    ratio = r["p_fused"] / r["p"]
    # per row the boost of any block over the least boosted one is <= 1 + lambda
    spread = ratio.max(axis=1) / ratio.min(axis=1)
    assert np.all(spread <= 1.0 + w.lam + 1e-12)
    # unvetted blocks (g <= tau) share one factor per row
    gh = route.rescale_overlap(w.overlap, w.tau, w.g_ref)
    for i in range(w.nqb):
        un = gh[i] == 0
        if un.any():
            assert np.ptp(ratio[i, un]) < 1e-12


def test_monotone_in_overlap():
    w, q, k = _c3_head()
    kr = w.k_per_row[: w.nqb]
    r = route.route_head(q, k, w.q_len, w.k_len, w.bs, scale=w.scale, k_per_row=kr,
                         overlap=w.overlap, lam=w.lam, tau=w.tau, g_ref=w.g_ref)
    g2 = w.overlap.copy()
    for i in range(w.nqb):
        if not r["zero_rows"][i]:
            g2[i, r["lists"][i]] = 1.0  # raise overlap of selected blocks
    r2 = route.route_head(q, k, w.q_len, w.k_len, w.bs, scale=w.scale, k_per_row=kr,
                          overlap=g2, lam=w.lam, tau=w.tau, g_ref=w.g_ref)
    for i in range(w.nqb):
        assert np.array_equal(r2["lists"][i], r["lists"][i])


def test_kappa_order_matches_fused_distribution():
    w, q, k = _c3_head(3)
    kr = w.k_per_row[: w.nqb]
    r = route.route_head(q, k, w.q_len, w.k_len, w.bs, scale=w.scale, k_per_row=kr,
                         overlap=w.overlap, lam=w.lam, tau=w.tau, g_ref=w.g_ref)
    vis = r["visible"]
    for i in range(w.nqb):
        a = route.top_k_ascending(r["kappa"][i], vis, kr[i])
        assert np.array_equal(a, r["lists"][i])


# ---------------------------------------------------------------- selection

def test_selection_predicate_every_row():
    w, q, k = _c3_head(5)
    kr = w.k_per_row[: w.nqb]
    r = route.route_head(q, k, w.q_len, w.k_len, w.bs, scale=w.scale, k_per_row=kr,
                         overlap=w.overlap, lam=w.lam, tau=w.tau, g_ref=w.g_ref)
    for i in range(w.nqb):
        sel = set(r["lists"][i].tolist())
        assert len(sel) == 50
        assert r["lists"][i].tolist() == sorted(sel)
        sc = r["p_fused"][i]
        worst_in = min((sc[j], -j) for j in sel)
        best_out = max((sc[j], -j) for j in range(w.nkb) if j not in sel)
        assert worst_in > best_out


def test_ties_go_to_lower_index():
    s = np.array([0.5, 0.9, 0.7, 0.9, 0.7, 0.1])
    vis = np.ones(6, dtype=bool)
    assert route.top_k_ascending(s, vis, 2).tolist() == [1, 3]
    assert route.top_k_ascending(s, vis, 3).tolist() == [1, 2, 3]
    s2 = np.array([0.0, -0.0, 0.0])
    assert route.top_k_ascending(s2, np.ones(3, bool), 2).tolist() == [0, 1]


def test_duplicate_block_tie():
    # copy KV block 4 into block 9; a budget that cuts between them keeps 4
    rng = np.random.default_rng(7)
    bs, d = 4, 8
    k = rng.standard_normal((12 * bs, d))
    k[9 * bs:10 * bs] = k[4 * bs:5 * bs]
    q = rng.standard_normal((1 * bs, d))
    base = route.route_head(q, k, [bs], [bs] * 12, bs, scale=1.0, k_per_row=[12])
    order = np.lexsort((np.arange(12), -base["p"][0]))
    pos4 = int(np.nonzero(order == 4)[0][0])
    r = route.route_head(q, k, [bs], [bs] * 12, bs, scale=1.0, k_per_row=[pos4 + 1])
    assert 4 in r["lists"][0] and 9 not in r["lists"][0]


def test_budget_above_candidates_selects_all():
    w = workloads.c4(c=1, heads=[0])
    q, k = _f64(w.q[0]), _f64(w.k[0])
    r = route.route_head(q, k, w.q_len, w.k_len, w.bs, scale=w.scale, k_per_row=w.k_per_row[:37])
    for i in range(w.nqb):
        assert r["lists"][i].tolist() == list(range(37))


def test_dense_tail_appended_and_empty_query_block():
    rng = np.random.default_rng(3)
    bs, d = 4, 8
    k = rng.standard_normal((10 * bs, d))
    q = rng.standard_normal((2 * bs, d))
    r = route.route_head(q, k, [bs, 0], [bs] * 8 + [bs, 2], bs, scale=1.0,
                         k_per_row=[3, 3], n_dense_tail=2)
    assert len(r["lists"][0]) == 5 and r["lists"][0][-2:].tolist() == [8, 9]
    assert len(r["lists"][1]) == 0


def test_random_routes_hit_budget_fraction(golden_dir):
    """Closed form from the pages: a budget of 50 of 143 blocks chosen
    without information overlaps any fixed set at 50/143 ~ 0.350."""
    c = json.load(open(os.path.join(golden_dir, "velox_constants.json")))
    rng = np.random.default_rng(11)
    bs, d, nkb, K = 2, 16, c["candidate_blocks"], c["route_budget"]
    fixed = set(rng.choice(nkb, K, replace=False).tolist())
    hits = []
    for _ in range(200):
        q = rng.standard_normal((bs, d))
        k = rng.standard_normal((nkb * bs, d))
        r = route.route_head(q, k, [bs], [bs] * nkb, bs, scale=1.0, k_per_row=[K])
        hits.append(len(fixed & set(r["lists"][0].tolist())) / K)
    assert abs(K / nkb - c["random_expectation"]) < 5e-4
    assert abs(np.mean(hits) - c["random_expectation"]) < 0.02


def test_csr_concatenation():
    rp, col = route.to_csr([[1, 4], [], [0, 2, 3]])
    assert rp.tolist() == [0, 2, 2, 5] and col.tolist() == [1, 4, 0, 2, 3]
