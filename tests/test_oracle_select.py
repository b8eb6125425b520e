"""Pins for O3 (Quest-style page scores, top-K page selection) and O4 (candidate lists).

Pins: a hand-computed score (tests/golden/page_score_closed_form.json); the special case of
one-token pages, where the bound is the dot product itself and the selection is textbook top-k of
q.k (numpy argsort of float64 dot products); the upper-bound property against float64 dot products;
tie-breaking and the budget count; keep fraction 1 keeps every page.  The group score's per-channel
form: for one head it is the per-head score bit for bit, for groups it is the exact sum of the
per-head bounds within its rounding error, and its float32 fused multiply-add matches exact rational
arithmetic, including sums that float64 rounds onto a float32 midpoint.
"""
from fractions import Fraction

import json
import os

import numpy as np
import pytest

from oracle import numerics, quantize, select

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _bits(x):
    return numerics.f32_to_bf16_bits(np.asarray(x, np.float32))


def test_closed_form_score():
    g = json.load(open(os.path.join(GOLD, "page_score_closed_form.json")))
    q = np.zeros(128, np.float32)
    for c, v in g["q"].items():
        q[int(c)] = v
    kmin = np.zeros((len(g["pages"]), 128), np.float32)
    kmax = np.zeros_like(kmin)
    for j, pg in enumerate(g["pages"]):
        for c, v in pg["min"].items():
            kmin[j, int(c)] = v
        for c, v in pg["max"].items():
            kmax[j, int(c)] = v
    s = select.page_scores_head(_bits(q), kmin, kmax)
    assert s.tolist() == [pg["sigma"] for pg in g["pages"]]


def test_one_token_pages_reduce_to_the_dot_product_and_textbook_topk():
    rng = np.random.default_rng(0)
    P = 500
    k = numerics.bf16_to_f32(_bits(rng.standard_normal((P, 128))))
    q = _bits(rng.standard_normal(128))
    s = select.page_scores_head(q, k, k)           # a one-token page: min = max = the key
    dot = k.astype(np.float64) @ numerics.bf16_to_f32(q).astype(np.float64)
    # a float32 fold of 128 exact products: error <= 127 * 2^-24 * sum |q_c k_c|
    absum = np.abs(k.astype(np.float64)) @ np.abs(numerics.bf16_to_f32(q).astype(np.float64))
    assert np.all(np.abs(s - dot) <= 127 * 2.0**-24 * absum)
    # selection = textbook top-k of q.k when the scores are well separated at the cut
    K = 125
    order = np.argsort(-dot, kind="stable")
    if dot[order[K - 1]] - dot[order[K]] > 1e-3:
        assert np.array_equal(select.top_pages(s, K), np.sort(order[:K]))


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_score_is_an_upper_bound_of_every_key_in_the_page(seed):
    rng = np.random.default_rng(seed)
    n, G = 16 * 40 + 7, 4
    kbits = _bits(rng.standard_normal((n, 1, 128)) * np.where(rng.random(128) < 0.05, 8, 1))
    qb = _bits(rng.standard_normal((G, 128)))
    kmin, kmax = quantize.page_bounds(kbits)
    kmin, kmax = kmin[:, 0], kmax[:, 0]
    k = numerics.bf16_to_f32(kbits[:, 0]).astype(np.float64)
    gs = select.group_scores(qb, kmin, kmax)
    qf = numerics.bf16_to_f32(qb).astype(np.float64)
    for h in range(G):
        s = select.page_scores_head(qb[h], kmin, kmax)
        dots = k @ qf[h]
        for j in range(kmin.shape[0]):
            assert s[j] >= dots[j * 16:(j + 1) * 16].max() - 1e-4
    summed = k @ qf.sum(0)
    for j in range(kmin.shape[0]):
        assert gs[j] >= summed[j * 16:(j + 1) * 16].max() - 1e-4


def test_keep_count_and_ties():
    assert select.keep_count(2048, 0.25) == 512
    assert select.keep_count(8192, 0.25) == 2048
    assert select.keep_count(5, 0.25) == 2
    assert select.keep_count(1, 0.25) == 1
    assert select.keep_count(0, 0.25) == 0
    assert select.keep_count(7, 1.0) == 7
    assert select.keep_count(7, 3.0) == 7
    scores = np.array([1.0, 5.0, 5.0, 2.0, 5.0, 5.0], np.float32)
    assert select.top_pages(scores, 3).tolist() == [1, 2, 4]          # ties to the lower id
    assert select.top_pages(scores, 6).tolist() == list(range(6))


def test_candidates():
    assert select.candidates_from_pages(np.array([0, 2]), 40).tolist() == list(range(16)) + list(range(32, 40))
    assert select.candidates_from_pages(np.array([], np.int32), 40).size == 0
    assert select.candidates_from_ranges(np.array([[5, 3], [20, 0], [30, 2]])).tolist() == [5, 6, 7, 30, 31]


def _fma_exact(a, b, c):
    """a*b + c rounded once to float32 (nearest, ties to even), in exact rational arithmetic."""
    x = Fraction(float(a)) * Fraction(float(b)) + Fraction(float(c))
    f = np.float32(float(x))  # nearest double, then float32: may round twice, so fix it up exactly
    lo = f if Fraction(float(f)) <= x else np.nextafter(f, np.float32(-np.inf))
    hi = np.nextafter(lo, np.float32(np.inf))
    dl, dh = x - Fraction(float(lo)), Fraction(float(hi)) - x
    if dl < dh:
        return lo
    if dh < dl:
        return hi
    return lo if (int(np.array([lo], np.float32).view(np.uint32)[0]) & 1) == 0 else hi


def test_f32_fma_matches_exact_rounding():
    rng = np.random.default_rng(5)
    n = 3000
    a = (rng.standard_normal(n) * 2.0 ** rng.integers(-20, 20, n)).astype(np.float32)
    b = numerics.bf16_to_f32(_bits(rng.standard_normal(n) * 2.0 ** rng.integers(-20, 20, n)))
    c = (rng.standard_normal(n) * 2.0 ** rng.integers(-30, 30, n)).astype(np.float32)
    c[::7] = 0.0
    got = numerics.f32_fma(a, b, c)
    want = np.array([_fma_exact(x, y, z) for x, y, z in zip(a, b, c)], np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    # float64 rounds these sums onto a float32 midpoint; the bits it dropped decide the rounding:
    # 1 + (2^-24 + 2^-60) rounds up, (1 + 2^-23) + (2^-24 - 2^-60) rounds down
    a2 = np.array([1774001 * 2.0**-30, 262143 * 2.0**-30, -1774001 * 2.0**-30], np.float32)
    b2 = np.array([38737 * 2.0**-30, 262145 * 2.0**-30, 38737 * 2.0**-30], np.float32)
    c2 = np.array([1.0, 1.0 + 2.0**-23, -1.0], np.float32)
    got2 = numerics.f32_fma(a2, b2, c2)
    want2 = np.array([_fma_exact(x, y, z) for x, y, z in zip(a2, b2, c2)], np.float32)
    assert np.array_equal(got2.view(np.uint32), want2.view(np.uint32))
    assert got2.tolist() == [1.0 + 2.0**-23, 1.0 + 2.0**-23, -(1.0 + 2.0**-23)]
    # the naive float64-then-float32 rounding gets the first two wrong
    naive = (a2.astype(np.float64) * b2.astype(np.float64) + c2.astype(np.float64)).astype(np.float32)
    assert naive.tolist()[:2] == [1.0, 1.0 + 2.0**-22]


@pytest.mark.parametrize("seed", [7, 8])
def test_group_score_of_one_head_is_the_head_score(seed):
    rng = np.random.default_rng(seed)
    P = 300
    kbits = _bits(rng.standard_normal((16 * P, 1, 128)) * np.where(rng.random(128) < 0.05, 8, 1))
    kmin, kmax = quantize.page_bounds(kbits)
    qb = _bits(rng.standard_normal((1, 128)) * 2.0 ** rng.integers(-3, 3, 128))
    qb[0, :5] = _bits(np.array([0.0, -0.0, 0.0, -0.0, 0.0]))
    gs = select.group_scores(qb, kmin[:, 0], kmax[:, 0])
    hs = select.page_scores_head(qb[0], kmin[:, 0], kmax[:, 0])
    assert np.array_equal(gs.view(np.uint32), hs.view(np.uint32))


@pytest.mark.parametrize("G", [2, 4, 8])
def test_group_score_is_the_sum_of_the_head_bounds(G):
    # the per-channel form computes sum_h sigma_h: compare with the exact rational sum of the per-head
    # bounds; the float32 error is at most (G + 256) * 2^-24 * sum_c (|P_c kmax_c| + |N_c kmin_c|),
    # far below what a dropped term, a swapped bound or a wrong sign would change
    rng = np.random.default_rng(40 + G)
    P = 40
    kbits = _bits(rng.standard_normal((16 * P, 1, 128)) * np.where(rng.random(128) < 0.05, 8, 1))
    kmin, kmax = quantize.page_bounds(kbits)
    kmin, kmax = kmin[:, 0], kmax[:, 0]
    qb = _bits(rng.standard_normal((G, 128)))
    gs = select.group_scores(qb, kmin, kmax)
    qf = numerics.bf16_to_f32(qb)
    Pc, Nc = select.group_query_parts(qb)
    for j in range(P):
        exact = sum(max(Fraction(float(qf[h, c])) * Fraction(float(kmin[j, c])),
                        Fraction(float(qf[h, c])) * Fraction(float(kmax[j, c]))) for h in range(G) for c in range(128))
        mag = float(np.sum(np.abs(Pc.astype(np.float64) * kmax[j]) + np.abs(Nc.astype(np.float64) * kmin[j])))
        assert abs(float(Fraction(float(gs[j])) - exact)) <= (G + 256) * 2.0**-24 * mag + 1e-30
