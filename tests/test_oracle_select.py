"""Pins for O3 (Quest-style page scores, top-K page selection) and O4 (candidate lists).

Pins: a hand-computed score (tests/golden/page_score_closed_form.json); the special case of
one-token pages, where the bound is the dot product itself and the selection is textbook top-k of
q.k (numpy argsort of float64 dot products); the upper-bound property against float64 dot products;
tie-breaking and the budget count; keep fraction 1 keeps every page.
"""

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
