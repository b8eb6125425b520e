"""Pins for O7 (minimal top-p set) and the model of its bisection search.

* Brute force over every subset for n <= 14: the oracle's set has the minimal size among all sets
  that reach p, and the largest mass among the minimal sets.
* Closed forms from tests/golden/topp_closed_form.json (geometric and uniform weights, explicit
  small vectors), one-hot weights, p = 1.
* Invariants: monotone in p, permutation invariant.
* The bisection on the uint32 image of the float32 threshold returns exactly the sort-based set (up
  to ties) once converged, a superset that still reaches p when stopped early, and after s steps the
  converged bit pattern with its low 31 - s bits cleared.
* Top-k is the k largest weights with ties at the k-th kept (rank characterisation by brute force).
* The band of an implementation's stated precision widens clause (i) by the two tokens' errors and
  the cut clause by twice their weighted mean.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import topp

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _brute(W, p):
    n = len(W)
    best_k, best_mass, best = None, -1.0, None
    for k in range(0, n + 1):
        for sub in itertools.combinations(range(n), k):
            m = math.fsum(W[list(sub)])
            if m >= p and (best_k is None or k < best_k or (k == best_k and m > best_mass)):
                best_k, best_mass, best = k, m, sub
        if best_k is not None:
            break
    return best_k, best_mass, best


@pytest.mark.parametrize("seed", range(12))
def test_brute_force_minimal_and_max_mass(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 15))
    W = rng.dirichlet(np.full(n, rng.choice([0.2, 1.0, 5.0])))
    p = float(rng.uniform(0.3, 0.99))
    r = topp.topp_sort(W, p)
    k, mass, _ = _brute(W, p)
    assert r["k"] == k
    assert math.isclose(r["mass"], mass, rel_tol=0, abs_tol=1e-15)
    assert math.fsum(W[r["sel"]]) >= p


def test_golden_closed_forms():
    g = json.load(open(os.path.join(GOLD, "topp_closed_form.json")))
    for c in g["geometric"]["cases"]:
        n = c["n"]
        W = 2.0 ** -np.arange(1, n + 1)
        W = W / W.sum()
        r = topp.topp_sort(W, c["p"])
        assert r["k"] == c["k"], c
        assert r["sel"].tolist() == list(range(c["k"]))
    for c in g["uniform"]["cases"]:
        W = np.full(c["n"], 1.0 / c["n"])
        assert topp.topp_sort(W, c["p"])["k"] == c["k"], c
    for c in g["explicit"]["cases"]:
        assert topp.topp_sort(np.array(c["W"]), c["p"])["sel"].tolist() == c["sel"], c


def test_one_hot_and_p_one():
    W = np.zeros(50)
    W[17] = 1.0
    assert topp.topp_sort(W, 0.9)["sel"].tolist() == [17]
    W = np.random.default_rng(0).dirichlet(np.ones(40))
    assert topp.topp_sort(W, 1.0)["sel"].tolist() == list(range(40))
    assert topp.topp_sort(np.zeros(0), 0.9)["k"] == 0


def test_monotone_in_p_and_permutation_invariant():
    rng = np.random.default_rng(4)
    W = rng.dirichlet(np.full(300, 0.3))
    prev = set()
    for p in np.linspace(0.05, 0.99, 25):
        cur = set(topp.topp_sort(W, p)["sel"].tolist())
        assert prev <= cur
        prev = cur
    perm = rng.permutation(300)
    a = topp.topp_sort(W, 0.85)["sel"]
    b = topp.topp_sort(W[perm], 0.85)["sel"]
    assert sorted(perm[b].tolist()) == a.tolist()


def test_ambiguity_sets_cover_ties_and_cut():
    W = np.array([0.4, 0.2, 0.2, 0.2])
    r = topp.topp_sort(W, 0.55)          # 0.4 then one of three equal 0.2
    assert r["sel"].tolist() == [0, 1]
    assert set(r["amb_i"].tolist()) == {1, 2, 3}
    ok, _ = topp.set_matches(np.array([0, 3]), r, W, 0.55)
    assert ok
    ok, _ = topp.set_matches(np.array([0]), r, W, 0.55)
    assert not ok
    W = np.array([0.5, 0.35, 0.15])
    r = topp.topp_sort(W, 0.85)          # prefix mass 0.85 sits exactly at p: clause (ii)
    assert 2 in r["amb_ii"].tolist()


@pytest.mark.parametrize("seed", range(8))
def test_bisection_equals_sort_based_set(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(1, 5000))
    logits = rng.standard_normal(n) * rng.choice([0.05, 1.0, 3.0, 12.0])
    w = np.exp(logits - logits.max()).astype(np.float32)        # float32 weights, max exactly 1
    if seed % 3 == 0:
        w[rng.integers(0, n, size=n // 4)] = w[0]                # many exact ties
    p = float(rng.uniform(0.5, 0.99))
    b = topp.topp_bisect(w, p, iters=32)
    assert b["converged"]
    W = w.astype(np.float64) / math.fsum(w.astype(np.float64))
    r = topp.topp_sort(W, p)
    # the search returns every token at or above the exact threshold weight w_(k*)
    thr = np.float32(w[r["order"][r["k"] - 1]])
    assert b["threshold"] == thr and b["key"] == int(np.float32(thr).view(np.uint32))
    ok, msg = topp.set_matches(b["sel"], r, W, p)
    assert ok, msg


def test_bisection_stopped_early_is_a_superset_reaching_p():
    rng = np.random.default_rng(9)
    w = np.exp(rng.standard_normal(4000) * 2).astype(np.float32)
    full = topp.topp_bisect(w, 0.9, iters=64)
    for it in (1, 4, 10, 20):
        b = topp.topp_bisect(w, 0.9, iters=it)
        assert set(full["sel"].tolist()) <= set(b["sel"].tolist())
        assert math.fsum(w[b["sel"]].astype(np.float64)) >= 0.9 * math.fsum(w.astype(np.float64))
    assert full["steps"] <= 31


def test_set_rule_on_empty_candidates():
    r = topp.topp_sort(np.zeros(0), 0.9)
    assert topp.set_matches(np.zeros(0, np.int64), r, np.zeros(0), 0.9)[0]
    assert not topp.set_matches(np.array([0]), r, np.zeros(0), 0.9)[0]


# ---- top-k baseline ------------------------------------------------------------------------------
def test_topk_by_hand_with_ties():
    W = np.array([0.1, 0.4, 0.4, 0.05, 0.05])
    assert topp.topk_sort(W, 2)["sel"].tolist() == [1, 2]
    assert topp.topk_sort(W, 1)["sel"].tolist() == [1, 2]          # the tie at the cut is kept
    assert topp.topk_sort(W, 3)["sel"].tolist() == [0, 1, 2]
    assert topp.topk_sort(W, 4)["sel"].tolist() == [0, 1, 2, 3, 4]
    assert topp.topk_sort(W, 0)["sel"].size == 0


@pytest.mark.parametrize("seed", range(6))
def test_topk_equals_rank_characterisation(seed):
    # brute force: i is kept iff fewer than k weights are strictly larger than W_i
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 60))
    W = rng.integers(1, 12, size=n).astype(np.float64)  # small integers: many ties
    W /= W.sum()
    for k in range(1, n + 1):
        want = [i for i in range(n) if sum(1 for j in range(n) if W[j] > W[i]) < k]
        assert topp.topk_sort(W, k)["sel"].tolist() == want, (seed, k)


def test_topk_is_the_k_largest_even_among_tiny_weights():
    W = np.array([1.0, 0.5, 2.0**-45, 2.0**-50])
    W = W / W.sum()
    assert topp.topk_sort(W, 2)["sel"].tolist() == [0, 1]
    assert topp.topk_sort(W, 3)["sel"].tolist() == [0, 1, 2]
    assert topp.topk_sort(W, 4)["sel"].tolist() == [0, 1, 2, 3]
    assert topp.topk_sort(W, 9)["sel"].tolist() == [0, 1, 2, 3]


# ---- the band of an implementation's stated precision ---------------------------------------------
def test_error_band_widens_only_clause_i_around_the_cut():
    W = np.array([0.5, 0.2, 0.2 * (1 - 3e-6), 0.1 - 0.2 * (1 - 3e-6) + 0.2])
    W = W / W.sum()
    p = W[0] + 0.5 * W[1]                   # the canonical set is {0, 1}, far from any prefix cut
    r0 = topp.topp_sort(W, p)
    assert r0["sel"].tolist() == [0, 1] and 2 not in r0["amb_i"].tolist()
    r1 = topp.topp_sort(W, p, err=np.full(4, 2e-6))   # 3e-6 apart < 1e-6 + 2e-6 + 2e-6
    assert 2 in r1["amb_i"].tolist() and 2 not in r1["amb_i_base"].tolist()
    ok, msg = topp.set_matches(np.array([0, 2]), r1, W, p)
    assert ok, msg
    c = topp.diff_counts(np.array([0, 2]), r1)
    assert (c["base"], c["band"], c["bad"]) == (1, 1, 0)   # token 1 is the threshold token itself
    assert not topp.set_matches(np.array([0, 2]), r0, W, p)[0]


def test_cut_clause_tolerance_follows_the_weighted_error():
    rng = np.random.default_rng(2)
    W = rng.dirichlet(np.ones(200))
    r = topp.topp_sort(W, 0.8, err=np.full(200, 1e-7), tau_p_extra=3e-9)
    assert math.isclose(r["tau_p"], topp.TAU_P + 2e-7 + 3e-9, rel_tol=1e-9)
    # an error carried only by tokens of no weight does not widen the cut
    e = np.where(W < np.sort(W)[5], 1.0, 0.0)
    r2 = topp.topp_sort(W, 0.8, err=e)
    assert r2["tau_p"] <= topp.TAU_P + 2 * 6 * W.max()


def test_bisection_stopped_early_keeps_the_top_bits_of_the_threshold():
    # one key bit per step from the top: after s steps the bit pattern is the converged one with its
    # low 31 - s bits cleared (no step decided within rounding here)
    rng = np.random.default_rng(21)
    for trial in range(6):
        W = np.exp(rng.standard_normal(3000) * rng.choice([0.3, 2.0, 6.0]))
        full = topp.topp_bisect(W, 0.9, iters=31)
        assert full["converged"]
        for s in (1, 3, 8, 13, 20, 30):
            b = topp.topp_bisect(W, 0.9, iters=s, tau=1e-6)
            if len(b["keys"]) == 1:
                assert b["key"] == full["key"] & ~((1 << (31 - s)) - 1), (trial, s)


def test_bisection_alternatives_when_a_step_is_within_tolerance():
    # weights chosen so that the mass of the first probe above the largest key bit equals the target
    W = np.array([1.0, 1.0, 1.0, 1.0])
    b = topp.topp_bisect(W, 0.5, iters=31, tau=0.0)
    assert b["sel"].tolist() == [0, 1, 2, 3]    # ties: all four weights equal the threshold
    b = topp.topp_bisect(W, 1.0, iters=31)
    assert b["sel"].tolist() == [0, 1, 2, 3]
    W = np.array([0.6, 0.4])
    b = topp.topp_bisect(W, 0.6, iters=31, tau=1e-3)
    assert len(b["keys"]) >= 1 and b["keys"][0] == b["key"]
