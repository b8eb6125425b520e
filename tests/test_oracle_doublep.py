"""Pins for O11 (Double-P cluster-level top-p).

* Singleton clusters whose centroid is the key itself: cluster weights are the token softmax of the
  exact bf16 logits, so the kept clusters are the token-level top-p set of float64 dense weights
  (up to the ambiguity rule).
* Zero within-cluster spread: every member equals its centroid, so the size-weighted centroid
  weight is exactly the cluster's true softmax mass.
* The cluster logit's float32 fold agrees with the float64 dot product within its error bound.
* Ranges are (begin, length) of the kept clusters in ascending order; empty clusters never appear.
"""

import math

import numpy as np

from gen import make_custom
from oracle import attention, doublep, numerics, topp

SM = float(np.float32(1 / math.sqrt(128)))


def test_singleton_clusters_reduce_to_token_topp():
    rng = np.random.default_rng(0)
    n = 600
    k = numerics.f32_to_bf16_bits((rng.standard_normal((n, 128)) * 2).astype(np.float32))
    q = numerics.f32_to_bf16_bits(rng.standard_normal((1, 128)).astype(np.float32))
    cs = doublep.select_clusters(q, k, np.ones(n, np.int32), 0.9, SM)
    W = attention.dense_weights(q[0], k, SM)
    r = topp.topp_sort(W, 0.9)
    ok, msg = topp.set_matches(cs["kept"], r, W, 0.9)
    assert ok, msg


def test_zero_spread_weight_is_true_cluster_mass():
    rng = np.random.default_rng(1)
    C = 20
    sizes = rng.integers(0, 30, size=C)
    sizes[3] = 0
    mu = numerics.f32_to_bf16_bits(rng.standard_normal((C, 128)).astype(np.float32))
    keys = np.repeat(mu, sizes, axis=0)
    q = numerics.f32_to_bf16_bits(rng.standard_normal(128).astype(np.float32))
    W = attention.dense_weights(q, keys, SM)
    labels = np.repeat(np.arange(C), sizes)
    true_mass = np.bincount(labels, weights=W, minlength=C)
    lam = doublep.cluster_logits_spec(q, mu, SM)
    u = doublep.cluster_weights(lam, sizes)
    assert u[3] == 0
    assert np.allclose(u, true_mass, rtol=2e-6, atol=1e-300)


def test_cluster_logit_fold_error_bound():
    rng = np.random.default_rng(2)
    mu = numerics.f32_to_bf16_bits(rng.standard_normal((500, 128)).astype(np.float32))
    q = numerics.f32_to_bf16_bits(rng.standard_normal(128).astype(np.float32))
    lam = doublep.cluster_logits_spec(q, mu, SM).astype(np.float64)
    m = numerics.bf16_to_f32(mu).astype(np.float64)
    qf = numerics.bf16_to_f32(q).astype(np.float64)
    exact = SM * (m @ qf)
    bound = SM * 128 * 2.0**-24 * (np.abs(m) @ np.abs(qf)) + 2.0**-24 * np.abs(exact)
    assert np.all(np.abs(lam - exact) <= bound)


def test_workload_clusters_and_ranges():
    w = make_custom(batch=1, num_q_heads=4, num_kv_heads=2, seq_lens=[3000], kind="cluster",
                    num_clusters=64, p=0.9, p1=0.95, seed=5)
    assert np.array_equal(w.coff[..., -1], np.full((1, 2), 3000))
    for h in range(2):
        cs = doublep.select_clusters(w.q[0, 2 * h:2 * h + 2], w.centroids[0, h], w.csize[0, h], 0.95, SM)
        rg = doublep.ranges_of(cs["kept"], w.coff[0, h])
        assert np.all(rg[:, 1] > 0) and np.all(np.diff(rg[:, 0]) > 0)
        # each kept range is exactly its cluster's member tokens
        for (b0, ln), c in zip(rg, cs["kept"]):
            assert b0 == w.coff[0, h, c] and ln == w.csize[0, h, c]


# ---- optional approximation of the unkept clusters ---------------------------------------------------
def test_value_means_by_hand():
    v = numerics.f32_to_bf16_bits(np.array([[1.0] * 128, [3.0] * 128, [2.0] * 128, [-4.0] * 128], np.float32))
    m = doublep.value_means(v, np.array([2, 0, 2]), np.array([0, 2, 2]))
    assert np.array_equal(m[0], np.full(128, 2.0)) and not m[1].any() and np.array_equal(m[2], np.full(128, -1.0))


def test_collapsed_clusters_make_the_approximation_exact():
    # every member of a cluster has key mu_c and value v_c: attention over the kept clusters' tokens,
    # combined with the unkept clusters' n_c exp(lambda_c) (v_c), is dense attention over every token
    rng = np.random.default_rng(7)
    C = 30
    sizes = rng.integers(1, 20, size=C)
    sizes[4] = 0
    mu = numerics.f32_to_bf16_bits(rng.standard_normal((C, 128)).astype(np.float32))
    vc = numerics.f32_to_bf16_bits(rng.standard_normal((C, 128)).astype(np.float32))
    keys, vals = np.repeat(mu, sizes, axis=0), np.repeat(vc, sizes, axis=0)
    coff = np.concatenate([[0], np.cumsum(sizes)])
    q = numerics.f32_to_bf16_bits(rng.standard_normal(128).astype(np.float32))
    kept = np.array([1, 2, 7, 11, 20])
    idx = np.concatenate([np.arange(coff[c], coff[c + 1]) for c in kept])
    o, lse = attention.sparse_attention(q, keys, vals, idx, SM)
    lam = doublep.cluster_logits_spec(q, mu, SM)
    vm = doublep.value_means(vals, sizes, coff[:-1])
    oa, la = doublep.approx_unkept(o, lse, lam, sizes, kept, vm)
    od, ld = attention.sparse_attention(q, keys, vals, np.arange(len(keys)), SM)
    assert np.allclose(oa, od, rtol=0, atol=1e-5) and abs(la - ld) < 1e-5
    # nothing kept: the clusters alone give the same; everything kept: the input is returned
    oz, lz = doublep.approx_unkept(np.zeros(128), -math.inf, lam, sizes, np.zeros(0, np.int64), vm)
    assert np.allclose(oz, od, rtol=0, atol=1e-5) and abs(lz - ld) < 1e-5
    allc = np.nonzero(sizes)[0]
    o2, l2 = doublep.approx_unkept(o, lse, lam, sizes, allc, vm)
    assert np.array_equal(o2, o) and l2 == lse
