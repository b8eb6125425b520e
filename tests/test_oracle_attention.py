"""Pins for O8 (union), O9 (sparse attention) and O10 (dense attention, top-p error bound).

* O9 with every index equals torch's scaled-dot-product attention (a library routine) in float64.
* One index returns that token's value row exactly; identical keys give the mean of the values.
* Permutation of the index set leaves the output unchanged.
* The bound of the pages, (1-p)||V||_F, in its three forms (theorems, so they must hold) on random
  heads and on the peaked single-head workload.
"""

import math

import numpy as np
import pytest
import torch

from gen import make_config
from oracle import attention, numerics

SM = float(np.float32(1 / math.sqrt(128)))


def _rand(seed, n, scale=1.0):
    rng = np.random.default_rng(seed)
    k = numerics.f32_to_bf16_bits((rng.standard_normal((n, 128)) * scale).astype(np.float32))
    v = numerics.f32_to_bf16_bits(rng.standard_normal((n, 128)).astype(np.float32))
    q = numerics.f32_to_bf16_bits(rng.standard_normal(128).astype(np.float32))
    return q, k, v


def test_all_indices_equals_library_attention():
    q, k, v = _rand(0, 777, 2.0)
    o, lse = attention.sparse_attention(q, k, v, np.arange(777), SM)
    tq = torch.from_numpy(numerics.bf16_to_f32(q).astype(np.float64)).view(1, 1, 1, 128)
    tk = torch.from_numpy(numerics.bf16_to_f32(k).astype(np.float64)).view(1, 1, 777, 128)
    tv = torch.from_numpy(numerics.bf16_to_f32(v).astype(np.float64)).view(1, 1, 777, 128)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=SM).view(128).numpy()
    assert np.allclose(o, ref, rtol=0, atol=1e-12)
    s = SM * (numerics.bf16_to_f32(k).astype(np.float64) @ numerics.bf16_to_f32(q).astype(np.float64))
    assert math.isclose(lse, float(torch.logsumexp(torch.from_numpy(s), 0)), rel_tol=1e-13)


def test_single_index_and_identical_keys():
    q, k, v = _rand(1, 50)
    o, _ = attention.sparse_attention(q, k, v, np.array([23]), SM)
    assert np.array_equal(o, numerics.bf16_to_f32(v[23]).astype(np.float64))
    k[:] = k[0]
    o, lse = attention.sparse_attention(q, k, v, np.arange(10, 30), SM)
    assert np.allclose(o, numerics.bf16_to_f32(v[10:30]).astype(np.float64).mean(0), atol=1e-14)
    o, lse = attention.sparse_attention(q, k, v, np.zeros(0, np.int64), SM)
    assert np.all(o == 0) and lse == -math.inf


def test_permutation_invariance():
    q, k, v = _rand(2, 300)
    idx = np.random.default_rng(2).choice(300, 120, replace=False)
    o1, l1 = attention.sparse_attention(q, k, v, idx, SM)
    o2, l2 = attention.sparse_attention(q, k, v, idx[::-1].copy(), SM)
    assert np.allclose(o1, o2, atol=1e-13) and math.isclose(l1, l2, rel_tol=1e-13)


def test_union():
    assert attention.union([np.array([5, 1]), np.array([3, 5]), np.array([], np.int64)]).tolist() == [1, 3, 5]


@pytest.mark.parametrize("seed,scale,p", [(3, 1.0, 0.9), (4, 3.0, 0.85), (5, 0.3, 0.7), (6, 6.0, 0.95)])
def test_topp_error_bound_random(seed, scale, p):
    q, k, v = _rand(seed, 2000, scale)
    r = attention.topp_bound_check(q, k, v, p, SM)
    assert r["s"] >= p
    assert r["err_masked"] <= r["bound_a"] * (1 + 1e-12)
    assert r["err_renorm"] <= r["bound_b"] * (1 + 1e-12)
    assert r["stable_rank"] >= 2
    assert r["err_renorm"] <= r["bound_c"] * (1 + 1e-12)


def test_topp_error_bound_peaked_single_head_workload():
    w = make_config("C1")
    k = w.logical("k", 0)[:, 0, :]
    v = w.logical("v", 0)[:, 0, :]
    r = attention.topp_bound_check(w.q[0, 0], k, v, w.p, SM)
    assert r["err_masked"] <= r["bound_a"] and r["err_renorm"] <= r["bound_c"]
