"""Pins for O5 (INT4 logit estimate) and O6 (softmax weights).

* The committed float32 order (``logits_spec``) agrees with the float64 definition (``logits_f64``)
  within the error bound that the float32 operation count implies (derived below); a dropped or
  mis-signed term in the factorised form misses that bound by orders of magnitude.
* Special case: keys already on the INT4 grid dequantise to themselves, so the estimate equals the
  exact bf16 attention logits (float64 dot product) within the same bound.
* Softmax: non-negative, sums to one, invariant under a common shift of the logits, and equal to
  scipy's softmax.
"""

import math

import numpy as np
import pytest
import scipy.special

from oracle import estimate, numerics, quantize

U = 2.0**-24
SM = float(np.float32(1 / math.sqrt(128)))


def _bound(qbits, codes, s16, z16, xhat, logits):
    """|spec - f64| <= sm * (34u * sum_g (|s_g| sum|q c| + |z_g| sum|q|) + u sum|q||x^|) + 2u|l|.

    Derivation: each group sum a_g, b_g is a 32-term float32 fold (error <= 31u * sum of |terms|);
    t_g adds two rounded products and a rounded sum (<= 2u relative each); r adds two levels of
    rounded sums; l rounds once more; the float64 reference itself uses x^ rounded to fp32 once per
    element (<= u |x^|).  34u covers 31u + the three further roundings of each group's terms.
    """
    q = np.abs(numerics.bf16_to_f32(qbits).astype(np.float64)).reshape(1, 4, 32)
    c = codes.astype(np.float64).reshape(-1, 4, 32)
    s = np.abs(s16.astype(np.float64))
    z = np.abs(z16.astype(np.float64))
    terms = (s * (q * c).sum(-1) + z * q.sum(-1)).sum(-1)
    xq = (np.abs(xhat.astype(np.float64)) * q.reshape(1, 128)).sum(-1)
    return SM * (34 * U * terms + U * xq) + 2 * U * np.abs(logits)


@pytest.mark.parametrize("seed,kscale,qscale", [(0, 1, 1), (1, 8, 1), (2, 1, 3.5), (3, 0.02, 0.05)])
def test_spec_order_matches_float64_definition(seed, kscale, qscale):
    rng = np.random.default_rng(seed)
    n = 3000
    kbits = numerics.f32_to_bf16_bits((rng.standard_normal((n, 128)) * kscale).astype(np.float32))
    qbits = numerics.f32_to_bf16_bits((rng.standard_normal(128) * qscale).astype(np.float32))
    qz = quantize.quantize_rows(kbits)
    spec = estimate.logits_spec(qbits, qz["codes"], qz["scale"], qz["zero"], SM).astype(np.float64)
    ref = estimate.logits_f64(qbits, qz["codes"], qz["scale"], qz["zero"], SM)
    xhat = quantize.dequantize(qz["codes"], qz["scale"], qz["zero"])
    bound = _bound(qbits, qz["codes"], qz["scale"], qz["zero"], xhat, ref)
    assert np.all(np.abs(spec - ref) <= bound)
    # the bound is tight enough to catch a dropped zero-point term
    q = numerics.bf16_to_f32(qbits).astype(np.float64)
    z = qz["zero"].astype(np.float64)
    dropped = ref - SM * (z * q.reshape(4, 32).sum(-1)).sum(-1)
    assert np.mean(np.abs(dropped - ref) > bound) > 0.9


def test_keys_on_grid_give_exact_bf16_logits():
    rng = np.random.default_rng(7)
    n = 2048
    codes = rng.integers(0, 16, size=(n, 4, 32))
    codes[:, :, 0], codes[:, :, 1] = 0, 15
    s16 = (2.0 ** rng.integers(-5, 0, size=(n, 4))).astype(np.float16)
    z16 = (rng.integers(-32, 32, size=(n, 4)) * s16.astype(np.float64)).astype(np.float16)
    x = codes * s16.astype(np.float64)[..., None] + z16.astype(np.float64)[..., None]
    kbits = numerics.f32_to_bf16_bits(x.reshape(n, 128).astype(np.float32))
    qbits = numerics.f32_to_bf16_bits(rng.standard_normal(128).astype(np.float32))
    qz = quantize.quantize_rows(kbits)
    spec = estimate.logits_spec(qbits, qz["codes"], qz["scale"], qz["zero"], SM).astype(np.float64)
    exact = SM * (numerics.bf16_to_f32(kbits).astype(np.float64) @ numerics.bf16_to_f32(qbits).astype(np.float64))
    bound = _bound(qbits, qz["codes"], qz["scale"], qz["zero"], x.reshape(n, 128), exact)
    assert np.all(np.abs(spec - exact) <= bound)


def test_group_sums_are_the_channel_sums():
    q = np.arange(128, dtype=np.float32) * np.float32(0.5)
    assert estimate.group_qsums(q).tolist() == [0.5 * sum(range(g * 32, g * 32 + 32)) for g in range(4)]


def test_softmax_properties():
    rng = np.random.default_rng(3)
    l = rng.standard_normal(1000) * 4
    W = estimate.softmax_f64(l)
    assert np.all(W >= 0) and abs(W.sum() - 1) < 1e-12
    assert np.allclose(W, estimate.softmax_f64(l + 123.25), rtol=1e-12, atol=0)
    assert np.allclose(W, scipy.special.softmax(l), rtol=1e-12, atol=1e-300)
    assert estimate.softmax_f64(np.zeros(0)).size == 0
