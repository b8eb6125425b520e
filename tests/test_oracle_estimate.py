"""Pins for O5 (INT4 logit estimate) and O6 (softmax weights).

* Keys already on the quantisation grid are reconstructed exactly, so the estimate must equal the
  textbook bf16 attention logit sm * q . k (float64) -- for every code width.  A dropped zero-point
  term, a scale applied to the wrong group or a transposed operand fails this.
* The estimate is linear in the query: exact for a power-of-two multiple of q, and additive over a
  split of q's channels into its four groups.
* A brute-force loop over channels (pure Python, fsum) agrees on a small case.
* Softmax: non-negative, sums to one, invariant under a common shift of the logits, and equal to
  scipy's softmax.
"""

import math

import numpy as np
import pytest
import scipy.special

from oracle import estimate, numerics, quantize

SM = float(np.float32(1 / math.sqrt(128)))


def _grid_keys(rng, n, bits):
    """bf16 keys whose every group sits on its own min/max grid (codes 0 and L both present)."""
    L = (1 << bits) - 1
    codes = rng.integers(0, L + 1, size=(n, 4, 32))
    codes[:, :, 0], codes[:, :, 1] = 0, L
    # power-of-two scales and zero = m * scale keep (code + m) * scale an integer of magnitude <= 255
    # times a power of two: within bf16's 8 significant bits
    s16 = (2.0 ** rng.integers(-5, 0, size=(n, 4))).astype(np.float16)
    m = rng.integers(-L, 256 - L, size=(n, 4))
    z16 = (m * s16.astype(np.float64)).astype(np.float16)
    x = codes * s16.astype(np.float64)[..., None] + z16.astype(np.float64)[..., None]
    kbits = numerics.f32_to_bf16_bits(x.reshape(n, 128).astype(np.float32))
    assert np.array_equal(numerics.bf16_to_f32(kbits).astype(np.float64), x.reshape(n, 128))
    return kbits


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_grid_keys_give_the_exact_bf16_logits(bits):
    rng = np.random.default_rng(7 + bits)
    kbits = _grid_keys(rng, 1500, bits)
    qbits = numerics.f32_to_bf16_bits((rng.standard_normal(128) * 2).astype(np.float32))
    qz = quantize.quantize_rows(kbits, bits)
    lg = estimate.logits_f64(qbits, qz["codes"], qz["scale"], qz["zero"], SM)
    exact = SM * (numerics.bf16_to_f32(kbits).astype(np.float64) @ numerics.bf16_to_f32(qbits).astype(np.float64))
    assert np.allclose(lg, exact, rtol=1e-14, atol=1e-14)


def test_linear_in_the_query():
    rng = np.random.default_rng(3)
    kbits = numerics.f32_to_bf16_bits(rng.standard_normal((800, 128)).astype(np.float32))
    q = rng.standard_normal(128).astype(np.float32)
    qz = quantize.quantize_rows(kbits)
    l1 = estimate.logits_f64(numerics.f32_to_bf16_bits(q), qz["codes"], qz["scale"], qz["zero"], SM)
    qb = numerics.bf16_to_f32(numerics.f32_to_bf16_bits(q))
    l4 = estimate.logits_f64(numerics.f32_to_bf16_bits(4 * qb), qz["codes"], qz["scale"], qz["zero"], SM)
    assert np.array_equal(l4, 4 * l1)
    parts = np.zeros_like(l1)
    for g in range(4):
        qg = np.zeros(128, np.float32)
        qg[32 * g:32 * g + 32] = qb[32 * g:32 * g + 32]
        parts += estimate.logits_f64(numerics.f32_to_bf16_bits(qg), qz["codes"], qz["scale"], qz["zero"], SM)
    assert np.allclose(parts, l1, rtol=1e-13, atol=1e-13)


def test_brute_force_loop():
    rng = np.random.default_rng(5)
    kbits = numerics.f32_to_bf16_bits((rng.standard_normal((40, 128)) * 3).astype(np.float32))
    qbits = numerics.f32_to_bf16_bits(rng.standard_normal(128).astype(np.float32))
    qz = quantize.quantize_rows(kbits)
    lg = estimate.logits_f64(qbits, qz["codes"], qz["scale"], qz["zero"], SM)
    q = [float(x) for x in numerics.bf16_to_f32(qbits)]
    for i in range(40):
        terms = []
        for c in range(128):
            g = c // 32
            xh = int(qz["codes"][i, c]) * float(qz["scale"][i, g]) + float(qz["zero"][i, g])
            terms.append(q[c] * xh)
        assert math.isclose(lg[i], SM * math.fsum(terms), rel_tol=1e-13, abs_tol=1e-13)


def test_softmax_properties():
    rng = np.random.default_rng(3)
    l = rng.standard_normal(1000) * 4
    W = estimate.softmax_f64(l)
    assert np.all(W >= 0) and abs(W.sum() - 1) < 1e-12
    assert np.allclose(W, estimate.softmax_f64(l + 123.25), rtol=1e-12, atol=0)
    assert np.allclose(W, scipy.special.softmax(l), rtol=1e-12, atol=1e-300)
    assert estimate.softmax_f64(np.zeros(0)).size == 0
