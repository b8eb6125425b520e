"""CPU checks of the estimate kernel's declared precision (``tests/kernel_model.py``), which sets the
per-token band of the GPU top-p parity tests.

* The fixed-point query meets its guarantees: |Q| <= 2088960, the three digits are int8 and rebuild
  Q, channels within 2^12 of their group's largest magnitude are held exactly, every channel within
  half a grid step, and the group exponent brackets the largest magnitude (computed here with log2).
* The declared arithmetic lands within the stated bound of the float64 definition on ordinary and
  extreme queries, at every code width.
* The bound is narrow: a dropped zero-point term or one group off by a factor of two would fall far
  outside it, so the band cannot excuse a real error of that kind.
"""

import math

import numpy as np
import pytest

from oracle import estimate, numerics, quantize
from tests import kernel_model as km

SM = float(np.float32(1 / math.sqrt(128)))


def _qvec(rng, scales):
    """A bf16 query whose four groups have the given magnitudes (0 gives an all-zero group)."""
    q = np.concatenate([rng.standard_normal(32) * sc for sc in scales]).astype(np.float32)
    return numerics.f32_to_bf16_bits(q)


QCASES = [(0, 1, (1, 1, 1, 1)), (1, 8, (1, 1, 1, 1)), (2, 1, (3.5, 3.5, 3.5, 3.5)), (3, 0.02, (0.05,) * 4),
          (4, 1, (1e-3, 1, 100, 0)), (5, 3, (2.0**-90, 1e-30, 7, 0.25)), (6, 1, (2.0**-110, 1, 0.5, 2)),
          (7, 1, (1e-5, 1, 1, 1))]


@pytest.mark.parametrize("seed,kscale,qscales", QCASES)
def test_fixed_point_query_guarantees(seed, kscale, qscales):
    rng = np.random.default_rng(seed)
    qbits = _qvec(rng, qscales)
    q = numerics.bf16_to_f32(qbits).astype(np.float64)
    # make one channel tiny next to its group's largest: it must be rounded to the grid
    Q, E = km.fixed_query(qbits)
    assert np.abs(Q).max() <= km.Q_MAX
    d2, d1, d0 = km.digits(Q)
    assert d2.min() >= -128 and d2.max() <= 127 and d1.min() >= 0 and d1.max() <= 127
    assert d0.min() >= 0 and d0.max() <= 127
    assert np.array_equal((d2 << 14) + (d1 << 7) + d0, Q)
    for g in range(4):
        seg, Qg = q[32 * g:32 * g + 32], Q[32 * g:32 * g + 32]
        m = np.abs(seg).max()
        if m == 0:
            assert not Qg.any()
            continue
        if E[g] > -100:
            assert E[g] == int(np.floor(np.log2(m)))
        back = np.ldexp(Qg.astype(np.float64), int(E[g]) - 20)
        assert np.all(np.abs(back - seg) <= 2.0 ** (int(E[g]) - 21))
        big = np.abs(seg) >= 2.0 ** (int(E[g]) - 12)
        assert np.array_equal(back[big], seg[big])


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("seed,kscale,qscales", QCASES)
def test_declared_arithmetic_within_the_bound(seed, kscale, qscales, bits):
    rng = np.random.default_rng(seed)
    n = 3000
    kbits = numerics.f32_to_bf16_bits((rng.standard_normal((n, 128)) * kscale).astype(np.float32))
    qbits = _qvec(rng, qscales)
    qz = quantize.quantize_rows(kbits, bits)
    model = km.kernel_logits(qbits, qz["codes"], qz["scale"], qz["zero"], SM).astype(np.float64)
    ref = estimate.logits_f64(qbits, qz["codes"], qz["scale"], qz["zero"], SM)
    bound = km.logit_err_bound(qbits, qz["codes"], qz["scale"], qz["zero"], ref)
    assert np.all(np.abs(model - ref) <= bound)
    # the bound is narrow: a dropped zero-point term misses it for most candidates
    q = numerics.bf16_to_f32(qbits).astype(np.float64)
    z = qz["zero"].astype(np.float64)
    zterm = SM * (z * q.reshape(4, 32).sum(-1)).sum(-1)
    live = np.abs(zterm) > 4 * bound
    assert live.mean() > 0.5


def test_group_scale_error_would_be_caught():
    # one group's contribution off by a factor 2 misses the bound for nearly every candidate
    rng = np.random.default_rng(11)
    kbits = numerics.f32_to_bf16_bits(rng.standard_normal((1000, 128)).astype(np.float32))
    qbits = _qvec(rng, (1, 1, 1, 1))
    qz = quantize.quantize_rows(kbits)
    ref = estimate.logits_f64(qbits, qz["codes"], qz["scale"], qz["zero"], SM)
    xhat = quantize.dequantize(qz["codes"], qz["scale"], qz["zero"])
    q = numerics.bf16_to_f32(qbits).astype(np.float64)
    g1 = SM * (xhat[:, 32:64] @ q[32:64])
    bound = km.logit_err_bound(qbits, qz["codes"], qz["scale"], qz["zero"], ref)
    assert np.mean(np.abs(g1) > bound) > 0.9


def test_ordinary_queries_are_held_exactly():
    # N(0,1) bf16 queries: no channel is 2^12 below its group's largest, so only the final float32
    # rounding separates the declared arithmetic from the definition
    rng = np.random.default_rng(12)
    kbits = numerics.f32_to_bf16_bits(rng.standard_normal((2000, 128)).astype(np.float32))
    qz = quantize.quantize_rows(kbits)
    for _ in range(20):
        qbits = numerics.f32_to_bf16_bits(rng.standard_normal(128).astype(np.float32))
        Q, E = km.fixed_query(qbits)
        q = numerics.bf16_to_f32(qbits).astype(np.float64)
        if np.array_equal(np.ldexp(Q.astype(np.float64), np.repeat(E - 20, 32)), q):
            model = km.kernel_logits(qbits, qz["codes"], qz["scale"], qz["zero"], SM)
            ref = estimate.logits_f64(qbits, qz["codes"], qz["scale"], qz["zero"], SM)
            assert np.array_equal(model, ref.astype(np.float32))


def test_band_hook_shape():
    rng = np.random.default_rng(1)
    kbits = numerics.f32_to_bf16_bits(rng.standard_normal((100, 128)).astype(np.float32))
    qbits = numerics.f32_to_bf16_bits(rng.standard_normal(128).astype(np.float32))
    qz = quantize.quantize_rows(kbits)
    ref = estimate.logits_f64(qbits, qz["codes"], qz["scale"], qz["zero"], SM)
    err, extra = km.band(qbits, qz["codes"], qz["scale"], qz["zero"], ref)
    assert err.shape == (100,) and np.all(err > 0) and np.all(err < 1e-5)
    assert extra == 100 * 2.0**-40
