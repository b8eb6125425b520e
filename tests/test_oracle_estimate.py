"""Pins for O5 (INT4 logit estimate) and O6 (softmax weights).

* The fixed-point query meets its definition's guarantees: |Q| <= 16320, channels within 2^6 of their
  group's largest magnitude are held exactly, every channel within half a grid step, and the group
  exponent brackets the largest magnitude (computed here with log2, independently of the oracle).
* The committed arithmetic (``logits_spec``) agrees with the float64 definition (``logits_f64``)
  within the error bound that the query rounding and the float32 operation count imply (derived
  below); a dropped or mis-signed term, or a group scale off by a power of two, misses that bound.
* Special case: a query on the fixed-point grid and keys already on the INT4 grid make the estimate
  the exact bf16 attention logit up to the final float32 roundings alone.
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


def _group_exponents(q):
    """floor(log2 max |q|) per 32-channel group, clamped to >= -100 (0 for an all-zero group)."""
    m = np.abs(np.asarray(q, np.float64)).reshape(4, 32).max(-1)
    return np.array([max(int(np.floor(np.log2(x))), -100) if x > 0 else 0 for x in m])


def _bound(qbits, codes, s16, z16, xhat, logits, bits=4):
    """|spec - f64| <= sm * (sum_c 2^(E_g - 14) |x^_c| (1 + u) + k u sum_g (|s_g a_g| + |z_g b_g|)
                             + u sum_c |q_c| |x^_c|) + 2u |l|,  k = 5 (6 for 8-bit codes).

    Derivation: spec in exact arithmetic is sm * sum_c q~_c x_c with |q_c - q~_c| <= 2^(E_g - 14)
    (half a grid step) and x_c = code_c s_g + z_g, whose float32 rounding x^_c is what the float64
    reference uses (<= u |x^_c|).  a_g and b_g are exact; t_g rounds two products and their sum
    (<= 2u (|s_g a_g| + |z_g b_g|)); r adds two levels of rounded sums (<= 2u of the same terms);
    l rounds once more (<= u |l|, doubled for the reference's own rounding).  5u covers 4u plus the
    second-order terms; 8-bit group sums also round once to float32 (<= u |a_g|), one u more.
    """
    q = numerics.bf16_to_f32(qbits).astype(np.float64)
    E = _group_exponents(q)
    step = np.repeat(2.0 ** (E - 14), 32)  # half a grid step per channel
    qa = np.abs(q).reshape(1, 4, 32)
    c = codes.astype(np.float64).reshape(-1, 4, 32)
    s = np.abs(s16.astype(np.float64))
    z = np.abs(z16.astype(np.float64))
    terms = (s * (qa * c).sum(-1) + z * qa.sum(-1)).sum(-1) * (1 + 2.0**-13)
    xa = np.abs(xhat.astype(np.float64))
    quant = (xa * step.reshape(1, 128)).sum(-1) * (1 + U)
    xq = (xa * np.abs(q).reshape(1, 128)).sum(-1)
    k = 6 if bits == 8 else 5
    return SM * (quant + k * U * terms + U * xq) + 2 * U * np.abs(logits)


def _qvec(rng, scales):
    """A bf16 query whose four groups have the given magnitudes (0 gives an all-zero group)."""
    q = np.concatenate([rng.standard_normal(32) * sc for sc in scales]).astype(np.float32)
    return numerics.f32_to_bf16_bits(q)


QCASES = [(0, 1, (1, 1, 1, 1)), (1, 8, (1, 1, 1, 1)), (2, 1, (3.5, 3.5, 3.5, 3.5)), (3, 0.02, (0.05,) * 4),
          (4, 1, (1e-3, 1, 100, 0)), (5, 3, (2.0**-90, 1e-30, 7, 0.25)), (6, 1, (2.0**-110, 1, 0.5, 2))]


@pytest.mark.parametrize("seed,kscale,qscales", QCASES)
def test_fixed_point_query_guarantees(seed, kscale, qscales):
    rng = np.random.default_rng(seed)
    q = numerics.bf16_to_f32(_qvec(rng, qscales)).astype(np.float64)
    Q, E = estimate.q_fixed(q)
    assert E.tolist() == _group_exponents(q).tolist()
    assert np.abs(Q).max() <= 16320
    for g in range(4):
        seg, Qg = q[32 * g:32 * g + 32], Q[32 * g:32 * g + 32]
        m = np.abs(seg).max()
        if m == 0:
            assert not Qg.any()
            continue
        if E[g] > -100:
            assert 2.0 ** E[g] <= m < 2.0 ** (E[g] + 1)
        back = np.ldexp(Qg.astype(np.float64), int(E[g]) - 13)
        assert np.all(np.abs(back - seg) <= 2.0 ** (int(E[g]) - 14))
        big = np.abs(seg) >= 2.0 ** (int(E[g]) - 6)
        assert np.array_equal(back[big], seg[big])


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("seed,kscale,qscales", QCASES)
def test_spec_matches_float64_definition(seed, kscale, qscales, bits):
    rng = np.random.default_rng(seed)
    n = 3000
    kbits = numerics.f32_to_bf16_bits((rng.standard_normal((n, 128)) * kscale).astype(np.float32))
    qbits = _qvec(rng, qscales)
    qz = quantize.quantize_rows(kbits, bits)
    spec = estimate.logits_spec(qbits, qz["codes"], qz["scale"], qz["zero"], SM).astype(np.float64)
    ref = estimate.logits_f64(qbits, qz["codes"], qz["scale"], qz["zero"], SM)
    xhat = quantize.dequantize(qz["codes"], qz["scale"], qz["zero"])
    bound = _bound(qbits, qz["codes"], qz["scale"], qz["zero"], xhat, ref, bits)
    assert np.all(np.abs(spec - ref) <= bound)
    # the bound is tight enough to catch a dropped zero-point term
    q = numerics.bf16_to_f32(qbits).astype(np.float64)
    z = qz["zero"].astype(np.float64)
    zterm = SM * (z * q.reshape(4, 32).sum(-1)).sum(-1)
    live = np.abs(zterm) > 4 * bound
    assert live.mean() > 0.5 and np.all(np.abs((ref - zterm) - ref)[live] > bound[live])


def test_scale_exponent_error_would_be_caught():
    # the same logits with one group's contribution off by a factor 2 miss the bound
    rng = np.random.default_rng(11)
    n = 1000
    kbits = numerics.f32_to_bf16_bits(rng.standard_normal((n, 128)).astype(np.float32))
    qbits = _qvec(rng, (1, 1, 1, 1))
    qz = quantize.quantize_rows(kbits)
    ref = estimate.logits_f64(qbits, qz["codes"], qz["scale"], qz["zero"], SM)
    xhat = quantize.dequantize(qz["codes"], qz["scale"], qz["zero"]).astype(np.float64)
    q = numerics.bf16_to_f32(qbits).astype(np.float64)
    g1 = SM * (xhat[:, 32:64] @ q[32:64])
    bound = _bound(qbits, qz["codes"], qz["scale"], qz["zero"], xhat, ref)
    assert np.mean(np.abs(g1) > bound) > 0.9


def test_grid_query_and_grid_keys_give_exact_bf16_logits():
    rng = np.random.default_rng(7)
    n = 2048
    codes = rng.integers(0, 16, size=(n, 4, 32))
    codes[:, :, 0], codes[:, :, 1] = 0, 15
    s16 = (2.0 ** rng.integers(-5, 0, size=(n, 4))).astype(np.float16)
    z16 = (rng.integers(-32, 32, size=(n, 4)) * s16.astype(np.float64)).astype(np.float16)
    x = codes * s16.astype(np.float64)[..., None] + z16.astype(np.float64)[..., None]
    kbits = numerics.f32_to_bf16_bits(x.reshape(n, 128).astype(np.float32))
    # every channel within 2^6 of its group's largest magnitude: held exactly in fixed point
    scale = (2.0 ** np.array([-2, 0, 1, 2])).repeat(32)
    q = rng.choice([-1, 1], 128) * rng.uniform(0.02, 0.99, 128) * scale
    q[::32] = 0.999 * scale[::32]  # each group's largest magnitude, pinning its exponent
    qbits = numerics.f32_to_bf16_bits(q.astype(np.float32))
    qz = quantize.quantize_rows(kbits)
    spec = estimate.logits_spec(qbits, qz["codes"], qz["scale"], qz["zero"], SM).astype(np.float64)
    exact = SM * (numerics.bf16_to_f32(kbits).astype(np.float64) @ numerics.bf16_to_f32(qbits).astype(np.float64))
    qq = numerics.bf16_to_f32(qbits).astype(np.float64)
    Q, E = estimate.q_fixed(qq)
    assert np.array_equal(np.ldexp(Q.astype(np.float64), np.repeat(E - 13, 32)), qq)
    xa = np.abs(x.reshape(n, 128))
    terms = (xa * np.abs(qq)).sum(-1)
    # only t_g, r and l round: <= sm * 5u * sum|q x| + 2u |l|
    assert np.all(np.abs(spec - exact) <= SM * 5 * U * terms + 2 * U * np.abs(exact))


def test_eight_bit_group_sums_round_once():
    # the largest 8-bit group sum (all codes 255 against Q = 16320) exceeds 2^24, so the spec rounds
    # it once to float32: compare with the integer sum rounded by hand (nearest even multiple of 8)
    codes = np.full((1, 128), 255, np.uint8)
    q = np.full(128, 0.99, np.float32)
    qbits = numerics.f32_to_bf16_bits(q)
    Q, E = estimate.q_fixed(numerics.bf16_to_f32(qbits))
    S = int(Q[:32].sum()) * 255
    assert S > 2**24
    step = 1 << (S.bit_length() - 24)
    lo = S - S % step
    rnd = lo + step if (S - lo > step // 2 or (S - lo == step // 2 and (lo // step) % 2 == 1)) else lo
    s16 = np.ones((1, 4), np.float16)
    z16 = np.zeros((1, 4), np.float16)
    l = estimate.logits_spec(qbits, codes, s16, z16, 1.0)
    a = np.float32(np.ldexp(float(rnd), int(E[0]) - 13))
    t = a  # s = 1, z = 0: each t_g is a_g, the same in every group
    assert l[0] == np.float32(np.float32(t + t) + np.float32(t + t))


def test_softmax_properties():
    rng = np.random.default_rng(3)
    l = rng.standard_normal(1000) * 4
    W = estimate.softmax_f64(l)
    assert np.all(W >= 0) and abs(W.sum() - 1) < 1e-12
    assert np.allclose(W, estimate.softmax_f64(l + 123.25), rtol=1e-12, atol=0)
    assert np.allclose(W, scipy.special.softmax(l), rtol=1e-12, atol=1e-300)
    assert estimate.softmax_f64(np.zeros(0)).size == 0
