"""O5 estimated attention logits from the INT4 K cache; O6 softmax weights over the candidates.

The pages estimate attention weights with a mixed-precision SpGEMV of the query against the
dequantised 4-bit keys (paperlayer §4.2; §B.1, Fig. 12) and then need the weights' values, not only
their order (Paper-Notes "局限与展望": top-p needs approximate weights rather than a ranking).

Two versions of O5 are given:

* ``logits_f64`` -- the plain definition: l_i = sm * sum_c q_c * x^_ic in float64, with x^ the fp32
  dequantised key (see ``quantize.dequantize``).
* ``logits_spec`` -- the arithmetic the GPU kernel commits to.  A top-p *set* is decided from these
  logits, so both sides must hold the same values.  The pages fix only the estimator's precision
  (fp16 queries against INT4 keys) and leave the arithmetic open; the reading taken holds the query
  per head and 32-channel group g in fixed point at least as fine as fp16 for the group's large
  channels, so that every group sum is exact:

      E_g = floor(log2 max_{c in g} |q_c|)  (clamped to >= -100; 0 for an all-zero group)
      Q_c = rne(q_c * 2^(13 - E_g))           integers, |Q_c| <= 16320; exact for every channel
                                              within 2^6 of the group's largest (bf16 has 8 bits)
      a_g = 2^(E_g - 13) * fl(sum_{c in g} Q_c * code_c)  exact for 2- and 4-bit codes (|sum| < 2^23);
                                                          8-bit sums (< 2^28) round once to float32
      b_g = 2^(E_g - 13) * sum_{c in g} Q_c              exact
      t_g = fl(s_g * a_g) + fl(z_g * b_g)                three rounded fp32 operations
      r = (t_0 + t_1) + (t_2 + t_3);   l = fl(sm * r)

  which is sm * q~ . x^ for the fixed-point query q~ (|q - q~| <= 2^(E_g - 14) per channel, below
  half an fp16 ulp of the group's largest channel) and is pinned to ``logits_f64`` within the bound
  that this rounding and the float32 operation count imply.  The exact integer sums are what an
  int8 matrix-core contraction computes, in any order.

O6 normalises over the candidates only (the selector's output is the domain of the top-p pruning,
Paper-Notes "整体框架"), in float64 from the given logits with the maximum subtracted.
"""

from __future__ import annotations

import math

import numpy as np

from .numerics import F32, bf16_to_f32
from .quantize import dequantize

GROUP = 32


QFIX_BITS = 13  # Q_c = rne(q_c * 2^(QFIX_BITS - E_g))
E_MIN = -100


def q_fixed(q: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Fixed-point query per 32-channel group: (Q int64 [128], E int64 [4]) as defined above."""
    q = np.asarray(q, np.float64)
    Q = np.zeros(128, np.int64)
    E = np.zeros(4, np.int64)
    for g in range(4):
        seg = q[g * GROUP:(g + 1) * GROUP]
        m = float(np.abs(seg).max())
        if m == 0.0:
            continue
        E[g] = max(math.frexp(m)[1] - 1, E_MIN)  # m = f * 2^e with f in [0.5, 1): floor(log2 m) = e - 1
        Q[g * GROUP:(g + 1) * GROUP] = np.rint(np.ldexp(seg, QFIX_BITS - int(E[g]))).astype(np.int64)
    return Q, E


def logits_spec(qbits_h: np.ndarray, codes: np.ndarray, scale16: np.ndarray, zero16: np.ndarray,
                sm: float) -> np.ndarray:
    """float32 logits in the committed arithmetic (see module docstring).

    ``qbits_h`` uint16 [128]; ``codes`` uint8 [N][128] (of any width up to 8 bits);
    ``scale16``/``zero16`` float16 [N][4]; ``sm`` the float32 softmax scale.
    """
    Q, E = q_fixed(bf16_to_f32(qbits_h))
    c = np.asarray(codes).astype(np.int64)
    s = np.asarray(scale16, np.float16).astype(F32)
    z = np.asarray(zero16, np.float16).astype(F32)
    t = []
    for g in range(4):
        sl = slice(g * GROUP, (g + 1) * GROUP)
        # the integer sum is exact in int64 and in float64; one rounding to float32 (none below 2^24)
        a = np.ldexp((c[:, sl] @ Q[sl]).astype(np.float64), int(E[g]) - QFIX_BITS).astype(F32)
        b = F32(np.ldexp(float(Q[sl].sum()), int(E[g]) - QFIX_BITS))                                # exact
        sa = (s[:, g] * a).astype(F32)
        zb = (z[:, g] * b).astype(F32)
        t.append((sa + zb).astype(F32))
    r = ((t[0] + t[1]).astype(F32) + (t[2] + t[3]).astype(F32)).astype(F32)
    return (F32(sm) * r).astype(F32)


def logits_f64(qbits_h: np.ndarray, codes: np.ndarray, scale16: np.ndarray, zero16: np.ndarray,
               sm: float) -> np.ndarray:
    """Plain definition: sm * q . x^ in float64 over the fp32 dequantised keys."""
    q = bf16_to_f32(qbits_h).astype(np.float64)
    xhat = dequantize(codes, scale16, zero16).astype(np.float64)
    return float(np.float32(sm)) * (xhat @ q)


def softmax_f64(logits: np.ndarray) -> np.ndarray:
    """O6: softmax in float64 (max subtracted)."""
    l = np.asarray(logits, dtype=np.float64)
    if l.size == 0:
        return l
    e = np.exp(l - l.max())
    return e / e.sum()
