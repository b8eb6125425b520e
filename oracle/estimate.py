"""O5 estimated attention logits from the INT4 K cache; O6 softmax weights over the candidates.

The pages estimate attention weights with a mixed-precision SpGEMV of the query against the
dequantised 4-bit keys (paperlayer §4.2; §B.1, Fig. 12) and then need the weights' values, not only
their order (Paper-Notes "局限与展望": top-p needs approximate weights rather than a ranking).

Two versions of O5 are given:

* ``logits_f64`` -- the plain definition: l_i = sm * sum_c q_c * x^_ic in float64, with x^ the fp32
  dequantised key (see ``quantize.dequantize``).
* ``logits_spec`` -- the float32 evaluation order the GPU kernel commits to.  A top-p *set* is decided
  from these logits, so both sides must hold the same values; the pages leave the arithmetic open
  (their kernel dequantises to FP16), so the reading taken is fp32 with this fixed order:

      per group g (32 channels) and head h:
          a_g = fold_{c in g, ascending} (a + q_c * code_c)     starting at +0; products are exact
          b_g = fold_{c in g, ascending} (b + q_c)              starting at +0
          t_g = fl(s_g * a_g) + fl(z_g * b_g)                   three rounded fp32 operations
      r = (t_0 + t_1) + (t_2 + t_3);   l = fl(sm * r)

  which equals the plain definition exactly in real arithmetic (x^ = code*s + z factorises per
  group) and is pinned to ``logits_f64`` within a derived float32 error bound.

O6 normalises over the candidates only (the selector's output is the domain of the top-p pruning,
Paper-Notes "整体框架"), in float64 from the given logits with the maximum subtracted.
"""

from __future__ import annotations

import numpy as np

from .numerics import F32, bf16_to_f32
from .quantize import dequantize

GROUP = 32


def group_qsums(q: np.ndarray) -> np.ndarray:
    """b_g = float32 fold of q over each 32-channel group."""
    out = np.zeros(4, F32)
    for g in range(4):
        acc = F32(0.0)
        for c in range(g * GROUP, (g + 1) * GROUP):
            acc = F32(acc + q[c])
        out[g] = acc
    return out


def logits_spec(qbits_h: np.ndarray, codes: np.ndarray, scale16: np.ndarray, zero16: np.ndarray,
                sm: float) -> np.ndarray:
    """float32 logits in the committed evaluation order (see module docstring).

    ``qbits_h`` uint16 [128]; ``codes`` uint8 [N][128]; ``scale16``/``zero16`` float16 [N][4];
    ``sm`` the float32 softmax scale.
    """
    q = bf16_to_f32(qbits_h)
    c = np.asarray(codes).astype(F32)
    s = np.asarray(scale16, np.float16).astype(F32)
    z = np.asarray(zero16, np.float16).astype(F32)
    bsum = group_qsums(q)
    N = c.shape[0]
    t = []
    for g in range(4):
        a = np.zeros(N, F32)
        for ch in range(g * GROUP, (g + 1) * GROUP):
            a = (a + (q[ch] * c[:, ch]).astype(F32)).astype(F32)
        sa = (s[:, g] * a).astype(F32)
        zb = (z[:, g] * bsum[g]).astype(F32)
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
