"""O5 estimated attention logits from the INT4 K cache; O6 softmax weights over the candidates.

The pages estimate attention weights with a mixed-precision SpGEMV of an FP16 query against the
dequantised low-bit keys (paperlayer §4.2; §B.1, Fig. 12), and top-p then needs the weights' values,
not only their order (Paper-Notes "局限与展望").

O5 is that product written out: l_i = sm * sum_c q_c * x^_ic, evaluated in float64, where

* q is the query head as given (bf16 values; every bf16 value of ordinary magnitude is also exactly an
  fp16 value, so this is the pages' FP16 query without a further rounding), and
* x^_ic = code_ic * s_g + z_g is the dequantised key of candidate i (``quantize.dequantize``), exact
  in float64.

Reading (the pages dequantise to FP16 on chip and leave the accumulation open): the estimate is
defined without intermediate roundings; an implementation reaches it within its own arithmetic's
error, which the parity rule of ``topp`` accepts per token when the implementation states it.

O6 normalises over the candidates only (the selector's output is the domain of the top-p pruning,
Paper-Notes "整体框架"), in float64 from the given logits with the maximum subtracted.
"""

from __future__ import annotations

import numpy as np

from .numerics import bf16_to_f32
from .quantize import dequantize


def logits_f64(qbits_h: np.ndarray, codes: np.ndarray, scale16: np.ndarray, zero16: np.ndarray,
               sm: float) -> np.ndarray:
    """sm * q . x^ in float64.  ``qbits_h`` uint16 [128] (bf16 bits); ``codes`` uint8 [N][128] of any
    width up to 8 bits; ``scale16``/``zero16`` float16 [N][4]; ``sm`` the softmax scale (a float32
    value, 1/sqrt(128) rounded once)."""
    q = bf16_to_f32(qbits_h).astype(np.float64)
    xhat = dequantize(codes, scale16, zero16)
    return float(np.float32(sm)) * (xhat @ q)


def softmax_f64(logits: np.ndarray) -> np.ndarray:
    """O6: softmax in float64 (max subtracted)."""
    l = np.asarray(logits, dtype=np.float64)
    if l.size == 0:
        return l
    e = np.exp(l - l.max())
    return e / e.sum()
