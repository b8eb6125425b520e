"""The estimate kernel's declared arithmetic and the parity band it implies (test infrastructure).

The oracle defines the estimated logit as sm * q . x^ in float64 (``oracle.estimate.logits_f64``).
The HIP kernel reaches that value within a stated error; this module writes that statement down so
that the GPU tests can widen the top-p ambiguity sets by exactly that much, per token, and no more.
It is a model of the kernel's precision, written from the kernel's documented arithmetic; it shares
no code with the kernel and is never used to decide a parity set.

Declared arithmetic (per query head and 32-channel group g):
  E_g = floor(log2 max_{c in g} |q_c|), clamped to >= -100 (0 for an all-zero group)
  Q_c = rne(q_c 2^(20 - E_g))     |Q_c| <= 2088960; three int8 digits Q = 2^14 d2 + 2^7 d1 + d0
  S_g = sum_{c in g} Q_c code_c    exact (integer matrix-core sums of the digits)
  a_g = 2^(E_g - 20) S_g, b_g = 2^(E_g - 20) sum_{c in g} Q_c    exact in float64
  t_g = fl64(s_g a_g + z_g b_g)    (both products exact in float64; one rounding)
  r = fl64(fl64(t_0 + t_1) + fl64(t_2 + t_3)),  logit = fl32(fl64(sm r))
so the kernel holds q~_c = Q_c 2^(E_g - 20), equal to q_c for every channel within 2^12 of its group's
largest magnitude (a bf16 value has 8 significant bits), and otherwise within 2^(E_g - 21).

Per-token logit error bound (``logit_err_bound``):
  |logit - l_f64| <= sm sum_c |q_c - q~_c| |x^_c|       (query grid; zero for most queries)
                    + 2^-24 |l| (1 + 2^-10)             (the final float32 rounding)
                    + 2^-45 sm sum_c |q_c| |x^_c|        (float64 roundings, with a wide margin)
The weights the kernel derives add an exponential error of at most 1.4e-7 relative (measured against
float64), which the 1e-6 band of the parity rule absorbs; the kernel's masses are 64-bit fixed point
floor(e 2^40) of the max-1 weights, off by at most N 2^-40 of the total (``tau_p_extra``).
"""

from __future__ import annotations

import math

import numpy as np

from oracle.numerics import bf16_to_f32
from oracle.quantize import dequantize

QBITS = 20
E_MIN = -100
Q_MAX = 2088960
MASS_FIX = 2.0**-40


def group_exponents(q: np.ndarray) -> np.ndarray:
    m = np.abs(np.asarray(q, np.float64)).reshape(4, 32).max(-1)
    return np.array([max(math.frexp(float(x))[1] - 1, E_MIN) if x > 0 else 0 for x in m], np.int64)


def fixed_query(qbits_h: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """(Q int64 [128], E int64 [4]) of the declared query grid."""
    q = bf16_to_f32(qbits_h).astype(np.float64)
    E = group_exponents(q)
    Q = np.rint(np.ldexp(q, np.repeat(QBITS - E, 32))).astype(np.int64)
    return Q, E


def digits(Q: np.ndarray) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    d2 = Q >> 14
    r = Q - (d2 << 14)
    return d2, r >> 7, r & 127


def kernel_logits(qbits_h, codes, scale16, zero16, sm) -> np.ndarray:
    """The declared arithmetic, operation by operation (float32 result)."""
    Q, E = fixed_query(qbits_h)
    c = np.asarray(codes).astype(np.int64)
    s = np.asarray(scale16, np.float16).astype(np.float64)
    z = np.asarray(zero16, np.float16).astype(np.float64)
    t = []
    for g in range(4):
        sl = slice(32 * g, 32 * g + 32)
        a = np.ldexp((c[:, sl] @ Q[sl]).astype(np.float64), int(E[g]) - QBITS)
        b = math.ldexp(float(Q[sl].sum()), int(E[g]) - QBITS)
        t.append(s[:, g] * a + z[:, g] * b)
    r = (t[0] + t[1]) + (t[2] + t[3])
    return (np.float64(np.float32(sm)) * r).astype(np.float32)


def logit_err_bound(qbits_h, codes, scale16, zero16, logits) -> np.ndarray:
    """Per-candidate bound on |kernel logit - logits_f64| (see the module docstring)."""
    sm = float(np.float32(1.0 / math.sqrt(128)))
    q = bf16_to_f32(qbits_h).astype(np.float64)
    Q, E = fixed_query(qbits_h)
    qt = np.ldexp(Q.astype(np.float64), np.repeat(E - QBITS, 32))
    xa = np.abs(dequantize(codes, scale16, zero16))
    dq = np.abs(q - qt)
    qerr = xa @ dq if dq.any() else np.zeros(xa.shape[0])
    return sm * qerr + 2.0**-24 * (1 + 2.0**-10) * np.abs(logits) + 2.0**-45 * sm * (xa @ np.abs(q))


def band(qbits_h, codes, scale16, zero16, logits):
    """The ``band`` hook of ``oracle.pipeline``: per-token logit error bounds and the mass resolution."""
    err = logit_err_bound(qbits_h, codes, scale16, zero16, logits)
    return err, len(logits) * MASS_FIX
