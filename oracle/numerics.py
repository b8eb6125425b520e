"""Bit-level number conversions used by the oracle (its own; nothing here is shared with the GPU path).

* bf16 values arrive as uint16 bit patterns; widening to float32 is exact (append 16 zero bits).
* fp16 rounding uses numpy's float32 -> float16 cast, which rounds to nearest, ties to even
  (checked by a pin on exact halfway cases).
* ``f32_key`` maps non-negative float32 values to uint32 in an order-preserving way (the IEEE bit
  pattern itself), the domain in which the bisection of the top-p threshold takes midpoints.
* ``f32_fma`` is the float32 fused multiply-add, a*b + c rounded once to nearest even, from float64
  arithmetic with the rounding error of the float64 sum recovered exactly (two-sum), so a float64
  result that lands exactly halfway between two float32 values is resolved by the bits float64 lost.
"""

from __future__ import annotations

import numpy as np

F32 = np.float32


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 values (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bits, round to nearest even (used only to build test fixtures)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return (u >> np.uint64(16)).astype(np.uint16)


def f32_to_f16(x: np.ndarray) -> np.ndarray:
    """float32 -> float16, round to nearest even."""
    return np.asarray(x, dtype=np.float32).astype(np.float16)


def f16_bits(x16: np.ndarray) -> np.ndarray:
    return np.asarray(x16, dtype=np.float16).view(np.uint16)


def f16_from_bits(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16)


def f32_key(x: np.ndarray) -> np.ndarray:
    """Order-preserving uint32 image of non-negative float32 values (their bit pattern)."""
    x = np.asarray(x, dtype=np.float32)
    if np.any(x < 0) or np.any(np.isnan(x)):
        raise ValueError("f32_key expects non-negative, non-NaN values")
    return (x + F32(0.0)).view(np.uint32)  # +0.0 turns -0.0 into +0.0


def f32_from_key(k) -> np.float32:
    return np.array([k], dtype=np.uint32).view(np.float32)[0]


def f32_fma(a, b, c) -> np.ndarray:
    """float32 a*b + c with one rounding (to nearest, ties to even), elementwise; finite inputs whose
    product has at most 53 significant bits (any float32 times a bf16 value or a float32 value)."""
    a64 = np.asarray(a, np.float32).astype(np.float64)
    b64 = np.asarray(b, np.float32).astype(np.float64)
    c64 = np.asarray(c, np.float32).astype(np.float64)
    p = a64 * b64                      # exact: at most 24 + 24 significant bits
    s = p + c64
    bp = s - c64
    err = (p - bp) + (c64 - (s - bp))  # two-sum: s + err == p + c exactly
    r = s.astype(np.float32)           # nearest even of s
    r64 = r.astype(np.float64)
    d = s - r64                        # exact (within half a float32 step of s)
    up = np.nextafter(r, np.float32(np.inf))
    dn = np.nextafter(r, np.float32(-np.inf))
    # s exactly halfway between r and a neighbour: the exact sum lies beyond the midpoint when err
    # points away from r, and then rounds to that neighbour
    to_up = (d > 0) & (d == (up.astype(np.float64) - r64) / 2) & (err > 0)
    to_dn = (d < 0) & (-d == (r64 - dn.astype(np.float64)) / 2) & (err < 0)
    return np.where(to_up, up, np.where(to_dn, dn, r)).astype(np.float32)
