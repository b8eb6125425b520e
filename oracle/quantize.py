"""O1 INT4 K quantisation and O2 page key bounds.

O1 follows the 4-bit K cache of the pages (Paper-Notes "关键设计 / 4-bit K缓存量化"; paperlayer
§4.2 and §B.1: dynamic quantisation with FP16 scales and zero points, two 4-bit values per byte).
The pages leave the granularity, the rounding and the nibble order open; the readings taken are:

* asymmetric min/max quantisation in groups of 32 consecutive channels of one (token, kv-head) row,
  one fp16 scale and one fp16 zero point per group (128 channels -> 4 groups);
* scale  s = fp16_rne( fp32(max - min) / 15 ),  zero  z = fp16_rne(min);
* code_c = 0 when s == 0, else clamp(rint_even( fp32(x_c - z) / s ), 0, 15), with the fp16 s and z
  widened to fp32 and every operation a correctly rounded fp32 operation;
* byte j of a row holds code_{2j} in its low nibble and code_{2j+1} in its high nibble;
* dequantised value  x^_c = code_c * s + z, exact (float64 holds it: an 8-bit code times an 11-bit
  scale plus an 11-bit zero spans fewer than 53 bits over the whole fp16 range).  The pages dequantise
  to FP16 on chip; the estimate's definition (``estimate.logits_f64``) takes the exact value.

This is an encoding, so its float32 operation sequence is the specification; numpy float32
arithmetic performs each operation with IEEE rounding, one at a time.

Other code widths (the pages' precision ablation of the estimator, paperlayer §4.2 and Fig. 6, and the
4-bit table in Paper-Notes "关键设计 / 4-bit K缓存量化", compare 2-, 4- and 8-bit K copies at p = 0.85
without defining the other widths' encodings).  Reading: the same scheme with L = 2^bits - 1 levels in
place of 15 (s = fp16_rne(fp32(max - min) / L), codes clamped to [0, L]), the same groups and fp16
scale/zero, and 8/bits codes per byte, the lowest-numbered channel in the lowest bits.

O2 is the per-page, per-channel key minimum and maximum over the page's valid slots, used by the
Quest-style page bound (the base selector that the Twilight pages name but do not define).  Min and
max of bf16 values are bf16 values, so the bounds are exact.
"""

from __future__ import annotations

import numpy as np

from .numerics import F32, bf16_to_f32, f16_bits

GROUP = 32
NGROUPS = 128 // GROUP
PAGE = 16


BITS = (2, 4, 8)  # code widths


def pack_codes(code: np.ndarray, bits: int = 4) -> np.ndarray:
    """codes uint8 [..., 128] -> uint8 [..., 16 * bits]: byte j holds codes (8/bits) j .. +(8/bits - 1),
    the first in the lowest bits."""
    per = 8 // bits
    c = np.asarray(code, np.uint16).reshape(code.shape[:-1] + (128 // per, per))
    out = np.zeros(c.shape[:-1], np.uint16)
    for i in range(per):
        out |= c[..., i] << (bits * i)
    return out.astype(np.uint8)


def quantize_rows(kbits: np.ndarray, bits: int = 4) -> dict:
    """Quantise bf16 key rows ``uint16 [..., 128]`` to ``bits``-bit codes.

    Returns ``codes`` uint8 [..., 128], ``packed`` uint8 [..., 16 * bits], ``scale`` and ``zero``
    float16 [..., 4].
    """
    if bits not in BITS:
        raise ValueError("bits must be 2, 4 or 8")
    L = (1 << bits) - 1
    x = bf16_to_f32(kbits)
    shp = x.shape[:-1]
    xg = x.reshape(shp + (NGROUPS, GROUP))
    mn = xg.min(axis=-1)
    mx = xg.max(axis=-1)
    if not (np.all(np.isfinite(x)) and np.all(np.abs(x) <= 65504.0)):
        raise ValueError("quantisation input must be finite and within the fp16 range")
    rng = (mx - mn).astype(F32)                      # fp32 subtraction
    s16 = (rng / F32(L)).astype(np.float16)         # fp32 division, then fp16 round-to-nearest-even
    z16 = mn.astype(np.float16)
    s = s16.astype(F32)
    z = z16.astype(F32)
    diff = (xg - z[..., None]).astype(F32)           # fp32 subtraction
    safe = np.where(s == 0, F32(1.0), s).astype(F32)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (diff / safe[..., None]).astype(F32)     # fp32 division
    code = np.clip(np.rint(t), 0, L)                 # rint = round half to even
    code = np.where((s == 0)[..., None], 0, code).astype(np.uint8).reshape(shp + (128,))
    return {"codes": code, "packed": pack_codes(code, bits), "scale": s16, "zero": z16}


def unpack_codes(packed: np.ndarray, bits: int = 4) -> np.ndarray:
    """uint8 [..., 16 * bits] -> codes uint8 [..., 128] (for 4 bits: element 2j = low nibble of byte j)."""
    packed = np.asarray(packed, dtype=np.uint8)
    per = 8 // bits
    out = np.empty(packed.shape[:-1] + (packed.shape[-1], per), np.uint8)
    for i in range(per):
        out[..., i] = (packed >> (bits * i)) & ((1 << bits) - 1)
    return out.reshape(packed.shape[:-1] + (128,))


def dequantize(codes: np.ndarray, scale16: np.ndarray, zero16: np.ndarray) -> np.ndarray:
    """x^ = code * s + z, exact in float64; codes [..., 128], scale/zero [..., 4]."""
    c = np.asarray(codes, dtype=np.float64).reshape(codes.shape[:-1] + (NGROUPS, GROUP))
    s = np.asarray(scale16, dtype=np.float16).astype(np.float64)[..., None]
    z = np.asarray(zero16, dtype=np.float16).astype(np.float64)[..., None]
    return (c * s + z).reshape(codes.shape)


def page_bounds(kbits_seq: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """O2: per-page channel-wise key min and max of one sequence.

    ``kbits_seq`` uint16 [n][Hkv][128] in logical order.  Returns float32 ``kmin``, ``kmax`` of
    shape [ceil(n/16)][Hkv][128]; a partial last page uses only its valid slots.
    """
    x = bf16_to_f32(kbits_seq)
    n = x.shape[0]
    npg = -(-n // PAGE)
    kmin = np.empty((npg,) + x.shape[1:], F32)
    kmax = np.empty((npg,) + x.shape[1:], F32)
    for j in range(npg):
        blk = x[j * PAGE:min(n, (j + 1) * PAGE)]
        kmin[j] = blk.min(axis=0)
        kmax[j] = blk.max(axis=0)
    return kmin, kmax


# --------------------------------------------------------------------------------------------------
# Expected device arrays in the paged layout (for element-by-element comparison)
# --------------------------------------------------------------------------------------------------
def expected_paged(k_pages: np.ndarray, page_table: np.ndarray, seq_lens: np.ndarray,
                   tok_begin=None, tok_end=None, bits: int = 4) -> dict:
    """Expected ``k4`` [P][Hkv][16][16 * bits] u8, ``k4_meta`` [P][Hkv][16][4][2] fp16 bits and ``kbound``
    [P][Hkv][2][128] bf16 bits for the tokens in [tok_begin[b], tok_end[b]) of each sequence
    (default: the whole sequence).  Entries that the range does not define are returned as masks
    ``tok_mask`` [P][Hkv?][16] and ``page_mask`` [P] so a comparison can skip them.
    """
    P, Hkv = k_pages.shape[0], k_pages.shape[1]
    B = len(seq_lens)
    tb = np.zeros(B, np.int64) if tok_begin is None else np.asarray(tok_begin, np.int64)
    te = np.asarray(seq_lens, np.int64) if tok_end is None else np.asarray(tok_end, np.int64)
    k4 = np.zeros((P, Hkv, PAGE, 16 * bits), np.uint8)
    meta = np.zeros((P, Hkv, PAGE, NGROUPS, 2), np.uint16)
    kb = np.zeros((P, Hkv, 2, 128), np.uint16)
    tok_mask = np.zeros((P, PAGE), bool)
    page_mask = np.zeros(P, bool)
    for b in range(B):
        if te[b] <= tb[b]:
            continue
        first_pg, last_pg = tb[b] // PAGE, (te[b] - 1) // PAGE
        for j in range(int(first_pg), int(last_pg) + 1):
            phys = int(page_table[b, j])
            rows = k_pages[phys]                      # [Hkv][16][128]
            q = quantize_rows(rows, bits)
            lo = max(int(tb[b]) - j * PAGE, 0)
            hi = min(int(te[b]) - j * PAGE, PAGE)
            sl = slice(lo, hi)
            k4[phys, :, sl] = q["packed"][:, sl]
            meta[phys, :, sl, :, 0] = f16_bits(q["scale"][:, sl])
            meta[phys, :, sl, :, 1] = f16_bits(q["zero"][:, sl])
            tok_mask[phys, sl] = True
            # bounds over the page's slots that hold tokens < tok_end
            valid = min(int(te[b]) - j * PAGE, PAGE)
            x = bf16_to_f32(rows[:, :valid, :])         # [Hkv][valid][128]
            kb[phys, :, 0, :] = (x.min(axis=1).view(np.uint32) >> 16).astype(np.uint16)
            kb[phys, :, 1, :] = (x.max(axis=1).view(np.uint32) >> 16).astype(np.uint16)
            page_mask[phys] = True
    return {"k4": k4, "k4_meta": meta, "kbound": kb, "tok_mask": tok_mask, "page_mask": page_mask}
