"""Pins for O1 (INT4 group quantisation) and O2 (page key bounds).

Each test checks the oracle against something other than itself: hand-derived closed forms
(tests/golden/quant_closed_form.json), the rounding-mode definition on exact halfway cases, the
error bound that the encoding implies, exact reconstruction of keys already on the INT4 grid, and
the characterisation of a min/max bound.  The 2- and 8-bit widths get the same checks (with
hand-packed bytes and a hand-derived scale) where they differ from 4 bits.
"""

import json
import os

import numpy as np
import pytest

from oracle import numerics, quantize

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _row_from_groups(groups):
    x = np.zeros(128, np.float32)
    for g, vals in enumerate(groups):
        x[g * 32:(g + 1) * 32] = vals
    return numerics.f32_to_bf16_bits(x)


def test_fp16_cast_is_round_to_nearest_even():
    # halfway cases between adjacent fp16 values must go to the even mantissa
    x = np.array([1 + 2**-11, 1 + 3 * 2**-11, 2049.0, 2051.0, -(1 + 2**-11)], np.float32)
    want = np.array([1.0, 1 + 2**-9, 2048.0, 2052.0, -1.0])
    assert np.array_equal(numerics.f32_to_f16(x).astype(np.float64), want)


def test_bf16_roundtrip_bits():
    bits = np.arange(0, 65536, 7, dtype=np.uint32).astype(np.uint16)
    f = numerics.bf16_to_f32(bits)
    finite = np.isfinite(f)
    assert np.array_equal(numerics.f32_to_bf16_bits(f[finite]), bits[finite])


@pytest.mark.parametrize("case", json.load(open(os.path.join(GOLD, "quant_closed_form.json")))["cases"],
                         ids=lambda c: c["name"])
def test_closed_form_groups(case):
    # put the case in group 1 of a row; the other groups hold the ramp case so they are non-trivial
    ramp = [-2.0 + 0.5 * (j % 16) for j in range(32)]
    row = _row_from_groups([ramp, case["values"], ramp, ramp])
    r = quantize.quantize_rows(row[None, :])
    assert int(numerics.f16_bits(r["scale"][0, 1])) == int(case["scale_bits"], 16)
    assert int(numerics.f16_bits(r["zero"][0, 1])) == int(case["zero_bits"], 16)
    assert r["codes"][0, 32:64].tolist() == case["codes"]
    if "packed" in case:
        assert r["packed"][0, 16:32].tolist() == [int(v, 16) for v in case["packed"]]
    # the packing puts element 2j in the low nibble
    assert np.array_equal(quantize.unpack_codes(r["packed"]), r["codes"])


def test_constant_group_dequantises_to_its_value():
    row = _row_from_groups([[1.25] * 32, [-3.0] * 32, [0.0] * 32, [7.5] * 32])
    r = quantize.quantize_rows(row[None, :])
    xh = quantize.dequantize(r["codes"], r["scale"], r["zero"])[0]
    assert np.array_equal(xh, numerics.bf16_to_f32(row))


def _random_rows(seed, n=4096, scale=1.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 128)).astype(np.float32) * np.float32(scale)
    return numerics.f32_to_bf16_bits(x)


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("seed,scale", [(0, 1.0), (1, 8.0), (2, 0.01), (3, 300.0)])
def test_min_max_codes_and_error_bound(seed, scale, bits):
    L = (1 << bits) - 1
    rows = _random_rows(seed, scale=scale)
    r = quantize.quantize_rows(rows, bits)
    x = numerics.bf16_to_f32(rows).reshape(-1, 4, 32).astype(np.float64)
    codes = r["codes"].reshape(-1, 4, 32)
    s = r["scale"].astype(np.float64)
    z = r["zero"].astype(np.float64)
    pos = s > 0
    # code of the group minimum is 0 and of the maximum is L whenever the scale is non-zero
    amin = x.argmin(-1)
    amax = x.argmax(-1)
    cmin = np.take_along_axis(codes, amin[..., None], -1)[..., 0]
    cmax = np.take_along_axis(codes, amax[..., None], -1)[..., 0]
    assert np.all(cmin[pos] == 0)
    assert np.all(cmax[pos] == L)
    assert r["packed"].shape[-1] == 16 * bits
    # reconstruction error: half a step, widened by the fp16 rounding of the scale (2^-11 relative,
    # times up to L steps at the top of the grid) and by fp32 rounding of x - z
    xh = quantize.dequantize(r["codes"], r["scale"], r["zero"]).reshape(-1, 4, 32).astype(np.float64)
    bound = 0.5 * s[..., None] * (1 + L * 2.0**-10) + 2.0**-22 * np.maximum(np.abs(x), np.abs(z[..., None]))
    assert np.all(np.abs(x - xh) <= bound)


def test_keys_on_the_int4_grid_are_reconstructed_exactly():
    rng = np.random.default_rng(5)
    n = 2048
    codes = rng.integers(0, 16, size=(n, 4, 32))
    codes[:, :, 0] = 0
    codes[:, :, 1] = 15                                      # span the full grid in every group
    s16 = (2.0 ** rng.integers(-6, 2, size=(n, 4))).astype(np.float16)   # powers of two: exact
    # zero = m * scale keeps every grid value (code + m) * scale within bf16's 8 significant bits
    z16 = (rng.integers(-64, 64, size=(n, 4)) * s16.astype(np.float64)).astype(np.float16)
    x = codes * s16.astype(np.float64)[..., None] + z16.astype(np.float64)[..., None]
    bits = numerics.f32_to_bf16_bits(x.reshape(n, 128).astype(np.float32))
    assert np.array_equal(numerics.bf16_to_f32(bits).astype(np.float64), x.reshape(n, 128))  # exact in bf16
    r = quantize.quantize_rows(bits)
    assert np.array_equal(r["codes"], codes.reshape(n, 128).astype(np.uint8))
    assert np.array_equal(r["scale"], s16)
    assert np.array_equal(r["zero"], z16)
    xh = quantize.dequantize(r["codes"], r["scale"], r["zero"])
    assert np.array_equal(xh.astype(np.float64), x.reshape(n, 128))


def test_packing_of_other_widths_by_hand():
    codes = np.array([[0, 1, 2, 3, 3, 2, 1, 0] * 16], np.uint8)
    p2 = quantize.pack_codes(codes, 2)
    assert p2.shape == (1, 32)
    assert p2[0, :2].tolist() == [0xE4, 0x1B]  # 0 | 1<<2 | 2<<4 | 3<<6, then 3 | 2<<2 | 1<<4
    c8 = np.arange(128, dtype=np.uint8)[None, :] * 2
    assert np.array_equal(quantize.pack_codes(c8, 8), c8)  # one code per byte
    p4 = quantize.pack_codes(codes, 4)
    assert p4[0, :2].tolist() == [0x10, 0x32]
    for bits, hi in ((2, 4), (4, 16), (8, 256)):
        c = np.random.default_rng(bits).integers(0, hi, size=(5, 128)).astype(np.uint8)
        assert np.array_equal(quantize.unpack_codes(quantize.pack_codes(c, bits), bits), c)
    with pytest.raises(ValueError):
        quantize.quantize_rows(np.zeros((1, 128), np.uint16), 3)


def test_scale_divisor_of_each_width_by_hand():
    # a group spanning [-1, 2]: range 3 over L levels.  2 bits: s = 1 (fp16 0x3c00), codes = x + 1;
    # 8 bits: s = fp16(3 / 255) = 1542 * 2^-17 (0x2206, worked out by hand)
    vals = [-1.0, 0.0, 1.0, 2.0] * 8
    ramp = [-2.0 + 0.5 * (j % 16) for j in range(32)]
    row = _row_from_groups([ramp, vals, ramp, ramp])
    r2 = quantize.quantize_rows(row[None, :], 2)
    assert int(numerics.f16_bits(r2["scale"][0, 1])) == 0x3C00
    assert r2["codes"][0, 32:64].tolist() == [0, 1, 2, 3] * 8
    r8 = quantize.quantize_rows(row[None, :], 8)
    assert int(numerics.f16_bits(r8["scale"][0, 1])) == 0x2206
    s = 1542 * 2.0**-17
    want = [min(255, max(0, int(np.rint((v + 1.0) / s)))) for v in vals]
    assert r8["codes"][0, 32:64].tolist() == want and want[3] == 255 and want[1] == 85


@pytest.mark.parametrize("bits", [2, 8])
def test_keys_on_the_grid_of_other_widths_are_reconstructed_exactly(bits):
    L = (1 << bits) - 1
    rng = np.random.default_rng(50 + bits)
    n = 1024
    codes = rng.integers(0, L + 1, size=(n, 4, 32))
    codes[:, :, 0] = 0
    codes[:, :, 1] = L
    s16 = (2.0 ** rng.integers(-6, 2, size=(n, 4))).astype(np.float16)
    # zero = m * scale with code + m in [-64, 255]: every grid value has at most 8 significant bits
    z16 = (rng.integers(-64, 1, size=(n, 4)) * s16.astype(np.float64)).astype(np.float16)
    x = codes * s16.astype(np.float64)[..., None] + z16.astype(np.float64)[..., None]
    kb = numerics.f32_to_bf16_bits(x.reshape(n, 128).astype(np.float32))
    assert np.array_equal(numerics.bf16_to_f32(kb).astype(np.float64), x.reshape(n, 128))
    r = quantize.quantize_rows(kb, bits)
    assert np.array_equal(r["codes"], codes.reshape(n, 128).astype(np.uint8))
    assert np.array_equal(r["scale"], s16) and np.array_equal(r["zero"], z16)


def test_out_of_fp16_range_is_rejected():
    row = _row_from_groups([[1e5] * 32, [0.0] * 32, [0.0] * 32, [0.0] * 32])
    with pytest.raises(ValueError):
        quantize.quantize_rows(row[None, :])


@pytest.mark.parametrize("n", [1, 15, 16, 17, 100])
def test_page_bounds_characterisation(n):
    rng = np.random.default_rng(n)
    kbits = numerics.f32_to_bf16_bits(rng.standard_normal((n, 3, 128)).astype(np.float32))
    kmin, kmax = quantize.page_bounds(kbits)
    x = numerics.bf16_to_f32(kbits)
    assert kmin.shape[0] == -(-n // 16)
    for j in range(kmin.shape[0]):
        blk = x[j * 16:min(n, j * 16 + 16)]
        # every key of the page lies inside the box, and each face of the box is touched by a key
        assert np.all(blk >= kmin[j]) and np.all(blk <= kmax[j])
        assert np.all(np.any(blk == kmin[j], axis=0)) and np.all(np.any(blk == kmax[j], axis=0))


def test_expected_paged_bulk_equals_incremental_appends():
    """Quantising a whole sequence at once equals appending it token by token (bounds updated)."""
    rng = np.random.default_rng(11)
    n, Hkv = 37, 2
    npg = -(-n // 16)
    P = npg + 2
    page_table = np.array([[3, 0, 4]], np.int32)
    k_pages = numerics.f32_to_bf16_bits(rng.standard_normal((P, Hkv, 16, 128)).astype(np.float32))
    bulk = quantize.expected_paged(k_pages, page_table, np.array([n]))
    k4 = np.zeros_like(bulk["k4"])
    meta = np.zeros_like(bulk["k4_meta"])
    kb = np.zeros_like(bulk["kbound"])
    for t in range(n):
        step = quantize.expected_paged(k_pages, page_table, np.array([n]), [t], [t + 1])
        m3 = np.broadcast_to(step["tok_mask"][:, None, :], k4.shape[:3])
        k4[m3] = step["k4"][m3]
        meta[m3] = step["k4_meta"][m3]
        kb[step["page_mask"]] = step["kbound"][step["page_mask"]]
    assert np.array_equal(k4, bulk["k4"])
    assert np.array_equal(meta, bulk["k4_meta"])
    assert np.array_equal(kb, bulk["kbound"])
