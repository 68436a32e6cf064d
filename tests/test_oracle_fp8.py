"""Pins of the oracle's E4M3 codec, per-tensor quantiser and bfloat16 rounding.

Each check compares the oracle with something other than itself: the closed
form of the format, a brute-force nearest-value search, and torch's own
float8_e4m3fn / bfloat16 casts (library routines).
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import fp8


def _closed_form_value(code):
    """E4M3 ("fn") value of a code, as an exact Fraction (None for NaN)."""
    s, e, m = code >> 7, (code >> 3) & 0xF, code & 7
    if e == 15 and m == 7:
        return None
    if e == 0:
        mag = Fraction(m, 512)
    else:
        mag = (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
    return -mag if s else mag


def test_decode_table_closed_form():
    tab = fp8.decode_table()
    for c in range(256):
        v = _closed_form_value(c)
        if v is None:
            assert np.isnan(tab[c])
        else:
            assert Fraction(tab[c]) == v, hex(c)
    assert tab[0x7E] == 448.0 and tab[0xFE] == -448.0
    assert tab[0x01] == 2.0 ** -9 and tab[0x08] == 2.0 ** -6
    assert tab[0x38] == 1.0 and tab[0x07] == 7 / 512
    assert np.signbit(tab[0x80]) and tab[0x80] == 0.0


def test_decode_table_matches_torch_float8():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    tab = fp8.decode_table()
    finite = ~np.isnan(tab)
    assert np.array_equal(np.isnan(ref), ~finite)
    assert np.array_equal(tab[finite], ref[finite])


def _brute_force_encode(v):
    """Nearest finite E4M3 value by search; ties -> even code; saturating."""
    tab = fp8.decode_table()
    pos_codes = np.arange(0x7F)                   # 0x00 .. 0x7E, ascending
    mags = tab[pos_codes]
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), 448.0)
    d = np.abs(a[:, None] - mags[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # among the (at most two) nearest, prefer the even code
    even = cand & (pos_codes[None, :] % 2 == 0)
    pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    code = pos_codes[pick]
    return np.where(np.signbit(v), code | 0x80, code).astype(np.uint8)


def _all_finite_bf16():
    bits = np.arange(65536, dtype=np.uint32) << 16
    vals = bits.view(np.float32)
    return vals[np.isfinite(vals)]


def test_encode_all_bf16_vs_brute_force():
    v = _all_finite_bf16()
    got = fp8.encode(v)
    for lo in range(0, v.size, 4096):
        sl = slice(lo, lo + 4096)
        assert np.array_equal(got[sl], _brute_force_encode(v[sl]))


def test_encode_ties_go_to_even():
    tab = fp8.decode_table()
    mags = tab[:0x7F]
    mids = (mags[:-1] + mags[1:]) / 2             # exact in float64
    got = fp8.encode(mids)
    lo_code = np.arange(0x7E)
    expect = np.where(lo_code % 2 == 0, lo_code, lo_code + 1)
    assert np.array_equal(got, expect.astype(np.uint8))
    assert np.array_equal(fp8.encode(-mids), (expect | 0x80).astype(np.uint8))


def test_encode_saturates_and_keeps_sign():
    assert fp8.encode(np.array([448.0, 463.9, 464.0, 1e30, np.inf])).tolist() == [0x7E] * 5
    assert fp8.encode(np.array([-1e30, -np.inf])).tolist() == [0xFE] * 2
    assert fp8.encode(np.array([0.0, -0.0, 1e-30, -1e-30])).tolist() == [0, 0x80, 0, 0x80]
    # just below / at half the smallest subnormal
    assert fp8.encode(np.array([2.0 ** -10, 2.0 ** -10 * 1.0001])).tolist() == [0, 1]


def test_encode_matches_torch_cast_in_range():
    rng = np.random.default_rng(7)
    v = np.concatenate([
        rng.standard_normal(200000) * s for s in (1e-3, 0.05, 1, 30, 150)
    ]).astype(np.float32)
    v = v[np.abs(v) <= 448]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(fp8.encode(v), ref)


def test_round_trip_finite_codes():
    tab = fp8.decode_table()
    codes = np.array([c for c in range(256) if not np.isnan(tab[c])], dtype=np.uint8)
    assert np.array_equal(fp8.encode(fp8.decode(codes)), codes)


def test_per_tensor_scale_closed_form():
    assert fp8.per_tensor_scale(np.array([448.0, -3.0])) == np.float32(1.0)
    assert fp8.per_tensor_scale(np.zeros(5)) == np.float32(1.0)
    assert fp8.per_tensor_scale(np.array([-1.0, 0.5])) == np.float32(1.0) / np.float32(448.0)
    # x = 448 * 2^j -> scale 2^j exactly and codes are the unscaled ones
    x = np.array([448.0, 1.0, -0.25, 3.5], dtype=np.float32) * np.float32(2.0 ** -5)
    codes, s = fp8.quantize(x)
    assert s == np.float32(2.0 ** -5)
    assert np.array_equal(fp8.decode(codes), [448.0, 1.0, -0.25, 3.5])


def test_quantize_error_bound():
    # |decode(q)*s - v| <= half an ulp: 2^-4 relative for normals, 2^-10 * s absolute below
    rng = np.random.default_rng(3)
    v = (rng.standard_normal(100000) * 3).astype(np.float32)
    codes, s = fp8.quantize(v)
    err = np.abs(fp8.dequantize(codes, s) - v.astype(np.float64))
    bound = np.maximum(np.abs(v) * 2.0 ** -4, 2.0 ** -10 * float(s)) * (1 + 1e-6)
    assert np.all(err <= bound)


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(11)
    v = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * 10,
        # exact ties: low half 0x8000 with even and odd kept bit
        (np.arange(1000, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
        np.array([0.0, -0.0, 3.3895314e38, 1e-40], dtype=np.float32),
    ])
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float32).numpy()
    got = fp8.bf16_round(v)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    assert np.array_equal(fp8.bf16_from_bits(fp8.bf16_bits(v)), got)


@pytest.mark.parametrize("bad", [np.nan])
def test_encode_rejects_nan(bad):
    with pytest.raises(ValueError):
        fp8.encode(np.array([bad]))


# ------------------------------------------------------------------ E5M2

def _closed_form_e5m2(code):
    """E5M2 value of a code as an exact Fraction; 'inf' / None for inf / NaN."""
    s, e, m = code >> 7, (code >> 2) & 0x1F, code & 3
    if e == 31:
        return ("-inf" if s else "inf") if m == 0 else None
    if e == 0:
        mag = Fraction(m, 1 << 16)
    else:
        mag = (1 + Fraction(m, 4)) * Fraction(2) ** (e - 15)
    return -mag if s else mag


def test_e5m2_decode_table_closed_form():
    tab = fp8.decode_table("e5m2")
    for c in range(256):
        v = _closed_form_e5m2(c)
        if v is None:
            assert np.isnan(tab[c])
        elif isinstance(v, str):
            assert tab[c] == (-np.inf if v == "-inf" else np.inf)
        else:
            assert Fraction(tab[c]) == v, hex(c)
    assert tab[0x7B] == 57344.0 and tab[0xFB] == -57344.0
    assert tab[0x01] == 2.0 ** -16 and tab[0x04] == 2.0 ** -14 and tab[0x3C] == 1.0


def test_e5m2_decode_matches_torch_float8():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e5m2).to(torch.float64).numpy()
    tab = fp8.decode_table("e5m2")
    assert np.array_equal(np.isnan(ref), np.isnan(tab))
    fin = ~np.isnan(tab)
    assert np.array_equal(tab[fin], ref[fin])


def _brute_force_e5m2(v):
    """Nearest finite E5M2 value by search; ties -> even code; saturating."""
    tab = fp8.decode_table("e5m2")
    pos_codes = np.arange(0x7C)                   # 0x00 .. 0x7B: +0 .. 57344
    mags = tab[pos_codes]
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), 57344.0)
    d = np.abs(a[:, None] - mags[None, :])
    cand = d == d.min(axis=1, keepdims=True)
    even = cand & (pos_codes[None, :] % 2 == 0)
    pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    code = pos_codes[pick]
    return np.where(np.signbit(v), code | 0x80, code).astype(np.uint8)


def test_e5m2_encode_all_bf16_vs_brute_force():
    v = _all_finite_bf16()
    got = fp8.encode(v, "e5m2")
    for lo in range(0, v.size, 4096):
        sl = slice(lo, lo + 4096)
        assert np.array_equal(got[sl], _brute_force_e5m2(v[sl]))


def test_e5m2_ties_saturation_sign():
    tab = fp8.decode_table("e5m2")
    mags = tab[:0x7C]
    mids = (mags[:-1] + mags[1:]) / 2
    lo_code = np.arange(0x7B)
    expect = np.where(lo_code % 2 == 0, lo_code, lo_code + 1).astype(np.uint8)
    assert np.array_equal(fp8.encode(mids, "e5m2"), expect)
    assert np.array_equal(fp8.encode(-mids, "e5m2"), expect | 0x80)
    assert fp8.encode(np.array([57344.0, 61439.0, 61440.0, 1e30, np.inf]), "e5m2").tolist() \
        == [0x7B] * 5
    assert fp8.encode(np.array([-0.0, 1e-30, -1e-30]), "e5m2").tolist() == [0x80, 0, 0x80]


def test_e5m2_encode_matches_torch_cast_in_range():
    rng = np.random.default_rng(9)
    v = np.concatenate([
        rng.standard_normal(200000) * s for s in (1e-5, 1e-2, 1, 300, 9000)
    ]).astype(np.float32)
    v = v[np.abs(v) <= 57344]
    ref = torch.from_numpy(v).to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert np.array_equal(fp8.encode(v, "e5m2"), ref)


def test_e5m2_quantize_scale_and_error_bound():
    assert fp8.per_tensor_scale(np.array([57344.0, 1.0]), "e5m2") == np.float32(1.0)
    x = np.array([57344.0, 1.0, -0.25, 3.5], dtype=np.float32) * np.float32(2.0 ** -12)
    codes, s = fp8.quantize(x, fmt="e5m2")
    assert s == np.float32(2.0 ** -12)
    assert np.array_equal(fp8.decode(codes, "e5m2"), [57344.0, 1.0, -0.25, 3.5])
    # half an ulp of a 2-bit mantissa: 2^-3 relative for normals
    rng = np.random.default_rng(5)
    v = (rng.standard_normal(100000) * 3).astype(np.float32)
    codes, s = fp8.quantize(v, fmt="e5m2")
    err = np.abs(fp8.dequantize(codes, s, "e5m2") - v.astype(np.float64))
    bound = np.maximum(np.abs(v) * 2.0 ** -3, 2.0 ** -17 * float(s)) * (1 + 1e-6)
    assert np.all(err <= bound)
