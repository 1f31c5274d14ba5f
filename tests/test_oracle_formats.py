"""Pins of the oracle's number formats (CPU only).

Each check ties oracle.formats to something other than itself: the OCP format tables
(tests/golden), hand-worked roundings, the torch CPU float8_e4m3fn cast (a library routine
the E4M3 case reduces to), IEEE binary16 facts, and closed-form error bounds."""
import numpy as np
import pytest
import torch

from conftest import read_golden
from oracle import formats as F


def _val(s):
    return float("nan") if s == "nan" else float(s)


def test_e4m3_table_matches_ocp_spec():
    for code_s, val_s in read_golden("e4m3fn_values.txt"):
        code = int(code_s, 16)
        got = F.e4m3_decode(np.array([code], dtype=np.uint8))[0]
        want = _val(val_s)
        if np.isnan(want):
            assert np.isnan(got), code_s
        else:
            assert got == want and np.signbit(got) == np.signbit(want), (code_s, got, want)


def test_e4m3_all_finite_codes_round_trip():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert len(codes) == 254
    vals = F.e4m3_decode(codes)
    assert np.array_equal(F.e4m3_encode(vals), codes)  # includes -0 -> 0x80


def test_e4m3_midpoints_go_to_even_code():
    mags = F.e4m3_magnitudes()
    assert np.all(np.diff(mags) > 0)
    mids = (mags[:-1] + mags[1:]) / 2  # exact in fp64
    got = F.e4m3_encode(mids).astype(np.int64)
    lo = np.arange(126)
    want = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(got, want)
    # just off the midpoint, nearest wins
    eps = np.minimum(np.diff(mags), 1) * 1e-6
    assert np.array_equal(F.e4m3_encode(mids - eps).astype(np.int64), lo)
    assert np.array_equal(F.e4m3_encode(mids + eps).astype(np.int64), lo + 1)


def test_e4m3_saturation_nan_and_signed_zero():
    v = np.array([448.0, 449.0, 464.0, 1e30, np.inf, -500.0, -np.inf, 0.0, -0.0, np.nan, -np.nan])
    got = F.e4m3_encode(v).tolist()
    assert got[:7] == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]
    assert got[7:9] == [0x00, 0x80]
    assert got[9] & 0x7F == 0x7F and got[10] & 0x7F == 0x7F


def test_e4m3_matches_torch_cast_on_clamped_fp32():
    rng = np.random.default_rng(123)
    parts = [
        rng.standard_normal(20000) * 50,
        rng.standard_normal(20000) * 2.0 ** -7,  # subnormal region
        (F.e4m3_magnitudes()[:-1] + F.e4m3_magnitudes()[1:]) / 2,  # every tie
        rng.uniform(-448, 448, 20000),
    ]
    x = np.clip(np.concatenate(parts), -448, 448).astype(np.float32)
    x = np.concatenate([x, -x])
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = F.e4m3_encode(x.astype(np.float64))
    assert np.array_equal(got, want)


def test_e4m3_error_bound_closed_form():
    # |x - dec(enc(x))| <= half the spacing of the grid at x, for |x| <= 448
    rng = np.random.default_rng(5)
    x = rng.uniform(-448, 448, 50000)
    err = np.abs(F.e4m3_decode(F.e4m3_encode(x)) - x)
    a = np.abs(x)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    half_ulp = 2.0 ** (e - 3) / 2
    assert np.all(err <= half_ulp * (1 + 1e-12))


def test_e2m1_table_matches_ocp_spec():
    for code_s, val_s in read_golden("e2m1_values.txt"):
        code = int(code_s, 16)
        got = F.e2m1_decode(np.array([code]))[0]
        want = _val(val_s)
        assert got == want and np.signbit(got) == np.signbit(want), (code_s, got, want)


def test_e2m1_round_trip_and_hand_worked_rounding():
    codes = np.arange(16, dtype=np.uint8)
    assert np.array_equal(F.e2m1_encode(F.e2m1_decode(codes)), codes)
    for v_s, c_s in read_golden("e2m1_rounding.txt"):
        got = int(F.e2m1_encode(np.array([float(v_s)]))[0])
        assert got == int(c_s, 16), (v_s, got, c_s)
    with pytest.raises(ValueError):
        F.e2m1_encode(np.array([np.nan]))


def test_fp16_and_bf16_bit_facts():
    # IEEE binary16: 1 = 0x3C00, ulp(1) = 2^-10, max 65504 = 0x7BFF, min subnormal 2^-24
    x = np.array([1.0, 1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 65504.0, 2.0 ** -24, 2.0 ** -25,
                  3 * 2.0 ** -26, -2.0, 65520.0])
    assert F.f16_encode(x).tolist() == [0x3C00, 0x3C00, 0x3C02, 0x7BFF, 0x0001, 0x0000,
                                       0x0001, 0xC000, 0x7C00]
    assert F.f16_decode(np.array([0x3C00, 0x0001, 0xFBFF], dtype=np.uint16)).tolist() == \
        [1.0, 2.0 ** -24, -65504.0]
    # bf16 is the top half of an fp32: 0x3F80 = 1, 0xC0C0 = -6, 0x0001 = 2^-133
    assert F.bf16_decode(np.array([0x3F80, 0xC0C0, 0x0001, 0x7F7F], dtype=np.uint16)).tolist() \
        == [1.0, -6.0, 2.0 ** -133, (2 - 2.0 ** -7) * 2.0 ** 127]


def test_f32_quotient_is_correctly_rounded():
    # fp32(1/3) = 0x3EAAAAAB; fp32(2/3) = 0x3F2AAAAB; 1/448 known bits
    q = F.f32_quotient(np.array([1.0, 2.0, 1.0]), np.array([3.0, 3.0, 448.0]))
    bits = q.astype(np.float32).view(np.uint32).tolist()
    assert bits[0] == 0x3EAAAAAB and bits[1] == 0x3F2AAAAB
    assert np.float32(q[2]) == np.float32(1.0) / np.float32(448.0)
    # against an exact rational check on random fp32 operands: the result is the fp32
    # value nearest to x/s (no other fp32 value is closer)
    rng = np.random.default_rng(9)
    xs = rng.standard_normal(2000).astype(np.float32).astype(np.float64)
    ss = np.abs(rng.standard_normal(2000)).astype(np.float32).astype(np.float64) + 1e-3
    ss = ss.astype(np.float32).astype(np.float64)
    q = F.f32_quotient(xs, ss)
    from fractions import Fraction
    for x, s, r in zip(xs[:300], ss[:300], q[:300]):
        exact = Fraction(x) / Fraction(s)
        r32 = np.float32(r)
        up, dn = np.nextafter(r32, np.float32(np.inf)), np.nextafter(r32, np.float32(-np.inf))
        d = abs(Fraction(float(r32)) - exact)
        assert d <= abs(Fraction(float(up)) - exact) and d <= abs(Fraction(float(dn)) - exact)


def _fval(s):
    return {"nan": float("nan"), "inf": float("inf"), "-inf": float("-inf")}.get(s, None) \
        if s in ("nan", "inf", "-inf") else float(s)


def test_e5m2_table_matches_ocp_spec():
    for code_s, val_s in read_golden("e5m2_values.txt"):
        code = int(code_s, 16)
        got = F.e5m2_decode(np.array([code], dtype=np.uint8))[0]
        want = _fval(val_s)
        if np.isnan(want):
            assert np.isnan(got), code_s
        else:
            assert got == want and np.signbit(got) == np.signbit(want), (code_s, got, want)


def test_e5m2_all_finite_codes_round_trip():
    codes = np.array([c for c in range(256) if (c & 0x7F) < 0x7C], dtype=np.uint8)
    assert len(codes) == 248
    assert np.array_equal(F.e5m2_encode(F.e5m2_decode(codes)), codes)  # includes -0 -> 0x80


def test_e5m2_midpoints_go_to_even_code():
    mags = F.e5m2_magnitudes()
    assert np.all(np.diff(mags) > 0) and mags[-1] == F.E5M2_MAX
    mids = (mags[:-1] + mags[1:]) / 2
    lo = np.arange(len(mags) - 1)
    assert np.array_equal(F.e5m2_encode(mids).astype(np.int64), np.where(lo % 2 == 0, lo, lo + 1))
    eps = np.diff(mags) * 1e-6
    assert np.array_equal(F.e5m2_encode(mids - eps).astype(np.int64), lo)
    assert np.array_equal(F.e5m2_encode(mids + eps).astype(np.int64), lo + 1)


def test_e5m2_saturation_nan_and_signed_zero():
    v = np.array([57344.0, 60000.0, 61440.0, 1e30, np.inf, -7e4, -np.inf, 0.0, -0.0, np.nan])
    got = F.e5m2_encode(v).tolist()
    assert got[:7] == [0x7B, 0x7B, 0x7B, 0x7B, 0x7B, 0xFB, 0xFB]
    assert got[7:9] == [0x00, 0x80]
    assert got[9] & 0x7F == 0x7F


def test_e5m2_matches_torch_cast_on_clamped_fp32():
    rng = np.random.default_rng(321)
    mags = F.e5m2_magnitudes()
    parts = [rng.standard_normal(20000) * 3000, rng.standard_normal(20000) * 2.0 ** -15,
             (mags[:-1] + mags[1:]) / 2, rng.uniform(-57344, 57344, 20000)]
    x = np.clip(np.concatenate(parts), -57344, 57344).astype(np.float32)
    x = np.concatenate([x, -x])
    want = torch.from_numpy(x).to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert np.array_equal(F.e5m2_encode(x.astype(np.float64)), want)


def test_e5m2_error_bound_closed_form():
    rng = np.random.default_rng(6)
    x = rng.uniform(-57344, 57344, 50000)
    x = np.concatenate([x, rng.standard_normal(50000) * 2.0 ** -14])
    err = np.abs(x - F.e5m2_decode(F.e5m2_encode(x)))
    a = np.abs(x)
    # spacing: 2^-16 below 2^-14, else 2^(floor(log2 a) - 2)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
    spacing = 2.0 ** (e - 2)
    assert np.all(err <= spacing / 2 + 1e-300)
