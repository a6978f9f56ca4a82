"""Pins of the oracle's number formats and quantizer (CPU only).

The oracle's binary16, E4M3 and int8 code is checked against things other
than itself: numpy's float16 and PyTorch's float8_e4m3fn conversions (library
routines), code points of the OCP OFP8 E4M3 format (with the +-448 range the
KVcache-learning page, chapter s09, states), exact rational arithmetic, and
closed-form error bounds.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

ALL_F16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)


def test_f16_decode_all_codes_match_numpy():
    got = oracle.f16_bits_to_f64(ALL_F16)
    ref = ALL_F16.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_f32_to_f16_rne_matches_numpy():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * np.float32(3),
        (rng.standard_normal(50000) * 1e-5).astype(np.float32),       # subnormal half range
        (rng.standard_normal(50000) * 3e4).astype(np.float32),        # near overflow
        np.array([0.0, -0.0, 65504, 65519.99, 65520, 65536, 1e9, -1e9, 2.0 ** -24,
                  2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -14, np.inf, -np.inf], np.float32),
    ])
    # every halfway point between consecutive fp16 values (ties go to even)
    f = ALL_F16[:0x7C00].view(np.float16).astype(np.float64)
    mids = ((f[:-1] + f[1:]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids])
    got = oracle.f32_to_f16_bits(x)
    ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


def test_e4m3_decode_all_codes_match_torch(golden_dir):
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.e4m3_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    spec = json.load(open(os.path.join(golden_dir, "e4m3_values.json")))
    for p in spec["points"]:
        v = oracle.e4m3_to_f64(np.array([p["code"]], np.uint8))[0]
        assert v == p["value"] and math.copysign(1, v) == math.copysign(1, p["value"]), p
    for c in spec["nan_codes"]:
        assert np.isnan(oracle.e4m3_to_f64(np.array([c], np.uint8))[0])


def test_e4m3_encode_roundtrip_and_ties():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = oracle.e4m3_to_f64(codes).astype(np.float32)
    assert np.array_equal(oracle.f32_to_e4m3(vals), codes)
    # midpoints between adjacent positive codes: ties go to the even code
    pos = np.arange(0, 0x7F, dtype=np.uint8)
    pv = oracle.e4m3_to_f64(pos)
    mids = ((pv[:-1] + pv[1:]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (pv[:-1] + pv[1:]) / 2)  # exact in fp32
    enc = oracle.f32_to_e4m3(mids)
    lo, hi = pos[:-1], pos[1:]
    expect = np.where(lo % 2 == 0, lo, hi)
    assert np.array_equal(enc, expect)


def test_e4m3_encode_matches_torch_inside_range_and_saturates():
    rng = np.random.default_rng(2)
    y = np.concatenate([rng.standard_normal(300000) * 60, rng.standard_normal(50000) * 1e-3,
                        rng.uniform(-463.9, 463.9, 50000)]).astype(np.float32)
    got = oracle.f32_to_e4m3(y)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)
    big = np.array([448.0001, 464.0, 500.0, 1e6, np.inf], np.float32)
    assert np.all(oracle.f32_to_e4m3(big) == 0x7E)
    assert np.all(oracle.f32_to_e4m3(-big) == 0xFE)
    assert oracle.f32_to_e4m3(np.array([np.nan], np.float32))[0] == 0x7F


def test_int8_rounding_points():
    y = np.array([0.5, 1.5, 2.5, -0.5, -1.5, 126.5, 127.4, 127.5, 200.0, -200.0, -127.6,
                  0.49999997], np.float32)
    expect = [0, 2, 2, 0, -2, 126, 127, 127, 127, -127, -127, 0]
    assert oracle.f32_to_i8(y).tolist() == expect


def _fl32(q: Fraction) -> Fraction:
    """Round an exact rational to the nearest binary32 value (ties to even), normal range."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    ulp = Fraction(2) ** (e - 23)
    m = a / ulp
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * ulp


def _round_half_even(q: Fraction) -> int:
    fl = q.numerator // q.denominator
    rem = q - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return fl


@pytest.mark.parametrize("amax_bits", [0x3C00, 0x4400, 0x4C00, 0x3555, 0x4247, 0x1F00])
def test_int8_quantizer_exhaustive_fp16(amax_bits):
    """All fp16 x with |x| <= a: scale and codes equal the definition written with
    exact rationals, amax maps to +-127 and |x - code*s| <= s/2."""
    a = np.array([amax_bits], np.uint16).view(np.float16)[0]
    xs = ALL_F16.view(np.float16)
    xs = xs[np.isfinite(xs) & (np.abs(xs) <= a)]
    rows = np.concatenate([xs, np.array([a], np.float16)])
    rows = np.resize(rows, (len(rows) // 64 + 1) * 64).reshape(-1, 64)  # pad by repetition
    rows[:, 0] = a                                  # every row has amax a
    codes, sbits = oracle.quantize_rows(rows.astype(np.float32), "i8")
    assert np.all(sbits == sbits[0, ...].reshape(-1)[0])
    s32 = _fl32(Fraction(float(a)) / 127)
    s16 = np.float16(float(s32))                    # numpy: RNE to binary16
    assert sbits.reshape(-1)[0] == np.array([s16]).view(np.uint16)[0]
    s = Fraction(float(s16))
    c = codes.view(np.int8)
    assert np.all(c[:, 0] == 127)
    # definition with exact rationals on a sample; numpy float32 division for all
    for x, code in list(zip(rows.reshape(-1), c.reshape(-1)))[::97]:
        y = _fl32(Fraction(float(x)) / s)
        assert code == max(-127, min(127, _round_half_even(y)))
    y = rows.astype(np.float32) / np.float32(float(s))
    assert np.array_equal(c, np.clip(np.rint(y), -127, 127).astype(np.int8))
    err = np.abs(rows.astype(np.float64) - c.astype(np.float64) * float(s))
    assert np.all(err <= float(s) / 2 * (1 + 2 ** -20))


def test_fp8_quantizer_error_bound_and_amax():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((2000, 128)).astype(np.float16).astype(np.float32)
    codes, sbits = oracle.quantize_rows(x, "e4m3")
    s = sbits.view(np.float16).astype(np.float64)
    deq = oracle.e4m3_to_f64(codes) * s[:, None]
    a = np.abs(x).max(axis=1)
    assert np.allclose(s, (a / np.float32(448)).astype(np.float16).astype(np.float64))
    # relative error of E4M3 nearest rounding <= 2^-4 for normals, plus the subnormal step
    err = np.abs(deq - x)
    bound = np.abs(x) * 2.0 ** -4 + s[:, None] * 2.0 ** -10 + 1e-12
    assert np.all(err <= bound)
    amax_codes = codes[np.arange(len(x)), np.abs(x).argmax(axis=1)]
    assert np.all((amax_codes & 0x7F) >= 0x7D)      # amax lands at the top of the range


def test_zero_row_gives_zero_codes():
    x = np.zeros((2, 64), np.float32)
    x[1, 3] = -0.0
    for kind in ("i8", "e4m3"):
        codes, s = oracle.quantize_rows(x, kind)
        assert np.all(codes == 0) and np.all(s == 0)
