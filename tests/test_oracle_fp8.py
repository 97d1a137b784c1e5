"""Pins for ``oracle.fp8`` against things other than the oracle itself.

* torch's float8_e4m3fn and bfloat16 casts (library routines);
* spot values fixed by the OCP e4m3 format (bias 7, largest finite 448, NaN at
  S.1111.111, subnormal step 2**-9);
* exhaustive round trips and brute-force nearest-code search.
"""

import math

import numpy as np
import pytest
import torch

from oracle import fp8, loops


def torch_decode_all():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def torch_encode(v):
    return torch.from_numpy(np.asarray(v, np.float64)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_matches_torch_all_codes():
    ours = fp8.e4m3_decode(np.arange(256, dtype=np.uint8))
    ref = torch_decode_all()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
    (0x38, 1.0), (0x39, 1.125), (0x3F, 1.875), (0x40, 2.0), (0x7E, 448.0),
    (0x7D, 416.0), (0xB8, -1.0), (0xFE, -448.0), (0x81, -(2.0 ** -9)),
])
def test_decode_spot_values(code, value):
    assert fp8.e4m3_decode(np.uint8(code)) == value


def test_decode_special_codes():
    v = fp8.e4m3_decode(np.array([0x7F, 0xFF, 0x80], np.uint8))
    assert math.isnan(v[0]) and math.isnan(v[1])
    assert v[2] == 0.0 and np.signbit(v[2])
    # the positive finite codes increase strictly, so the format has 126 positive values
    pos = fp8.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)


def test_loop_decoder_agrees_with_table():
    for c in range(256):
        a, b = loops.dec(c), float(fp8.e4m3_decode(np.uint8(c)))
        assert (math.isnan(a) and math.isnan(b)) or a == b


def test_encode_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    back = fp8.e4m3_encode(fp8.e4m3_decode(codes))
    assert np.array_equal(back, codes)


@pytest.mark.parametrize("value,code", [
    (1.0625, 0x38),      # halfway 1 .. 1.125 -> even mantissa (1.0)
    (1.1875, 0x3A),      # halfway 1.125 .. 1.25 -> even (1.25)
    (2.0 ** -10, 0x00),  # halfway 0 .. 2**-9 -> even (0)
    (3 * 2.0 ** -10, 0x02),  # halfway 2**-9 .. 2**-8 -> even
    (432.0, 0x7E),       # halfway 416 .. 448 -> even (448, mantissa 110)
    (448.0 * (1 + 2.0 ** -23), 0x7E),
    (463.9, 0x7E), (464.0, 0x7E), (1.0e6, 0x7E), (-1.0e6, 0xFE),  # saturation
    (-1e-9, 0x80), (-0.0, 0x80), (0.0, 0x00),
])
def test_encode_spot_values(value, code):
    assert int(fp8.e4m3_encode(np.float64(value))) == code


def test_encode_matches_torch_on_ties_and_random():
    # torch converts float64 -> float32 -> e4m3, so feed it float32 values only (the
    # first step is then exact); near-tie float64 inputs are covered by the brute
    # force test below.
    pos = fp8.e4m3_decode(np.arange(0x7F, dtype=np.uint8)).astype(np.float32)
    mids = (pos[:-1] + pos[1:]) / np.float32(2)
    rng = np.random.default_rng(7)
    vals = np.concatenate([
        mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9)), pos,
        rng.uniform(-448, 448, 20000).astype(np.float32),
        rng.normal(0, 1, 20000).astype(np.float32),
        rng.uniform(-2.0 ** -6, 2.0 ** -6, 5000).astype(np.float32),  # subnormal range
        rng.uniform(440, 463.99, 2000).astype(np.float32),
    ]).astype(np.float64)
    vals = np.concatenate([vals, -vals])
    assert np.array_equal(fp8.e4m3_encode(vals), torch_encode(vals))


def test_encode_single_rounding_from_float64():
    # just below a midpoint in float64 must round down (no detour through float32)
    pos = fp8.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2
    below = fp8.e4m3_encode(np.nextafter(mids, 0))
    above = fp8.e4m3_encode(np.nextafter(mids, 1e9))
    assert np.array_equal(below, np.arange(0, 0x7E, dtype=np.uint8))
    assert np.array_equal(above, np.arange(1, 0x7F, dtype=np.uint8))


def test_encode_is_nearest_code_brute_force():
    pos = fp8.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    rng = np.random.default_rng(3)
    vals = np.concatenate([rng.uniform(0, 448, 3000), rng.uniform(0, 0.05, 1000)])
    codes = fp8.e4m3_encode(vals)
    for v, c in zip(vals, codes):
        d = np.abs(pos - v)
        assert d[c] == d.min()
        if (d == d.min()).sum() > 1:
            assert c % 2 == 0
        assert loops.enc(float(v)) == c


def test_bf16_decode_and_round_match_torch():
    rng = np.random.default_rng(11)
    f32 = np.concatenate([rng.normal(0, 1, 50000), rng.normal(0, 1e3, 5000),
                          rng.uniform(-1e-30, 1e-30, 1000)]).astype(np.float32)
    ours = fp8.f64_to_bf16(f32.astype(np.float64))
    ref = torch.from_numpy(f32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = fp8.bf16_to_f64(ref)
    assert np.array_equal(back, torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16)
                          .to(torch.float64).numpy())


def test_bf16_round_half_even_in_double():
    # x = b + half_ulp exactly (not representable in float32 rounding first)
    base = np.array([1.0, 1.0078125, 3.0, -5.25, 1000.0])
    ulp = np.ldexp(1.0, np.frexp(np.abs(base))[1] - 8)
    tie = base + np.sign(base) * ulp / 2
    got = fp8.bf16_to_f64(fp8.f64_to_bf16(tie))
    for b, u, g in zip(base, ulp, got):
        lo, hi = b, b + np.sign(b) * u
        even = lo if (int(abs(lo) / u) % 2 == 0) else hi
        assert g == even
    # just above a tie rounds away, just below rounds toward
    assert fp8.bf16_to_f64(fp8.f64_to_bf16(np.nextafter(1.00390625, 2)))[()] == 1.0078125
    assert fp8.bf16_to_f64(fp8.f64_to_bf16(np.nextafter(1.00390625, 0)))[()] == 1.0
    # agrees with the Fraction-based rounding of the loop version
    rng = np.random.default_rng(5)
    vals = rng.normal(0, 10, 2000)
    for v, b in zip(vals, fp8.f64_to_bf16(vals)):
        assert loops.float_to_bf16_bits(float(v)) == int(b)


def test_scale_rounding_equals_float32_division_for_all_bf16():
    # every positive finite bf16 value as an amax
    b = np.arange(0x0001, 0x7F80, dtype=np.uint32)
    amax = (b << 16).view(np.float32)
    ours = fp8.fp32_round(amax.astype(np.float64) / 448.0)
    ieee = (amax / np.float32(448.0)).astype(np.float64)
    assert np.array_equal(ours, ieee)
