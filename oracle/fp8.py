"""OCP FP8 e4m3 and bf16 number formats, written out from their definitions.

Test infrastructure (see ``oracle/__init__.py``): never imported by the product path.

The pages only say "FP8" (Blackwell 1,000 TPS/user blog, zh translation, the
paragraph on FP8 data types for GEMM, MoE and attention).  The variant used here is
the OCP 8-bit floating point e4m3 format ("e4m3fn"): 1 sign bit, 4 exponent bits
with bias 7, 3 mantissa bits, subnormals, no infinities, NaN only at S.1111.111
(0x7F and 0xFF), largest finite magnitude 1.75 * 2**8 = 448.  This format, and
saturating round-to-nearest-even for the encoder, are readings: the pages fix neither.

Pinned by ``tests/test_oracle_fp8.py`` (torch's float8_e4m3fn and bfloat16 casts,
spot values of the format, exhaustive round trips and brute-force nearest-code
search).
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E4M3_MAX_CODE = 0x7E


def _decode_one(code: int) -> float:
    """Value of one e4m3 code from its bit fields (closed form of the format)."""
    sign = -1.0 if (code >> 7) & 1 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        # subnormal: 0.mmm * 2**(1 - 7) = mmm * 2**-9
        return sign * man * 2.0 ** -9
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


# Value of every code, float64.  Built once from the closed form above.
DECODE_TABLE = np.array([_decode_one(c) for c in range(256)], dtype=np.float64)

# Magnitudes of the non-negative finite codes 0x00..0x7E, strictly increasing in the
# code (the format is sign-magnitude with the exponent above the mantissa).
_POS = DECODE_TABLE[: E4M3_MAX_CODE + 1].copy()
# Midpoint between code c and code c+1, exact in float64 (short mantissas).
_MID = (_POS[:-1] + _POS[1:]) / 2.0


def e4m3_decode(codes) -> np.ndarray:
    """Decode uint8 e4m3 codes to float64 (NaN for 0x7F/0xFF, -0.0 for 0x80)."""
    codes = np.asarray(codes, dtype=np.uint8)
    return DECODE_TABLE[codes]


def e4m3_encode(values) -> np.ndarray:
    """Encode float64 values to e4m3 codes.

    Round to the nearest representable magnitude; on an exact tie take the code
    whose mantissa LSB is 0 (round half to even).  Magnitudes at or above 448
    saturate to 448 (0x7E).  The sign bit follows the sign of the input, also when
    the magnitude rounds to zero (so -1e-9 encodes to 0x80).  NaN maps to 0x7F;
    the step never produces NaN inputs.
    """
    v = np.asarray(values, dtype=np.float64)
    a = np.abs(v)
    # idx = number of midpoints strictly below a  -> nearest code unless a is a tie
    idx = np.searchsorted(_MID, a, side="left")  # first midpoint >= a
    code = idx.astype(np.int64)
    # a == _MID[idx]: exact tie between codes idx and idx+1 -> pick the even one
    in_range = idx < _MID.size
    tie = np.zeros(a.shape, dtype=bool)
    tie[in_range] = a[in_range] == _MID[idx[in_range]]
    code = np.where(tie & (code % 2 == 1), code + 1, code)
    code = np.where(a >= E4M3_MAX, E4M3_MAX_CODE, code)
    code = np.where(np.isnan(a), 0x7F, code)
    neg = np.signbit(v) & ~np.isnan(v)
    code = np.where(neg, code | 0x80, code)
    return code.astype(np.uint8)


def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) to float64: they are the top half of a float32."""
    bits = np.asarray(bits, dtype=np.uint16)
    f32 = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return f32.astype(np.float64)


def f64_to_bf16(values) -> np.ndarray:
    """Round float64 values to bf16 (8 significant bits), half to even, one rounding.

    Only normal, finite results are produced by the step; zeros keep their sign.
    """
    v = np.asarray(values, dtype=np.float64)
    m, e = np.frexp(v)  # v = m * 2**e with 0.5 <= |m| < 1
    # 8 significant bits: scale the mantissa to [128, 256) and round half to even.
    r = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)
    f32 = r.astype(np.float32)  # exact: r has 8 significant bits
    return (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def fp32_round(values) -> np.ndarray:
    """Round float64 values to the nearest float32 (half to even), back to float64."""
    return np.asarray(values, dtype=np.float64).astype(np.float32).astype(np.float64)
