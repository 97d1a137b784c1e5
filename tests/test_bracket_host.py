"""The quantisers' brackets (fp8_moe_ffn_amd/csrc/codec.hpp), replayed in float32 on the
CPU against the oracle: the activation quantiser's one-end rule (e4m3_quant4_bf16_end /
_even) over every bf16 value, and the general fast path's two ends (e4m3_quant2_fast) on
sampled float32 values and planted rounding midpoints.

The kernel codes a bf16 row over its scale s = fp32(amax / 448) from products with a
moved reciprocal: fp32(v * rhi) when amax > 448 s, fp32(v * rlo) when amax < 448 s, and
the even code of the two where amax = 448 s, with rhi / rlo = fp32(fp32(1 / s) * (1 +- 2^-21)).
Here numpy's float32 arithmetic (IEEE, round to nearest even) stands in for the GPU's, and
the oracle's e4m3 encoder for the hardware conversion (round to nearest even; the products
never reach the saturation range).  Every finite bf16 value v with |v| <= amax is checked,
for maxima of every significand at several exponents (among them the rows whose scale is
exact), against ``oracle.ffn.quantize_rows``, whose quotient is taken in float64.
"""

import numpy as np
import pytest

from oracle import ffn, fp8

KLO = np.float32(1.0 - 2.0**-21)
KHI = np.float32(1.0 + 2.0**-21)


def all_finite_bf16() -> np.ndarray:
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = ((bits >> 7) & 0xFF) != 0xFF
    return fp8.bf16_to_f64(bits[finite])


def kernel_codes(v: np.ndarray, amax: float):
    """Codes of the bf16 values v of a row whose largest magnitude is amax (> 0)."""
    s = np.float32(amax) / np.float32(448.0)  # IEEE float32 division
    direction = np.sign(np.float64(amax) - 448.0 * np.float64(s))  # exact in float64
    rs = np.float32(1.0) / s
    v32 = v.astype(np.float32)
    lo = fp8.e4m3_encode((v32 * np.float32(rs * KLO)).astype(np.float64))
    hi = fp8.e4m3_encode((v32 * np.float32(rs * KHI)).astype(np.float64))
    if direction > 0:
        return hi, s, direction
    if direction < 0:
        return lo, s, direction
    return np.where((lo & 1) == 1, hi, lo), s, direction


ALL = all_finite_bf16()
# the maxima: every bf16 significand at a few exponents, and the extremes of the range that
# takes this path (s >= 2^-96)
MAXIMA = [m / 128.0 * 2.0**e for e in (-5, 0, 3) for m in range(128, 256)] + [2.0**-80 * 1.5, 2.0**120 * 1.25]


@pytest.mark.parametrize("chunk", range(4))
def test_one_end_codes_equal_the_oracle_for_every_bf16_value(chunk):
    seen = set()
    for amax in MAXIMA[chunk::4]:
        v = ALL[np.abs(ALL) <= amax]
        v = np.concatenate([v, [amax]])  # the row's maximum is amax
        got, s, direction = kernel_codes(v, amax)
        want, s_or = ffn.quantize_rows(v[None, :])
        assert np.float64(s) == s_or[0], amax
        bad = np.nonzero(got != want[0])[0]
        assert bad.size == 0, (amax, v[bad[:5]], got[bad[:5]], want[0][bad[:5]])
        seen.add(int(direction))
    assert seen >= {-1, 1}  # both one-end cases in every chunk of maxima


def test_rows_with_an_exact_scale_take_the_even_code():
    """amax = 448 s exactly (the significand of amax a multiple of 7): ties of the ideal
    ratio land exactly on a midpoint, where only the even rule gives the oracle's code."""
    exact = [a for a in MAXIMA if float(np.float32(a) / np.float32(448.0)) * 448.0 == a]
    assert len(exact) >= 10
    for amax in exact:
        v = np.concatenate([ALL[np.abs(ALL) <= amax], [amax]])
        got, _, direction = kernel_codes(v, amax)
        assert direction == 0
        assert np.array_equal(got, ffn.quantize_rows(v[None, :])[0][0]), amax


def test_a_narrower_or_one_sided_rule_fails():
    """The pin has teeth: taking the upper end on every row (ignoring the direction) or
    the plain product without the moved reciprocal gives codes the oracle does not."""
    wrong_dir = 0
    plain = 0
    for amax in MAXIMA[:128]:
        v = np.concatenate([ALL[np.abs(ALL) <= amax], [amax]])
        want = ffn.quantize_rows(v[None, :])[0][0]
        s = np.float32(amax) / np.float32(448.0)
        rs = np.float32(1.0) / s
        v32 = v.astype(np.float32)
        up = fp8.e4m3_encode((v32 * np.float32(rs * KHI)).astype(np.float64))
        wrong_dir += int(np.count_nonzero(up != want))
        plain += int(np.count_nonzero(fp8.e4m3_encode((v32 * rs).astype(np.float64)) != want))
    assert wrong_dir > 0 and plain > 0


def test_fast_bracket_contains_the_exact_quotient():
    """The general fast path (e4m3_quant2_fast): for float32 values over float32 scales, the
    ends fp32(v * fp32(r (1 -+ 2^-21))) lie on either side of the float64 quotient, and where
    their codes agree that is the oracle's code of the quotient; where they differ (a
    midpoint inside, the exact path's case) they are adjacent codes."""
    rng = np.random.default_rng(7)
    n = 300_000
    s = np.exp2(rng.uniform(-90.0, 20.0, 2 * n)).astype(np.float32)  # s >= 2^-96: the fast path's range
    # values of dynamic-scale rows (|v| <= 448 s), then values whose quotient is a rounding
    # midpoint of e4m3 up to the rounding of v (the exact path's case)
    mids = np.array([(fp8.e4m3_decode(np.uint8(c)) + fp8.e4m3_decode(np.uint8(c + 1))) / 2 for c in range(0x7E)])
    u = np.concatenate([rng.uniform(-1.0, 1.0, n) * 448.0, rng.choice(mids, n) * rng.choice([-1.0, 1.0], n)])
    v = (u * s.astype(np.float64)).astype(np.float32)
    r = np.float32(1.0) / s
    lo = v * (r * KLO).astype(np.float32)
    hi = v * (r * KHI).astype(np.float32)
    q = v.astype(np.float64) / s.astype(np.float64)
    live = (np.abs(q) >= 2.0**-126) & (q != 0)
    a, b = np.minimum(lo, hi).astype(np.float64), np.maximum(lo, hi).astype(np.float64)
    assert np.all((a < q)[live]) and np.all((q < b)[live])
    clo, chi, want = fp8.e4m3_encode(lo.astype(np.float64)), fp8.e4m3_encode(hi.astype(np.float64)), fp8.e4m3_encode(q)
    agree = clo == chi
    assert np.array_equal(clo[agree], want[agree])
    diff = ~agree
    assert np.all(np.abs((clo[diff] & 0x7F).astype(int) - (chi[diff] & 0x7F).astype(int)) == 1)
    assert np.count_nonzero(diff[:n]) < n // 1000  # rare for ordinary values
    assert np.count_nonzero(diff[n:]) > n // 2  # the planted midpoints reach the exact path
