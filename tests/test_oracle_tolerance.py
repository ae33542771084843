"""Pins of the parity tolerance's "1 fp16 ulp" term (reading xiv of the
page's float16 output): ``oracle.ulp16`` against numpy's own float16 spacing
for every finite float16, and ``oracle.check`` on hand-built results where the
ulp term, not the 1e-3 relative term, decides acceptance.

The relative term 1e-3 * sum|t| always exceeds about one ulp when the sum of
magnitudes is at least the result's magnitude and the result is a float16
normal (an ulp is at most 2^-10 of the value), so the cases that isolate the
ulp term are (a) results whose terms cancel, so sum|t| is tiny against one
ulp, (b) float16 subnormal results, and (c) a normal result where 1 + 1.024
ulps of tolerance separate 2 ulps off (accepted) from 3 (rejected)."""
import numpy as np
import pytest

import oracle

FINITE_BITS = np.array([b for b in range(1 << 16) if (b & 0x7C00) != 0x7C00], dtype=np.uint16)


def test_ulp16_equals_numpy_spacing_for_every_finite_float16():
    x = FINITE_BITS.view(np.float16)
    got = oracle.ulp16(x.astype(np.float64))
    mag = np.abs(x)
    with np.errstate(over="ignore"):
        want = np.abs(np.spacing(mag)).astype(np.float64)     # distance to the next float16 away from 0
    top = mag == np.float16(65504.0)
    # the largest finite value has no finite neighbour above it: its ulp is
    # the spacing of its binade, the distance to the value below it
    want[top] = 65504.0 - float(np.nextafter(np.float16(65504.0), np.float16(0.0)))
    assert np.array_equal(got, want)
    assert oracle.ulp16(np.array([0.0]))[0] == 2.0 ** -24
    assert oracle.ulp16(np.array([2.0 ** -14]))[0] == 2.0 ** -24        # smallest normal
    assert oracle.ulp16(np.array([2.0 ** -14 - 2.0 ** -24]))[0] == 2.0 ** -24
    assert oracle.ulp16(np.array([1.0, 1024.0, 2047.0, 2048.0]))[0] == 2.0 ** -10


def result(s_units: int, s_abs: float) -> oracle.Result:
    """A one-element oracle result with exact sum s_units * 2^-20 (its
    float16 bits by numpy's round-to-nearest-even cast) and the given sum of
    magnitudes."""
    S = s_units * 2.0 ** -20
    c = np.array([[np.float16(S).view(np.uint16)]], dtype=np.uint16)
    return oracle.Result(c=c, s_f64=np.array([[S]]), s_abs=np.array([[s_abs]]),
                         s_exact=np.array([[s_units]], dtype=np.int64), nan=np.zeros((1, 1), np.uint8))


def accepted(bits: int, ref: oracle.Result) -> bool:
    return bool(oracle.check(np.array([[bits]], dtype=np.uint16), ref)[0, 0])


def f16bits(v: float) -> int:
    return int(np.float16(v).view(np.uint16))


def test_ulp_term_decides_for_cancelling_terms():
    # two terms +-2^-20 cancel: S = 0, sum|t| = 2^-19, so 1e-3 * sum|t| is
    # about 2^-29, far below half of one float16 ulp at 0 (2^-24)
    ref = result(0, 2.0 ** -19)
    assert accepted(0x0000, ref) and accepted(0x8000, ref)
    assert accepted(0x0001, ref) and accepted(0x8001, ref)            # one ulp off
    assert not accepted(0x0002, ref) and not accepted(0x8002, ref)    # two ulps off


def test_ulp_term_decides_for_subnormal_results():
    # S = 2^-20 = 16 * 2^-24, a float16 subnormal; sum|t| = S
    ref = result(1, 2.0 ** -20)
    o = f16bits(2.0 ** -20)
    assert o == 16
    for d, ok in ((0, True), (1, True), (-1, True), (2, False), (-2, False)):
        assert accepted(o + d, ref) is ok, d
    # S = 5 * 2^-20 (80 * 2^-24), still subnormal
    ref = result(5, 5 * 2.0 ** -20)
    o = f16bits(5 * 2.0 ** -20)
    assert o == 80
    assert accepted(o + 1, ref) and accepted(o - 1, ref)
    assert not accepted(o + 2, ref) and not accepted(o - 2, ref)


@pytest.mark.parametrize("value,max_ok_ulps", [(1024.0, 2), (2047.0, 3), (1.0, 2), (-1536.0, 2)])
def test_ulp_term_at_normal_results(value, max_ok_ulps):
    # all terms of one sign: sum|t| = |S|; tolerance = 1e-3 |S| + ulp(o)
    units = int(value * 2 ** 20)
    ref = result(units, abs(value))
    ulp = float(oracle.ulp16(np.array([value]))[0])
    rel = 1e-3 * abs(value)
    assert max_ok_ulps * ulp <= rel + ulp < (max_ok_ulps + 1) * ulp
    for sgn in (1, -1):
        assert accepted(f16bits(value + sgn * max_ok_ulps * ulp), ref)
        assert not accepted(f16bits(value + sgn * (max_ok_ulps + 1) * ulp), ref)
