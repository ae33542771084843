"""Pins for the oracle's float16 round-to-nearest-even (bit-exact vs numpy).

numpy's float64 -> float16 cast is a correctly rounded IEEE conversion, so it
fixes every rounding decision, including ties, subnormals and overflow.
"""
import numpy as np

import oracle


def numpy_bits(x):
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def test_random_doubles(oracle_lib):
    rng = np.random.default_rng(1)
    x = rng.standard_normal(200000) * np.exp2(rng.uniform(-30, 20, 200000))
    np.testing.assert_array_equal(oracle.fp16_from_double(x), numpy_bits(x))


def test_all_midpoints_and_neighbours(oracle_lib):
    # every finite positive float16, the midpoints to the next one, and values
    # just off the midpoints
    h = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = (h[:-1] + h[1:]) / 2
    x = np.concatenate([h, mids, np.nextafter(mids, 0), np.nextafter(mids, np.inf)])
    x = np.concatenate([x, -x])
    np.testing.assert_array_equal(oracle.fp16_from_double(x), numpy_bits(x))


def test_overflow_edge(oracle_lib):
    x = np.array([65504.0, 65519.99, 65519.999999, 65520.0, 65520.0001, 65536.0, 1e30,
                  -65519.99, -65520.0, np.inf, -np.inf])
    got = oracle.fp16_from_double(x)
    np.testing.assert_array_equal(got, numpy_bits(x))
    assert got[3] == 0x7C00 and got[2] == 0x7BFF


def test_subnormals_and_zero(oracle_lib):
    x = np.concatenate([np.arange(0, 2048) * 2.0 ** -25, [2.0 ** -26, 3 * 2.0 ** -26, 0.0, -0.0, 2.0 ** -40]])
    np.testing.assert_array_equal(oracle.fp16_from_double(x), numpy_bits(x))


def test_scaled_integer_rounding(oracle_lib):
    # the path used for the exact sum: mag * 2^e2 with an integer mag
    rng = np.random.default_rng(2)
    for _ in range(20000):
        mag = int(rng.integers(1, 2 ** 52))
        e2 = int(rng.integers(-60, 20))
        neg = bool(rng.integers(0, 2))
        x = (-1.0 if neg else 1.0) * float(mag) * 2.0 ** e2   # exact: mag < 2^53
        assert oracle.fp16_round(neg, mag, e2) == int(numpy_bits(x)), (mag, e2, neg)
    # magnitudes beyond 2^53 (not representable in a double): keep the top 53
    # bits and fold every lower bit into the lowest kept one (a sticky bit);
    # float16 keeps only 11 bits, so this rounds the same as the full value
    for _ in range(2000):
        mag = int(rng.integers(2 ** 53, 2 ** 62))
        e2 = int(rng.integers(-80, -40))
        drop = mag.bit_length() - 53
        keep = (mag >> drop) | (1 if mag & ((1 << drop) - 1) else 0)
        x = float(keep) * 2.0 ** (e2 + drop)
        assert oracle.fp16_round(False, mag, e2) == int(numpy_bits(x)), (mag, e2)


def test_bits_to_double_roundtrip(oracle_lib):
    bits = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    vals = oracle.fp16_bits_to_double(bits)
    fin = np.isfinite(vals)
    np.testing.assert_array_equal(oracle.fp16_from_double(vals[fin]), bits[fin])
