"""Pins for the oracle's E2M1 and E4M3 decode (bit-exact).

Each table is checked against something other than its own formula:
  * the golden value lists (format definitions, cited in the fixtures),
  * torch's float8_e4m3fn decode (a library routine) for all 256 E4M3 codes,
  * numpy's float16 decode of an independent bit construction for E2M1.
"""
import json
import os

import numpy as np
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_e2m1_matches_format_value_list(oracle_lib):
    golden = json.load(open(os.path.join(GOLDEN, "e2m1_values.json")))["codes_to_values"]
    t2, _ = oracle.tables()
    for code_s, val in golden.items():
        code = int(code_s)
        assert t2[code] == val, (code, t2[code], val)
        # signed zero: code 8 is -0
        assert np.signbit(t2[code]) == np.signbit(val), code
        assert oracle.e2m1(code) == val


def test_e2m1_matches_fp16_bit_construction(oracle_lib):
    # Independent derivation: placing the 3 magnitude bits of an E2M1 code at
    # float16 bits 11..9 and its sign at bit 15 yields exactly e2m1 * 2^-14
    # (the exponent fields line up, E2M1 bias 1 vs float16 bias 15).
    t2, _ = oracle.tables()
    codes = np.arange(16, dtype=np.uint16)
    bits = ((codes & 7) << 9) | ((codes & 8) << 12)
    vals = bits.astype(np.uint16).view(np.float16).astype(np.float64) * 2.0 ** 14
    np.testing.assert_array_equal(vals, t2)
    np.testing.assert_array_equal(np.signbit(vals), np.signbit(t2))


def test_e4m3_matches_torch_decode_all_codes(oracle_lib):
    _, t8 = oracle.tables()
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    ref = ref.to(torch.float64).numpy()
    nan = np.isnan(ref)
    np.testing.assert_array_equal(np.isnan(t8), nan)
    np.testing.assert_array_equal(t8[~nan], ref[~nan])
    np.testing.assert_array_equal(np.signbit(t8[~nan]), np.signbit(ref[~nan]))


def test_e4m3_landmarks(oracle_lib):
    g = json.load(open(os.path.join(GOLDEN, "e4m3_landmarks.json")))
    for code_s, val in g["values"].items():
        v = oracle.e4m3(int(code_s, 16))
        assert v == val and np.signbit(v) == np.signbit(val), (code_s, v, val)
    for code_s in g["nan_codes"]:
        assert np.isnan(oracle.e4m3(int(code_s, 16)))
    # exactly two NaN codes, no infinities
    _, t8 = oracle.tables()
    assert np.isnan(t8).sum() == 2
    assert not np.isinf(t8).any()
    assert np.nanmax(t8) == 448.0 and np.nanmin(t8) == -448.0


def test_e4m3_monotone_positive_half(oracle_lib):
    # codes 0x00..0x7E are increasing (a sign-magnitude format)
    _, t8 = oracle.tables()
    pos = t8[:0x7F]
    assert np.all(np.diff(pos) > 0)
    np.testing.assert_array_equal(t8[0x80:0xFF], -pos)
