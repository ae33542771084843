"""Pins for the oracle's GEMV (CPU only).

  * hand-computed cases (tests/golden/hand_cases.json, with derivations),
  * brute force with exact rationals on tiny inputs (Python Fractions, decode
    from the golden value list and torch's float8 decode),
  * reduction to a library routine: numpy's float64 matrix-vector product of
    the dequantised operands, exact for scales drawn as 2^U[-3,3],
  * the exact int64 sum against the plain fp64 sum,
  * invariants: zero scales, sign flip, scale doubling, block permutation,
    plain vs blocked scales, batch-slice independence, thread count.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden_e2m1():
    g = json.load(open(os.path.join(GOLDEN, "e2m1_values.json")))["codes_to_values"]
    return np.array([g[str(i)] for i in range(16)], dtype=np.float64)


def torch_e4m3():
    t = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def dequant(inp):
    """Dequantised A [L][M][K] and b [L][K] in float64, decoded without the oracle."""
    w = inp.w
    t2, t8 = golden_e2m1(), torch_e4m3()
    a = t2[synth.unpack_nibbles(inp.a)] * np.repeat(t8[inp.sfa_plain], 16, axis=-1)
    b = t2[synth.unpack_nibbles(inp.b)] * np.repeat(t8[inp.sfb_plain], 16, axis=-1)
    return a.reshape(w.L, w.M, w.K), b.reshape(w.L, w.K)


SMALL = [synth.TINY,
         synth.Workload("small_balanced", 256, 2048, 4, "uniform", 1),
         synth.Workload("small_batched", 128, 7168, 3, "uniform", 2),
         synth.Workload("small_headline", 64, 16384, 1, "uniform", 3),
         synth.Workload("small_edge", 127, 4096, 3, "edge", 4),
         synth.Workload("small_edge_k64", 1000, 64, 3, "edge", 4)]


# ---------------------------------------------------------------- hand cases

def hand_inputs(case):
    a = np.array(case["a_codes"], np.uint8).reshape(1, 1, 32)
    b = np.array(case["b_codes"], np.uint8).reshape(1, 32)
    sfa = np.array(case["sfa"], np.uint8).reshape(1, 1, 2)
    sfb = np.array(case["sfb"], np.uint8).reshape(1, 2)
    return synth.from_codes(a, b, sfa, sfb, name=case["name"])


HAND = json.load(open(os.path.join(GOLDEN, "hand_cases.json")))["cases"]


@pytest.mark.parametrize("case", HAND, ids=[c["name"] for c in HAND])
@pytest.mark.parametrize("layout", ["plain", "blocked"])
def test_hand_cases(oracle_lib, case, layout):
    r = oracle.gemv(hand_inputs(case), layout)
    assert Fraction(int(r.s_exact[0, 0]), 2 ** 20) == Fraction(case["exact_sum"])
    assert r.value[0, 0] == float(case["fp16"])


# ---------------------------------------------------------------- brute force

@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("dist", ["uniform", "edge"])
def test_brute_force_fractions(oracle_lib, seed, dist):
    inp = synth.random_inputs(3, 64, 2, seed, dist)
    t2, t8 = golden_e2m1(), torch_e4m3()
    ac = synth.unpack_nibbles(inp.a)
    bc = synth.unpack_nibbles(inp.b)
    r = oracle.gemv(inp, "plain")
    for l in range(2):
        for m in range(3):
            s = Fraction(0)
            for k in range(64):
                s += (Fraction(t2[ac[l, m, k]]) * Fraction(t8[inp.sfa_plain[l, m, k // 16]])
                      * Fraction(t2[bc[l, k]]) * Fraction(t8[inp.sfb_plain[l, k // 16]]))
            assert Fraction(int(r.s_exact[l, m]), 2 ** 20) == s
            # and the once-rounded fp16 value is numpy's rounding of it
            with np.errstate(over="ignore"):
                want = np.float16(float(s))
            assert r.value[l, m] == float(want)


# ---------------------------------------------------------------- library reduction

@pytest.mark.parametrize("w", SMALL[:4], ids=lambda w: w.name)
def test_matches_numpy_matvec(oracle_lib, w):
    # With scales in [1/8, 8] every partial sum is a multiple of 2^-14 below
    # 2^26, so float64 matrix-vector products are exact.
    inp = synth.make_inputs(w)
    A, b = dequant(inp)
    r = oracle.gemv(inp, "plain")
    for l in range(w.L):
        S = A[l] @ b[l]
        np.testing.assert_array_equal(r.s_exact[l].astype(np.float64) * 2.0 ** -20, S)
        with np.errstate(over="ignore"):
            np.testing.assert_array_equal(r.c[l], S.astype(np.float16).view(np.uint16))


def test_sabs_matches_numpy(oracle_lib):
    inp = synth.make_inputs(SMALL[1])
    A, b = dequant(inp)
    r = oracle.gemv(inp, "plain")
    for l in range(inp.w.L):
        np.testing.assert_allclose(r.s_abs[l], np.abs(A[l]) @ np.abs(b[l]), rtol=1e-12)


# ---------------------------------------------------------------- twins

@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_exact_and_fp64_agree(oracle_lib, w):
    inp = synth.make_inputs(w)
    r = oracle.gemv(inp, "blocked")
    with np.errstate(over="ignore"):
        from_f64 = r.s_f64.astype(np.float16).view(np.uint16)
    np.testing.assert_array_equal(r.c, from_f64)
    assert not r.nan.any()


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_plain_equals_blocked(oracle_lib, w):
    inp = synth.make_inputs(w)
    rp = oracle.gemv(inp, "plain")
    rb = oracle.gemv(inp, "blocked")
    np.testing.assert_array_equal(rp.c, rb.c)
    np.testing.assert_array_equal(rp.s_exact, rb.s_exact)


def test_thread_count_independent(oracle_lib):
    inp = synth.make_inputs(SMALL[4])
    r1 = oracle.gemv(inp, "blocked", nthreads=1)
    r7 = oracle.gemv(inp, "blocked", nthreads=7)
    np.testing.assert_array_equal(r1.c, r7.c)
    np.testing.assert_array_equal(r1.s_exact, r7.s_exact)
    np.testing.assert_array_equal(r1.s_abs, r7.s_abs)


def test_rows_subset_matches_full(oracle_lib):
    inp = synth.make_inputs(SMALL[4])
    full = oracle.gemv(inp, "blocked")
    rows = np.array([0, 5, 126, 127, 200, 380], np.int64)
    sub = oracle.gemv_rows(inp, rows, "blocked")
    np.testing.assert_array_equal(sub.c, full.c.reshape(-1)[rows])
    np.testing.assert_array_equal(sub.s_exact, full.s_exact.reshape(-1)[rows])


# ---------------------------------------------------------------- invariants

def test_zero_scales_give_zero(oracle_lib):
    inp = synth.make_inputs(SMALL[1])
    z = synth.from_codes(synth.unpack_nibbles(inp.a), synth.unpack_nibbles(inp.b),
                         np.zeros_like(inp.sfa_plain), inp.sfb_plain)
    r = oracle.gemv(z, "blocked")
    assert np.all(r.s_exact == 0) and np.all(r.value == 0)


def test_sign_flip_negates_exactly(oracle_lib):
    inp = synth.make_inputs(SMALL[4])
    r = oracle.gemv(inp, "plain")
    flipped = synth.Inputs(inp.w, inp.a ^ np.uint8(0x88), inp.b, inp.sfa_plain,
                           inp.sfb_plain, inp.sfa_blocked, inp.sfb_blocked)
    rf = oracle.gemv(flipped, "plain")
    np.testing.assert_array_equal(rf.s_exact, -r.s_exact)
    np.testing.assert_array_equal(rf.value, -r.value)


def test_scale_doubling(oracle_lib):
    # +8 on an E4M3 code with exponent field 1..13 doubles its value exactly
    inp = synth.make_inputs(SMALL[1])
    e = (inp.sfa_plain >> 3) & 15
    assert np.all((e >= 1) & (e <= 13))
    doubled = synth.from_codes(synth.unpack_nibbles(inp.a), synth.unpack_nibbles(inp.b),
                               inp.sfa_plain + np.uint8(8), inp.sfb_plain)
    r = oracle.gemv(inp, "plain")
    r2 = oracle.gemv(doubled, "blocked")
    np.testing.assert_array_equal(r2.s_exact, 2 * r.s_exact)
    fin = np.abs(r.value) < 32000
    np.testing.assert_array_equal(r2.value[fin], 2 * r.value[fin])


def test_block_permutation_invariance(oracle_lib):
    inp = synth.make_inputs(SMALL[2])
    w = inp.w
    nkb = w.K // 16
    perm = np.random.default_rng(5).permutation(nkb)
    ac = synth.unpack_nibbles(inp.a).reshape(w.L, w.M, nkb, 16)[:, :, perm].reshape(w.L, w.M, w.K)
    bc = synth.unpack_nibbles(inp.b).reshape(w.L, nkb, 16)[:, perm].reshape(w.L, w.K)
    p = synth.from_codes(ac, bc, inp.sfa_plain[:, :, perm], inp.sfb_plain[:, perm])
    np.testing.assert_array_equal(oracle.gemv(p, "blocked").s_exact, oracle.gemv(inp, "plain").s_exact)


def test_batch_slices_independent(oracle_lib):
    inp = synth.make_inputs(SMALL[4])
    full = oracle.gemv(inp, "blocked")
    for l in range(inp.w.L):
        one = synth.from_codes(synth.unpack_nibbles(inp.a[l:l + 1]), synth.unpack_nibbles(inp.b[l:l + 1]),
                               inp.sfa_plain[l:l + 1], inp.sfb_plain[l:l + 1])
        np.testing.assert_array_equal(oracle.gemv(one, "blocked").c[0], full.c[l])


def test_nan_scale_propagates(oracle_lib):
    case = HAND[0]
    inp = hand_inputs(dict(case, sfa=[0x7F, 0x38]))
    r = oracle.gemv(inp, "plain")
    assert r.nan[0, 0] == 1 and np.isnan(r.value[0, 0])


def test_rejects_bad_shapes(oracle_lib):
    inp = synth.make_inputs(synth.TINY)
    with pytest.raises(ValueError):
        oracle.gemv_arrays(inp.a, inp.b, inp.sfa_plain, inp.sfb_plain, 128, 255, 1, "plain")
    with pytest.raises(ValueError):
        oracle.gemv_arrays(inp.a, inp.b, inp.sfa_plain, inp.sfb_plain, 128, 256, 1, "blocked")


# ---------------------------------------------------------------- the tolerance check

def test_check_accepts_oracle_and_rejects_perturbations(oracle_lib):
    inp = synth.make_inputs(SMALL[1])
    r = oracle.gemv(inp, "plain")
    assert oracle.check(r.c, r).all()
    # tolerance is 1e-3 * s_abs + 1 ulp: move one output far outside it
    bad = r.c.copy()
    v = r.value[0, 3]
    bad[0, 3] = np.float16(v + 0.01 * r.s_abs[0, 3] + 1.0).view(np.uint16)
    ok = oracle.check(bad, r)
    assert not ok[0, 3] and ok.sum() == ok.size - 1
    # one ulp off is accepted
    near = r.c.copy()
    near[0, 4] = near[0, 4] + 1 if near[0, 4] not in (0x7BFF, 0xFBFF) else near[0, 4] - 1
    assert oracle.check(near, r)[0, 4]
    # NaN where the oracle is finite is rejected
    nan = r.c.copy()
    nan[1, 0] = 0x7E00
    assert not oracle.check(nan, r)[1, 0]


def test_check_overflow_edge(oracle_lib):
    def res(S_units, s_abs, c_bits):
        return oracle.Result(np.array([[c_bits]], np.uint16), np.array([[S_units * 2.0 ** -20]]),
                             np.array([[s_abs]]), np.array([[S_units]], np.int64), np.zeros((1, 1), np.uint8))
    inf, big = 0x7C00, 0x7BFF
    # S just above 65520 with a large s_abs: finite 65504 and inf both fine
    r = res(int(65521 * 2 ** 20), 1e6, inf)
    assert oracle.check(np.array([[inf]], np.uint16), r)[0, 0]
    assert oracle.check(np.array([[big]], np.uint16), r)[0, 0]
    assert not oracle.check(np.array([[0xFC00]], np.uint16), r)[0, 0]   # wrong sign
    # far above the edge with a small s_abs: only inf
    r = res(int(80000 * 2 ** 20), 100.0, inf)
    assert oracle.check(np.array([[inf]], np.uint16), r)[0, 0]
    assert not oracle.check(np.array([[big]], np.uint16), r)[0, 0]
