"""Pins for the oracle's global float32 scale alpha: c = fp16(alpha * sum) (CPU only).

NVFP4 pairs its per-16-element E4M3 scales with one float32 scale per tensor
(two-level scaling, described alongside the format in submission 69575); the
oracle applies it to the exact sum and rounds once. These pins hold it to:
  * alpha = 1 is the unscaled oracle, bit for bit,
  * alpha = -1 negates every output exactly, alpha = 0 zeroes it,
  * alpha = 2^k shifts the exact value (doubling, halving into subnormals,
    overflow to inf at the float16 edge),
  * brute force: exact rationals times a random float32 alpha, rounded once to
    float16 by a round-half-even routine written here from the float16 format
    (not numpy's cast, which would round twice through float64).
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from test_oracle_gemv import golden_e2m1, torch_e4m3


def fraction_to_fp16(x: Fraction) -> float:
    """Value of the float16 nearest to x (ties to even); +-inf past the edge."""
    if x == 0:
        return 0.0
    neg, ax = x < 0, abs(x)
    e = ax.numerator.bit_length() - ax.denominator.bit_length()
    if Fraction(2) ** e > ax:
        e -= 1
    while Fraction(2) ** (e + 1) <= ax:
        e += 1
    e = max(e, -14)                          # subnormals share the 2^-24 quantum
    q = Fraction(2) ** (e - 10)
    n, rem = divmod(ax, q)
    n = int(n)
    if rem * 2 > q or (rem * 2 == q and n % 2 == 1):
        n += 1
    v = n * q
    if v > 65504:
        return float("-inf") if neg else float("inf")
    return -float(v) if neg else float(v)


def exact_sums(inp):
    """Exact rational sums [L][M] from the golden value list and torch's float8 decode."""
    w = inp.w
    t2, t8 = golden_e2m1(), torch_e4m3()
    ac, bc = synth.unpack_nibbles(inp.a), synth.unpack_nibbles(inp.b)
    out = [[Fraction(0)] * w.M for _ in range(w.L)]
    for l in range(w.L):
        for m in range(w.M):
            s = Fraction(0)
            for k in range(w.K):
                s += (Fraction(t2[ac[l, m, k]]) * Fraction(t8[inp.sfa_plain[l, m, k // 16]])
                      * Fraction(t2[bc[l, k]]) * Fraction(t8[inp.sfb_plain[l, k // 16]]))
            out[l][m] = s
    return out


def test_fraction_to_fp16_matches_numpy_on_fp16_and_midpoints():
    # every finite float16 and every midpoint between neighbours: exact in
    # float64, so numpy's cast is a single rounding there
    vals = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = (vals[:-1] + vals[1:]) / 2
    for x in np.concatenate([vals[::97], mids[::89], mids[-3:], [65519.99, 65520.0]]):
        want = float(np.float16(x)) if x < 65520 else float("inf")
        assert fraction_to_fp16(Fraction(x)) == want, x
        assert fraction_to_fp16(-Fraction(x)) == -want, x


@pytest.mark.parametrize("layout", ["plain", "blocked"])
def test_alpha_one_is_unscaled(oracle_lib, layout):
    inp = synth.make_inputs(synth.Workload("a1", 127, 4096, 2, "edge", 7))
    r0 = oracle.gemv(inp, layout)
    r1 = oracle.gemv(inp, layout, alpha=1.0)
    np.testing.assert_array_equal(r1.c, r0.c)
    np.testing.assert_array_equal(r1.s_f64, r0.s_f64)
    np.testing.assert_array_equal(r1.s_abs, r0.s_abs)


def test_alpha_minus_one_negates(oracle_lib):
    inp = synth.make_inputs(synth.Workload("am1", 200, 2048, 3, "edge", 8))
    r = oracle.gemv(inp, "blocked")
    rn = oracle.gemv(inp, "blocked", alpha=-1.0)
    np.testing.assert_array_equal(rn.c, r.c ^ np.uint16(0x8000))
    np.testing.assert_array_equal(rn.s_exact, r.s_exact)       # unscaled
    np.testing.assert_array_equal(rn.s_f64, -r.s_f64)
    np.testing.assert_array_equal(rn.s_abs, r.s_abs)


def test_alpha_zero(oracle_lib):
    inp = synth.make_inputs(synth.Workload("a0", 64, 1024, 2, "uniform", 9))
    r = oracle.gemv(inp, "plain", alpha=0.0)
    assert np.all(r.value == 0) and np.all(r.s_abs == 0)


@pytest.mark.parametrize("k", [-30, -20, -9, -1, 1, 3, 12])
def test_alpha_power_of_two(oracle_lib, k):
    inp = synth.random_inputs(4, 64, 2, 50 + k, "edge")
    sums = exact_sums(inp)
    r = oracle.gemv(inp, "plain", alpha=2.0 ** k)
    for l in range(2):
        for m in range(4):
            assert r.value[l, m] == fraction_to_fp16(sums[l][m] * Fraction(2) ** k)


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_random_alpha(oracle_lib, seed):
    rng = np.random.default_rng(100 + seed)
    inp = synth.random_inputs(3, 64, 2, 40 + seed, "edge" if seed % 2 else "uniform")
    sums = exact_sums(inp)
    # float32 alphas with full 24-bit mantissas, spanning results that are
    # subnormal, normal and past the float16 edge
    alphas = np.float32(rng.uniform(1, 2, 6)) * np.float32(2.0) ** rng.integers(-40, 12, 6).astype(np.float32)
    alphas *= np.where(rng.random(6) < 0.5, -1, 1).astype(np.float32)
    for a in alphas:
        fa = Fraction(float(a))
        r = oracle.gemv(inp, "plain", alpha=float(a))
        for l in range(2):
            for m in range(3):
                assert r.value[l, m] == fraction_to_fp16(sums[l][m] * fa), (a, l, m)
                assert r.s_f64[l, m] == pytest.approx(float(sums[l][m] * fa), rel=1e-12, abs=1e-300)


def test_alpha_large_products_use_all_bits(oracle_lib):
    # |sum| near 2^49 in 2^-20 units times a 24-bit mantissa exceeds 64 bits:
    # the rounding must still see every bit (sticky), checked against rationals
    M, K = 2, 4096
    a = np.full((1, M, K), 7, np.uint8)               # e2m1 code 7 = 6.0
    a[0, 1, ::3] = 1                                  # 0.5: a sum with low bits set
    b = np.full((1, K), 7, np.uint8)
    sfa = np.full((1, M, K // 16), 0x7E, np.uint8)     # 448
    sfb = np.full((1, K // 16), 0x7E, np.uint8)
    sfb[0, 0] = 0x01                                  # smallest subnormal: 2^-9
    inp = synth.from_codes(a, b, sfa, sfb)
    sums = exact_sums(inp)
    for alpha in [np.float32(1.0000001), np.float32(3.3e-12), np.float32(-7.77e-9),
                  np.float32(16777215.0) * np.float32(2.0 ** -50)]:
        r = oracle.gemv(inp, "plain", alpha=float(alpha))
        for m in range(M):
            assert r.value[0, m] == fraction_to_fp16(sums[0][m] * Fraction(float(alpha))), (alpha, m)


def e4m3_pow2(p: int) -> int:
    """E4M3 code of 2^p, p in [-9, 8] (subnormals below 2^-6)."""
    return (p + 7) << 3 if p >= -6 else {-7: 0x04, -8: 0x02, -9: 0x01}[p]


E2M1_POW2 = {-1: 1, 0: 2, 1: 4, 2: 6}       # e2m1 codes of 0.5, 1, 2, 4


def one_row_with_sum(S: int):
    """Codes of a 1 x K x 1 problem whose exact sum is S * 2^-20: one nonzero
    element per 16-element block, one block per set bit of S."""
    terms = []
    for i in range(S.bit_length()):
        if S >> i & 1:
            e = i - 20
            terms += [20] * (1 << (e - 20)) if e > 20 else [e]
    K = -(-16 * len(terms) // 32) * 32
    a, b = np.zeros((1, 1, K), np.uint8), np.zeros((1, K), np.uint8)
    sfa, sfb = np.zeros((1, 1, K // 16), np.uint8), np.zeros((1, K // 16), np.uint8)
    for blk, e in enumerate(terms):
        y = max(-9, min(8, e))
        z = max(-9, min(8, e - y))
        x = max(-1, min(2, e - y - z))
        x2 = e - y - z - x
        assert -1 <= x2 <= 2
        a[0, 0, 16 * blk], b[0, 16 * blk] = E2M1_POW2[x], E2M1_POW2[x2]
        sfa[0, 0, blk], sfb[0, blk] = e4m3_pow2(y), e4m3_pow2(z)
    return synth.from_codes(a, b, sfa, sfb)


def sticky_case(top: int, tail: int):
    """(S, ma): S * ma has its top bit at ``top``, an even 11-bit float16
    significand, then exactly half an ulp, zeros, and ``tail`` in the bits the
    oracle folds into its sticky bit. Rounding that dropped those bits would
    see an exact tie and round down to even; the true value rounds up."""
    bpos = top - 10                              # lowest kept bit
    mod = 1 << bpos
    for ma in range((1 << 23) + 1, 1 << 24, 2):
        S = ((1 << (bpos - 1)) + tail) * pow(ma, -1, mod) % mod
        P = S * ma
        if P >> top == 1 and (P >> bpos) & 1 == 0:
            return S, ma
    raise AssertionError("no case found")


@pytest.mark.parametrize("top,tail", [(63, 1), (63, 3), (64, 5), (64, 7)])
def test_alpha_sticky_bits_decide_a_tie(oracle_lib, top, tail):
    S, ma = sticky_case(top, tail)
    inp = one_row_with_sum(S)
    r = oracle.gemv(inp, "plain", alpha=float(ma) * 2.0 ** -34)
    assert int(r.s_exact[0, 0]) == S
    want = fraction_to_fp16(Fraction(S * ma, 2 ** (20 + 34)))
    assert r.value[0, 0] == want
    # the rounded-down neighbour is what a dropped sticky bit gives
    assert want > fraction_to_fp16(Fraction(S * ma - tail, 2 ** (20 + 34)))


@pytest.mark.parametrize("bad", [float("inf"), float("-inf"), float("nan"), 1e39])
def test_rejects_non_finite_alpha(oracle_lib, bad):
    inp = synth.make_inputs(synth.TINY)
    with pytest.raises(ValueError):
        oracle.gemv(inp, "plain", alpha=bad)


def test_check_uses_scaled_values(oracle_lib):
    inp = synth.make_inputs(synth.Workload("ac", 96, 2048, 2, "uniform", 12))
    r = oracle.gemv(inp, "plain", alpha=0.37)
    assert oracle.check(r.c, r).all()
    unscaled = oracle.gemv(inp, "plain")
    # rows where forgetting alpha (a 0.63*|S| error) exceeds the tolerance
    big = 0.63 * np.abs(unscaled.value) > 2e-3 * unscaled.s_abs + 2 * oracle.ulp16(unscaled.value)
    assert big.sum() > 20
    assert not oracle.check(unscaled.c, r)[big].any()
