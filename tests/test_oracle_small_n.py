"""Pins for the oracle of the N-vector skinny GEMM (CPU only). Its definition
is N independent GEMVs, one per right-hand vector, so the pins check the
assembly: N = 1 is the GEMV oracle; column n is the GEMV against vector n;
permuting the vectors permutes the columns; a zero vector gives a zero column;
a brute-force rational sum on a tiny case."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from test_oracle_gemv import golden_e2m1, torch_e4m3


def inputs(M, N, K, L, seed):
    rng = np.random.default_rng(seed)
    a = synth.pack_nibbles(rng.integers(0, 16, (L, M, K), dtype=np.uint8))
    b = synth.pack_nibbles(rng.integers(0, 16, (L, N, K), dtype=np.uint8))
    sfa = synth.scale_codes(rng, (L, M, K // 16))
    sfb = synth.scale_codes(rng, (L, N, K // 16))
    return a, b, sfa, sfb


def test_n1_is_the_gemv(oracle_lib):
    inp = synth.random_inputs(100, 2048, 2, seed=4)
    r = oracle.gemm_small_n(inp.a, inp.b.reshape(2, 1, -1), inp.sfa_plain, inp.sfb_plain.reshape(2, 1, -1),
                            100, 1, 2048, 2)
    np.testing.assert_array_equal(r.c[:, 0], oracle.gemv(inp, "plain").c)


@pytest.mark.parametrize("N", [2, 5, 8])
def test_columns_and_permutation(oracle_lib, N):
    M, K, L = 64, 1024, 2
    a, b, sfa, sfb = inputs(M, N, K, L, N)
    r = oracle.gemm_small_n(a, b, sfa, sfb, M, N, K, L)
    perm = np.random.default_rng(1).permutation(N)
    rp = oracle.gemm_small_n(a, b[:, perm], sfa, sfb[:, perm], M, N, K, L)
    np.testing.assert_array_equal(rp.c, r.c[:, perm])
    b0 = b.copy()
    b0[:, 1] = 0
    r0 = oracle.gemm_small_n(a, b0, sfa, sfb, M, N, K, L)
    assert np.all(r0.s_exact[:, 1] == 0)
    np.testing.assert_array_equal(np.delete(r0.c, 1, axis=1), np.delete(r.c, 1, axis=1))


def test_brute_force_tiny(oracle_lib):
    M, N, K, L = 2, 3, 32, 1
    a, b, sfa, sfb = inputs(M, N, K, L, 9)
    t2, t8 = golden_e2m1(), torch_e4m3()
    ac, bc = synth.unpack_nibbles(a), synth.unpack_nibbles(b)
    r = oracle.gemm_small_n(a, b, sfa, sfb, M, N, K, L)
    for n in range(N):
        for m in range(M):
            s = sum(Fraction(t2[ac[0, m, k]]) * Fraction(t8[sfa[0, m, k // 16]]) *
                    Fraction(t2[bc[0, n, k]]) * Fraction(t8[sfb[0, n, k // 16]]) for k in range(K))
            assert Fraction(int(r.s_exact[0, n, m]), 2 ** 20) == s
