"""Pins for the oracle's plain -> 128x4 blocked reblock (CPU only).

The oracle scatters each scale to its blocked byte with the closed-form map
(itself pinned to submission 69953's view chain and 69575's index formula in
test_oracle_layout) and writes 0 into padding. Here it is held to:
  * the literal view / permute / reshape chain of `to_blocked_batch` (synth's
    input generator, padding 0), byte for byte, with and without padding,
  * the inverse map: reading every (row, column) back through the map returns
    the plain scale; every other byte is 0,
  * the GEMV it feeds: oracle GEMV on the reblocked scales equals the oracle
    GEMV on the plain scales, bit for bit.
"""
import numpy as np
import pytest

import oracle
import synth

SHAPES = [(1, 32, 1), (1, 16384, 2), (127, 4096, 3), (128, 64, 1), (129, 96, 2),
          (300, 4128, 1), (1000, 224, 2), (7, 32, 4)]


def plain_scales(rows, K, L, seed):
    return np.random.default_rng(seed).integers(0, 256, (L, rows, K // 16), dtype=np.uint8)


@pytest.mark.parametrize("rows,K,L", SHAPES)
def test_reblock_equals_view_chain(oracle_lib, rows, K, L):
    p = plain_scales(rows, K, L, rows + K + L)
    got = oracle.reblock(p, rows, K, L)
    want = synth.to_blocked(p, pad=0)
    assert got.shape == want.shape
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("rows,K,L", SHAPES[:5])
def test_reblock_inverse_map(oracle_lib, rows, K, L):
    p = plain_scales(rows, K, L, 7)
    got = oracle.reblock(p, rows, K, L)
    nkb = K // 16
    hit = np.zeros(got.shape, bool)
    for l in range(L):
        for r in range(rows):
            for kb in range(nkb):
                off = oracle.sf_offset(1, r, kb, rows, nkb)
                assert got[l, off] == p[l, r, kb]
                hit[l, off] = True
    assert np.all(got[~hit] == 0), "padding must be zero"


def test_reblocked_scales_give_the_same_gemv(oracle_lib):
    M, K, L = 200, 2080, 2
    inp = synth.random_inputs(M, K, L, seed=5, dist="edge")
    sfa_b = oracle.reblock(inp.sfa_plain, M, K, L)
    sfb_b = oracle.reblock(inp.sfb_plain[:, None, :], 1, K, L)
    r_plain = oracle.gemv(inp, "plain")
    r_blk = oracle.gemv_arrays(inp.a, inp.b, sfa_b, sfb_b, M, K, L, "blocked")
    np.testing.assert_array_equal(r_blk.c, r_plain.c)
    np.testing.assert_array_equal(r_blk.s_exact, r_plain.s_exact)


@pytest.mark.parametrize("rows,K,L", [(0, 32, 1), (1, 48, 1), (1, 16, 1), (1, 32, 0)])
def test_reblock_rejects_bad_shapes(oracle_lib, rows, K, L):
    with pytest.raises(ValueError):
        oracle.reblock(np.zeros(max(0, L * rows * (K // 16)), np.uint8), rows, K, L)
