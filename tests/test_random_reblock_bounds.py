"""Seeded random reblock shapes (ragged rows and columns, both tile counts,
aligned and unaligned plain input): the CPU mirror of the reblock kernel walks
each grid and must produce the view chain's bytes; the same shapes run on the
GPU in test_gpu_random_reblock.py, byte for byte against the oracle."""
import numpy as np
import pytest

import synth
from test_reblock_bounds import emulate, tiles_of


def random_reblock_shapes(seed=909, n=10):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        if i % 3 == 0:    # grids that take 32 tiles (256 workgroups or more of 128 rows x 128 columns)
            rows, K, L = int(rng.integers(1, 129)), 2048 * int(rng.integers(8, 11)), int(rng.integers(32, 41))
        else:
            rows, K, L = int(rng.integers(1, 1000)), 32 * int(rng.integers(1, 300)), int(rng.integers(1, 4))
        out.append((rows, K, L))
    return out


SHAPES = random_reblock_shapes()


@pytest.mark.parametrize("rows,K,L", SHAPES)
@pytest.mark.parametrize("aligned", [True, False])
def test_random_reblock_indexing(rows, K, L, aligned):
    plain = np.random.default_rng(rows * K + L).integers(0, 256, (L, rows, K // 16), dtype=np.uint8)
    out, writes = emulate(plain, rows, K, L, aligned)
    assert np.all(writes == 1), "each blocked byte is written exactly once"
    np.testing.assert_array_equal(out, synth.to_blocked(plain, pad=0))


def test_random_reblock_shapes_take_both_tile_counts():
    assert {tiles_of(r, K, L) for r, K, L in SHAPES} == {16, 32}
