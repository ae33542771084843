"""Seeded random shapes across the plan's branches (row, wide-row, multi-row
and main kernels, with and without a K-split): the CPU mirrors of the kernels'
addressing walk each shape's whole grid in both scale layouts. The same shapes
run on the GPU against the oracle in test_gpu_random_shapes.py."""
import numpy as np
import pytest

from test_kernel_bounds import check_shape


def random_shapes(seed=2026, n=30):
    """Shapes drawn per branch: short rows and few rows, longer K and few
    rows, short K on about one workgroup per CU, general shapes (ragged M, K a
    multiple of 32, up to 8 batches) and few rows with long K (K-splits), each
    small enough for the oracle."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        kind = i % 5
        if kind == 0:      # few rows, K <= 4096
            M, K, L = int(rng.integers(1, 600)), 32 * int(rng.integers(1, 129)), int(rng.integers(1, 4))
        elif kind == 1:    # few rows, longer K
            M, K, L = int(rng.integers(1, 200)), 32 * int(rng.integers(129, 1025)), int(rng.integers(1, 3))
        elif kind == 2:    # short K on a grid of about one workgroup per CU
            M, K, L = int(rng.integers(6017, 8193)), 32 * int(rng.integers(1, 129)), 1
        elif kind == 3:    # general
            M, K, L = int(rng.integers(1, 3000)), 32 * int(rng.integers(1, 640)), int(rng.integers(1, 9))
        else:              # few rows, long K: K-splits
            M, K, L = int(rng.integers(1, 130)), 32 * int(rng.integers(1025, 2049)), int(rng.integers(1, 3))
        out.append((M, K, L))
    return out


SHAPES = random_shapes()


@pytest.mark.parametrize("M,K,L", SHAPES)
@pytest.mark.parametrize("layout", [0, 1])
def test_random_shape_addresses_in_bounds(M, K, L, layout):
    check_shape(M, K, L, layout)
