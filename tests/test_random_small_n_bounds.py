"""Seeded random shapes for the N-vector GEMM (nvfp4_gemm_small_n), drawn so
that every routing branch is hit: N = 1 (the GEMV's kernels), N = 2 (the
dot-product kernel, or the matrix-core kernels on large blocked shapes) and
N = 3..8 (streamed or up-front staged kernels for blocked scales, the unstaged
kernel for plain scales). For each shape and layout the CPU mirror of the
kernel the library picks walks its whole grid (the GEMV kernel with two
vectors included). The same shapes run on the GPU against the oracle in
test_gpu_random_small_n.py."""
import numpy as np
import pytest

import block_scaled_fp4_gemv_amd as g
import test_small_n_bounds as dot_mirror
import test_small_n_mfma_bounds as unstaged_mirror
import test_small_n_staged_bounds as streamed_mirror
import test_small_n_upfront_bounds as upfront_mirror
from test_kernel_bounds import check_shape


def route(M, N, K, L, layout):
    """The kernel nvfp4_gemm_small_n runs (layout 0 plain, 1 blocked)."""
    grid = L * -(-M // 128) * 4
    ws = g.nvfp4_gemv_workspace_bytes(M, K, L)
    mf = N >= 3 or (N == 2 and layout == 1 and K >= 4096 and grid >= 128)
    if N == 1 and ws == 0:
        return "gemv"
    if N == 2 and not mf and ws == 0:
        return "gemv2"
    if mf:
        if layout == 0:
            return "unstaged"
        return "upfront" if grid > 256 and upfront_mirror.staged_lds_bytes(M, N, K, L) >= 0 else "streamed"
    return "dot"


def random_small_n_shapes(seed=77, n=25):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        kind = i % 5
        if kind == 4:      # N = 1 or 2 where the GEMV would split K: the dot-product kernel
            M, N, K, L = (int(rng.integers(1, 130)), int(rng.integers(1, 3)), 32 * int(rng.integers(1025, 2049)),
                          int(rng.integers(1, 3)))
        elif kind == 0:    # N = 1 or 2, small to mid shapes (ragged M and K)
            M, N, K, L = (int(rng.integers(1, 1500)), int(rng.integers(1, 3)), 32 * int(rng.integers(1, 300)),
                          int(rng.integers(1, 4)))
        elif kind == 1:    # N = 2 on the matrix-core kernels: blocked, K >= 4096, 128 workgroups or more
            M, N, K, L = (int(rng.integers(4000, 6000)), 2, 32 * int(rng.integers(128, 260)), 1)
        elif kind == 2:    # N = 3..8, up to 256 workgroups: the streamed kernel (blocked)
            M, N, K, L = (int(rng.integers(1, 2000)), int(rng.integers(3, 9)), 32 * int(rng.integers(1, 400)),
                          int(rng.integers(1, 4)))
        else:              # N = 3..8, many batches: the up-front kernel (blocked)
            M, N, K, L = (int(rng.integers(129, 257)), int(rng.integers(3, 9)), 32 * int(rng.integers(1, 160)),
                          int(rng.integers(33, 45)))
        out.append((M, N, K, L))
    return out


SHAPES = random_small_n_shapes()


def mirror(M, N, K, L, layout):
    kind = route(M, N, K, L, layout)
    if kind == "gemv":
        check_shape(M, K, L, layout)
    elif kind == "gemv2":
        check_shape(M, K, L, layout, nv=2)
    elif kind == "dot":
        dot_mirror.check(M, N, K, L, layout)
    elif kind == "unstaged":
        taken, written = unstaged_mirror.emulate(M, N, K, L, "plain")
        assert np.all(taken == 1) and np.all(written == 1)
    else:
        em = upfront_mirror.emulate if kind == "upfront" else streamed_mirror.emulate
        taken, written = em(M, N, K, L)
        assert np.all(taken == 1) and np.all(written == 1)
    return kind


@pytest.mark.parametrize("M,N,K,L", SHAPES)
@pytest.mark.parametrize("layout", [0, 1])
def test_random_small_n_addresses(M, N, K, L, layout):
    mirror(M, N, K, L, layout)


def test_random_small_n_shapes_cover_the_kernels():
    kinds = {route(M, N, K, L, lay) for M, N, K, L in SHAPES for lay in (0, 1)}
    assert {"gemv", "gemv2", "dot", "unstaged", "streamed", "upfront"} <= kinds, kinds
