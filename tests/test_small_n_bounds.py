"""CPU mirror of the index arithmetic of nvfp4_gemm_small_n's dot-product
kernel (N <= 2; from N = 3 the matrix-core kernel runs, mirrored in
test_small_n_mfma_bounds.py) over its whole grid (keep in step with
nvfp4_gemm_small_n.hip: 256 lanes, one chunk per lane per 256-chunk segment,
a ring of 8 rows): every A, B, SFA and SFB read is inside
its tensor, the per-wave row sums stay inside the planned LDS, and every
output (l, n, m) is written exactly once."""
import numpy as np
import pytest

import block_scaled_fp4_gemv_amd as g

THREADS, RING, WAVES = 256, 8, 4


def cdiv(a, b):
    return -(-a // b)


def xcd_remap(i, n):
    x, j = i % 8, i // 8
    q, r = n // 8, n % 8
    return x * q + np.minimum(x, r) + j


def pair_offset(layout, r, c, nkb, ncb):
    if layout == 0:
        return r * nkb + 2 * c
    return ((r >> 7) * ncb + (c >> 1)) * 512 + (r & 31) * 16 + ((r >> 5) & 3) * 4 + (c & 1) * 2


def check(M, N, K, L, layout):
    p = g.nvfp4_gemm_small_n_plan(M, N, K, L, layout)
    R, n_wg, lds = p["rows_per_wg"], p["workgroups"], p["lds_bytes"]
    assert lds == R * N * WAVES * 4 and lds <= 48 * 1024
    P = n_wg // L
    assert P * L == n_wg and P == cdiv(M, R)
    nchunks, nkb = K // 32, K // 16
    ncb = cdiv(nkb, 4)
    sizes = g.small_n_operand_bytes(M, N, K, L, layout)
    sfa_b, sfb_b = sizes["sfa"] // L, sizes["sfb"] // L
    lids = xcd_remap(np.arange(n_wg), n_wg)
    assert np.array_equal(np.sort(lids), np.arange(n_wg))
    written = np.zeros(L * N * M, np.int64)
    tid = np.arange(THREADS)
    for lid in lids:
        tile, l = lid % P, lid // P
        r0 = tile * R
        nr = min(R, M - r0)
        assert nr >= 1
        for c0 in range(0, nchunks, THREADS):
            c = np.minimum(c0 + tid, nchunks - 1)
            for i in range(cdiv(nr, RING) * RING + RING):        # rows read, with the ring past the end
                r = r0 + min(i, nr - 1)
                a_off = l * M * (K // 2) + r * (K // 2) + c * 16
                assert a_off.min() >= 0 and (a_off + 16).max() <= sizes["a"]
                so = l * sfa_b + pair_offset(layout, r, c, nkb, ncb)
                assert (so + 2).max() <= sizes["sfa"]
            for n in range(N):
                b_off = l * N * (K // 2) + n * (K // 2) + c * 16
                assert (b_off + 16).max() <= sizes["b"]
                so = l * sfb_b + pair_offset(layout, n, c, nkb, ncb)
                assert (so + 2).max() <= sizes["sfb"]
        for i in range(nr):
            for n in range(N):
                assert ((i * N + n) * WAVES + WAVES) * 4 <= lds
                written[(l * N + n) * M + r0 + i] += 1
    assert np.all(written == 1)


@pytest.mark.parametrize("M,N,K,L", [(1, 1, 32, 1), (7, 2, 96, 2), (128, 1, 2048, 1), (300, 2, 20480, 2),
                                     (1000, 2, 4096, 3), (7168, 2, 2048, 1), (4096, 1, 7168, 8),
                                     (129, 2, 16384, 1), (100000, 2, 64, 1)])
@pytest.mark.parametrize("layout", [0, 1])
def test_small_n_addresses(M, N, K, L, layout):
    if layout == 1 and N == 2 and K >= 4096 and L * cdiv(M, 128) * 4 >= 128:
        pytest.skip("blocked scales, N = 2, K >= 4096, 128 workgroups or more: a matrix-core kernel runs")
    check(M, N, K, L, layout)
