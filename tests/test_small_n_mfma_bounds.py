"""CPU mirror of the matrix-core N-vector kernel's index arithmetic
(nvfp4_gemm_small_n_mfma_kernel in nvfp4_gemm_small_n.hip), run over its whole
grid before it runs on a GPU: every load of A, SFA, B and SFB is inside its
buffer, every (row, chunk) of A is taken by exactly one live lane slot, every
output (vector, row) is written exactly once, and nothing outside c is. Keep in
step with the kernel: 4 waves of 64 lanes, 2 tiles of 16 rows per workgroup,
the whole steps of 4 chunks dealt to the waves in turn, GROUP consecutive
steps at a time (scale pairs addressed as chunk g's pair plus s steps), a
ragged last step taken by the last wave, lane group g = lane/16 on chunk g of a step, the 16x16 result with lane L holding rows 4 (L/16) + j
of vector slot L % 16."""
import numpy as np
import pytest

import block_scaled_fp4_gemv_amd as g

WAVES, RT, GROUP = 4, 2, 2


def pair_offset(r, c, nkb, ncb, layout):
    if layout == "plain":
        return r * nkb + 2 * c
    return ((r >> 7) * ncb + (c >> 1)) * 512 + (r & 31) * 16 + ((r >> 5) & 3) * 4 + (c & 1) * 2


def wave_steps(wave, nfull, group=GROUP):
    """The K-steps of one wave, in its order: the kernel's local step u maps
    to (u // group) * WAVES * group + wave * group + u % group."""
    span = WAVES * group
    ncyc = nfull // span
    nu = ncyc * group + min(max(nfull - ncyc * span - wave * group, 0), group)
    return [(u // group) * span + wave * group + u % group for u in range(nu)]


def emulate(M, N, K, L, layout):
    plan = g.nvfp4_gemm_small_n_plan(M, N, K, L, layout)
    assert plan["lds_bytes"] == 0, "the unstaged kernel runs for this shape and layout"
    P = -(-M // (16 * RT))
    assert plan["workgroups"] == L * P
    nchunks, nkb = K // 32, K // 16
    ncb = (nkb + 3) // 4
    a_bytes = L * M * K // 2
    b_bytes = L * N * K // 2
    sfa_batch = M * nkb if layout == "plain" else -(-M // 128) * ncb * 512
    sfb_batch = N * nkb if layout == "plain" else -(-N // 128) * ncb * 512
    taken = np.zeros((L, M, nchunks), np.int64)
    written = np.zeros((L, N, M), np.int64)
    lane = np.arange(64)
    grp, i16 = lane >> 4, lane & 15
    for lid in range(L * P):
        tile, l = lid % P, lid // P
        assert l < L
        r0 = tile * 16 * RT
        n = np.minimum(i16, N - 1)
        step = 8 if layout == "plain" else 1024
        nfull = nchunks // 4

        def visit(s, c, live, via_step):
            for t in range(RT):
                r_real = r0 + 16 * t + i16
                rows = np.minimum(r_real, M - 1)
                a_off = (l * M + rows) * (K // 2) + c * 16
                assert a_off.min() >= 0 and (a_off + 16).max() <= a_bytes
                sa = l * sfa_batch + pair_offset(rows, c, nkb, ncb, layout)
                if via_step:      # the kernel's form: chunk grp's pair plus s steps
                    assert np.array_equal(sa, l * sfa_batch + pair_offset(rows, grp, nkb, ncb, layout) + s * step)
                assert sa.min() >= 0 and (sa + 2).max() <= L * sfa_batch
                ok = live & (r_real < M)
                np.add.at(taken, (l, r_real[ok], c[ok]), 1)
            b_off = (l * N + n) * (K // 2) + c * 16
            assert b_off.min() >= 0 and (b_off + 16).max() <= b_bytes
            sb = l * sfb_batch + pair_offset(n, c, nkb, ncb, layout)
            if via_step:
                assert np.array_equal(sb, l * sfb_batch + pair_offset(n, grp, nkb, ncb, layout) + s * step)
            assert sb.min() >= 0 and (sb + 2).max() <= L * sfb_batch

        for wave in range(WAVES):
            for s in wave_steps(wave, nfull):
                assert 0 <= s < nfull
                visit(s, 4 * s + grp, np.ones(64, bool), True)
        if nchunks % 4:          # the ragged last step, taken by the last wave
            c = np.minimum(4 * nfull + grp, nchunks - 1)
            visit(nfull, c, 4 * nfull + grp < nchunks, False)
        for e in range(RT * 64 * 4):
            t, ln, j = e >> 8, (e >> 2) & 63, e & 3
            col, row = ln & 15, r0 + 16 * t + 4 * (ln >> 4) + j
            if col < N and row < M:
                written[l, col, row] += 1
    return taken, written


# plain scales only: blocked scales take the staged kernel
@pytest.mark.parametrize("M,N,K,L,layout", [
    (M, N, K, L, "plain") for M, N, K, L in [(1, 3, 32, 1), (7, 3, 96, 2), (33, 8, 160, 1), (64, 4, 4096, 1),
                                             (129, 5, 1056, 2), (300, 4, 20480, 1), (45, 7, 224, 3),
                                             (100, 5, 160, 300), (300, 4, 1056, 120)]])
def test_mfma_kernel_indexing(M, N, K, L, layout):
    taken, written = emulate(M, N, K, L, layout)
    assert np.all(taken == 1), "each (row, chunk) of A is taken exactly once"
    assert np.all(written == 1), "each output is written exactly once"


@pytest.mark.parametrize("group", [1, 2, 4, 8])
def test_wave_steps_partition(group):
    """The waves' steps are a partition of 0 .. nfull-1, each wave's in
    increasing order, for every step count up to a few spans."""
    for nfull in range(0, 5 * WAVES * group + 3):
        seen = []
        for wave in range(WAVES):
            st = wave_steps(wave, nfull, group)
            assert st == sorted(st)
            seen += st
        assert sorted(seen) == list(range(nfull))
