"""CPU mirror of the up-front staged matrix-core N-vector kernel's index
arithmetic (nvfp4_gemm_small_n_mfma_upfront_kernel in nvfp4_gemm_small_n.hip), run over its
whole grid before it runs on a GPU. For every workgroup it replays the
prologue's copies into a model of LDS (which global byte each LDS byte holds),
then every LDS read and global load of the loop and the ragged last step, and
checks: global loads inside their buffers, LDS copies and reads inside the
dynamic LDS and each region, every LDS read returning exactly the scale pair or
chunk of B the MFMA step needs, every (row, chunk) of A taken exactly once, and
every output written exactly once.

Keep in step with the kernel: 4 waves of 64 lanes, 2 tiles of 16 rows;
workgroup h of a 128-row block owns rows 8h + p + 32j (p < 8, j < 4); MFMA row m
of tile t is row 8h + (m & 7) + 32 (2 (m >> 3) + t); wave w takes the K-steps
w, w + 4, ...; lane group g = lane / 16 takes chunk 4s + g of step s; the LDS
layout of ms_layout; the ragged last step by the last wave."""
import numpy as np
import pytest

import block_scaled_fp4_gemv_amd as g

WAVES, RT, THREADS, MAXN = 4, 2, 256, 8
DMA = 64 * 16
LDS_LIMIT = 150 * 1024
MAX_DMA_PER_WAVE = 40


def layout(K, N):
    nchunks, ncb = K // 32, (K // 16 + 3) // 4
    n_dma_b = (nchunks + 63) // 64
    n_dma_sfa = (ncb * 8 + 63) // 64
    n_dma_sfb = (ncb + 63) // 64
    b_vec = n_dma_b * DMA + 16
    sfb_vec = n_dma_sfb * 256 + 8
    return dict(n_dma_b=n_dma_b, n_dma_sfa=n_dma_sfa, n_dma_sfb=n_dma_sfb, b_vec=b_vec, sfb_vec=sfb_vec,
                b_bytes=(N * b_vec + 127) // 128 * 128, sfa_bytes=n_dma_sfa * DMA, sfb_bytes=N * sfb_vec)


def staged_lds_bytes(M, N, K, L):
    """Mirror of mu_lds_bytes: the dynamic LDS of the up-front kernel, or -1."""
    if N < 2 or N > MAXN:
        return -1
    o = layout(K, N)
    total = o["b_bytes"] + o["sfa_bytes"] + o["sfb_bytes"]
    ncb = (K // 16 + 3) // 4
    per_wave = N * (-(-o["n_dma_b"] // WAVES)) + (-(-o["n_dma_sfa"] // WAVES)) + N * (-(-o["n_dma_sfb"] // WAVES))
    if total > LDS_LIMIT or per_wave > MAX_DMA_PER_WAVE or ncb > 256 or \
            L * (-(-M // 128)) * 4 > 2 ** 31 - 1:
        return -1
    return total


def blocked_offset(r, kb, ncb):
    return ((r >> 7) * ncb + (kb >> 2)) * 512 + (r & 31) * 16 + ((r >> 5) & 3) * 4 + (kb & 3)


def emulate(M, N, K, L):
    lds_total = staged_lds_bytes(M, N, K, L)
    assert lds_total >= 0
    plan = g.nvfp4_gemm_small_n_plan(M, N, K, L, "blocked")
    assert plan["workgroups"] == L * (-(-M // 128)) * 4
    # the library runs this kernel for grids of more than 256 workgroups
    assert (plan["lds_bytes"] == lds_total) == (plan["workgroups"] > 256)
    o = layout(K, N)
    nchunks, nkb = K // 32, K // 16
    ncb = (nkb + 3) // 4
    nfull = nchunks // 4
    row_bytes = K // 2
    a_bytes, b_bytes = L * M * row_bytes, L * N * row_bytes
    sfa_batch, sfb_batch = -(-M // 128) * ncb * 512, ncb * 512
    P = -(-M // 128) * 4
    sB, sSFA = 0, o["b_bytes"]
    sSFB = sSFA + o["sfa_bytes"]
    taken = np.zeros((L, M, nchunks), np.int64)
    written = np.zeros((L, N, M), np.int64)
    lane = np.arange(64)
    grp, i16 = lane >> 4, lane & 15
    for lid in range(L * P):
        wgb, l = lid % P, lid // P
        blk, h = wgb // 4, wgb % 4
        rbase = blk * 128 + 8 * h
        lds = np.full(lds_total, -1, np.int64)     # global byte index held (B: b_base +, SFA: sfa_base +, SFB: sfb_base +)
        B0, SA0, SB0 = 0, 1 << 40, 2 << 40         # tags of the three global buffers

        def store(dst, src):
            if dst.size:
                assert dst.min() >= 0 and dst.max() < lds_total
                lds[dst] = src

        for wave in range(WAVES):
            for nv in range(N):                    # B copies of vector nv
                for i in range(wave, o["n_dma_b"], WAVES):
                    c = np.minimum(i * 64 + lane, nchunks - 1)
                    src = (l * N + nv) * row_bytes + c * 16
                    assert src.min() >= 0 and (src + 16).max() <= b_bytes
                    dst = sB + nv * o["b_vec"] + i * DMA + lane * 16
                    assert (dst + 16).max() <= sB + o["b_bytes"]
                    for k in range(16):
                        store(dst + k, B0 + src + k)
            for i in range(wave, o["n_dma_sfa"], WAVES):
                it = np.minimum(i * 64 + lane, ncb * 8 - 1)
                src = l * sfa_batch + (blk * ncb + (it >> 3)) * 512 + (8 * h + (it & 7)) * 16
                assert src.min() >= 0 and (src + 16).max() <= L * sfa_batch
                dst = sSFA + i * DMA + lane * 16
                assert (dst + 16).max() <= sSFA + o["sfa_bytes"]
                for k in range(16):
                    store(dst + k, SA0 + src + k)
            for nv in range(N):                    # SFB dwords of vector nv: group q = i * 64 + lane
                for i in range(wave, o["n_dma_sfb"], WAVES):
                    q = np.minimum(i * 64 + lane, ncb - 1)
                    src = l * sfb_batch + q * 512 + nv * 16
                    assert src.min() >= 0 and (src + 4).max() <= L * sfb_batch
                    dst = sSFB + nv * o["sfb_vec"] + i * 256 + lane * 4
                    assert (dst + 4).max() <= sSFB + nv * o["sfb_vec"] + o["sfb_vec"]
                    for k in range(4):
                        store(dst + k, SB0 + src + k)

        n = np.minimum(i16, N - 1)
        n_live = i16 < N

        def rows_of(t):
            return rbase + (i16 & 7) + 32 * (2 * (i16 >> 3) + t)

        def check_step(c, live, a_addr_fn):
            # B chunk c of vector n
            lb = sB + n * o["b_vec"] + c * 16
            for k in range(16):
                assert np.all(lds[lb + k] == B0 + (l * N + n) * row_bytes + c * 16 + k)
            # SFB pair (blocks 2c, 2c+1 of vector n), where live
            lsb = sSFB + n * o["sfb_vec"] + 2 * c
            m = live & n_live
            for k in range(2):
                want = SB0 + l * sfb_batch + blocked_offset(n, 2 * c + k, ncb)
                assert np.all(lds[lsb + k][m] == want[m])
            # SFA: an 8-byte read, tile t's dword = bytes 4t .. 4t+3, pair at 2 (c & 1)
            lsa = sSFA + (c >> 1) * 128 + (i16 & 7) * 16 + 8 * (i16 >> 3)
            assert lsa.min() >= sSFA and (lsa + 8).max() <= sSFA + o["sfa_bytes"]
            for t in range(RT):
                r_real = rows_of(t)
                r = np.minimum(r_real, M - 1)
                for k in range(2):
                    got = lds[lsa + 4 * t + 2 * (c & 1) + k]
                    # padding rows (>= M) hold the tile's padding bytes; their outputs are not written
                    want = SA0 + l * sfa_batch + blocked_offset(r_real, 2 * c + k, ncb)
                    assert np.all(got[live] == want[live])
                a_off = a_addr_fn(r, t)
                assert a_off.min() >= 0 and (a_off + 16).max() <= a_bytes
                assert np.array_equal(a_off, (l * M + r) * row_bytes + c * 16)
                ok = live & (r_real < M)
                np.add.at(taken, (l, r_real[ok], c[ok]), 1)

        for wave in range(WAVES):
            nu = nfull // WAVES + (1 if wave < nfull % WAVES else 0)
            for u in range(nu):
                s = u * WAVES + wave
                assert s < nfull
                c = 4 * s + grp
                check_step(c, np.ones(64, bool),
                           lambda r, t: (l * M + r) * row_bytes + grp * 16 + wave * 64 + u * 64 * WAVES)
        if nchunks % 4:
            c = np.minimum(4 * nfull + grp, nchunks - 1)
            live = 4 * nfull + grp < nchunks
            check_step(c, live, lambda r, t: (l * M + r) * row_bytes + c * 16)
        for e in range(RT * 64 * 4):
            t, ln, j = e >> 8, (e >> 2) & 63, e & 3
            mrow = 4 * (ln >> 4) + j
            col, row = ln & 15, rbase + (mrow & 7) + 32 * (2 * (mrow >> 3) + t)
            if col < N and row < M:
                written[l, col, row] += 1
    return taken, written


@pytest.mark.parametrize("M,N,K,L", [(1, 3, 32, 1), (7, 3, 96, 2), (33, 8, 160, 1), (128, 4, 4096, 1),
                                     (129, 5, 1056, 2), (300, 4, 16384, 1), (45, 7, 224, 3),
                                     (256, 8, 16384, 1), (200, 3, 2048, 4), (100, 6, 7168, 2),
                                     # grids of more than 256 workgroups: the library runs this kernel
                                     (8320, 3, 256, 1), (600, 5, 160, 14), (8320, 2, 4096, 1)])
def test_upfront_kernel_indexing(M, N, K, L):
    taken, written = emulate(M, N, K, L)
    assert np.all(taken == 1), "each (row, chunk) of A is taken exactly once"
    assert np.all(written == 1), "each output is written exactly once"


def streamed_lds_bytes(N):
    NP = 4 if N <= 4 else 8
    return 3 * 32 * (64 * NP + 256 + 8 * NP)


@pytest.mark.parametrize("M,N,K,L", [(7168, 8, 16384, 1), (4096, 4, 7168, 8), (4096, 8, 7168, 8),
                                     (7168, 3, 2048, 4), (7168, 4, 32768, 1), (4096, 4, 32768, 8),
                                     (64, 3, 16448, 1), (100, 5, 160, 300), (1, 3, 32, 1), (8192, 3, 256, 1),
                                     (8320, 3, 256, 1), (4096, 2, 7168, 8), (7168, 2, 16384, 1)])
def test_kernel_choice(M, N, K, L):
    """Mirror of mf_runs and mf_select: blocked scales, N >= 3 (or N = 2 from
    128 workgroups on): the up-front kernel for grids of more than 256
    workgroups where all of K fits in LDS, else the streamed kernel; plain
    scales: the unstaged kernel (no dynamic LDS)."""
    p = g.nvfp4_gemm_small_n_plan(M, N, K, L, "blocked")
    grid = L * (-(-M // 128)) * 4
    assert N >= 3 or (grid >= 128 and K >= 4096)
    assert p["workgroups"] == grid
    up = staged_lds_bytes(M, N, K, L)
    want = up if grid > 256 and up >= 0 else streamed_lds_bytes(N)
    assert p["lds_bytes"] == want
    if N >= 3:
        assert g.nvfp4_gemm_small_n_plan(M, N, K, L, "plain")["lds_bytes"] == 0
