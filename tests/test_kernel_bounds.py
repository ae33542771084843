"""CPU check that every address the GEMV kernel forms stays inside its buffers.

This mirrors the kernel's index arithmetic (nvfp4_gemv.hip) for the whole grid
of each tested shape, using the launch plan the library reports, and checks:
  * A, B, SFA, SFB reads are in bounds, and scale reads never touch the padding
    of the blocked layout,
  * every output row is written exactly once, by the right workgroup,
  * LDS slots stay inside the dynamic LDS allocation,
  * split-K partial and counter indices stay inside the workspace.
It runs before any kernel change goes to the GPU. Keep it in step with the
kernel's constants: kWaves = 4, kRows = 2, kPrefetch = 4, kStage = 8,
kMaxChunksPerWG = 512 (LDS segment), 1024 tickets.
"""
import numpy as np
import pytest

import block_scaled_fp4_gemv_amd as g
import synth

K_WAVES, K_ROWS, K_PREFETCH, K_THREADS = 4, 2, 4, 256
K_STAGE = 512 * 4 // K_THREADS
XCDS = 8


def cdiv(a, b):
    return (a + b - 1) // b


def xcd_remap(i, n):
    x, j = i % XCDS, i // XCDS
    q, r = n // XCDS, n % XCDS
    return x * q + np.minimum(x, r) + j


def sf_row_offset(layout, r, nkb, ncb):
    if layout == 0:
        return r * nkb
    return (r >> 7) * ncb * 512 + (r & 31) * 16 + ((r >> 5) & 3) * 4


def sf_chunk_offset(layout, c):
    if layout == 0:
        return 2 * c
    return (c >> 1) * 512 + (c & 1) * 2


def lds_slot(ci, q):
    return ((ci >> 6) << 8) + (q << 6) + (ci & 63)


def check_shape(M, K, L, layout):
    p = g.nvfp4_gemv_plan(M, K, L)
    lpr, rows_wg, S, kc = p["lanes_per_row"], p["rows_per_wg"], p["k_splits"], p["k_per_split"] // 32
    n_wg = p["workgroups"]
    G = 64 // lpr
    assert rows_wg == K_WAVES * G * K_ROWS
    n_tiles = cdiv(M, rows_wg)
    nchunks, nkb = K // 32, K // 16
    ncb = cdiv(nkb, 4)
    a_size, b_size = L * M * K // 2, L * K // 2
    sfa_batch = M * nkb if layout == 0 else cdiv(M, 128) * ncb * 512
    sfb_batch = nkb if layout == 0 else ncb * 512
    lds_slots = p["lds_bytes"] // 16

    # valid (non-padding) scale bytes of one batch
    valid_sfa = np.zeros(sfa_batch, bool)
    rr, kk = np.meshgrid(np.arange(M), np.arange(nkb), indexing="ij")
    valid_sfa[sf_row_offset(layout, rr, nkb, ncb) + (kk if layout == 0 else (kk >> 2) * 512 + (kk & 3))] = True
    valid_sfb = np.zeros(sfb_batch, bool)
    kb = np.arange(nkb)
    valid_sfb[kb if layout == 0 else (kb >> 2) * 512 + (kb & 3)] = True

    written = np.zeros(L * M, np.int64)
    lids = xcd_remap(np.arange(n_wg), n_wg)
    assert np.array_equal(np.sort(lids), np.arange(n_wg)), "remap is not a bijection"
    tid = np.arange(K_THREADS)
    lane, wave = tid & 63, tid >> 6
    grp, j = lane // lpr, lane % lpr
    for lid in lids:
        s = lid % S
        t2 = lid // S
        tile = t2 % n_tiles
        l = t2 // n_tiles
        assert l < L
        c_begin = s * kc
        c_end = min(c_begin + kc, nchunks)
        assert c_end > c_begin
        for c0 in range(c_begin, c_end, 512):
            nck = min(512, c_end - c0)
            npass = cdiv(nck, lpr)
            # staging loads (clamped pieces) and LDS writes (real pieces only)
            for i in range(K_STAGE):
                pc_raw = tid + i * K_THREADS
                pc = np.minimum(pc_raw, nck * 4 - 1)
                boff = l * (K // 2) + (c0 * 4 + pc) * 4
                assert boff.min() >= 0 and (boff + 4).max() <= b_size
                kbb = 2 * (c0 + (pc >> 2)) + ((pc & 3) >> 1)
                so = kbb if layout == 0 else (kbb >> 2) * 512 + (kbb & 3)
                assert so.max() < sfb_batch and valid_sfb[so].all()
                real = pc_raw < nck * 4
                slots = lds_slot(pc_raw[real] >> 2, pc_raw[real] & 3)
                assert slots.size == 0 or slots.max() < lds_slots
            # main-loop loads: passes run to a multiple of kPrefetch, plus the
            # prefetch issued past the end
            last_pass = cdiv(npass, K_PREFETCH) * K_PREFETCH + K_PREFETCH
            for i in range(K_ROWS):
                r = tile * rows_wg + (wave * G + grp) * K_ROWS + i
                rc = np.minimum(r, M - 1)
                abase = (l * M + rc) * (K // 2)
                sbase = l * sfa_batch + sf_row_offset(layout, rc, nkb, ncb)
                for pas in (0, 1, npass - 1, npass, last_pass - 1):
                    ci = c0 + np.minimum(pas * lpr + j, nck - 1)
                    ao = abase + ci * 16
                    assert ao.min() >= 0 and (ao + 16).max() <= a_size
                    so = sbase + sf_chunk_offset(layout, ci)
                    assert (so + 2).max() <= L * sfa_batch
                    loc = so - l * sfa_batch
                    assert valid_sfa[loc].all() and valid_sfa[loc + 1].all(), "scale read hits padding"
                    slots = np.concatenate([lds_slot(ci - c0, q) for q in range(4)])
                    assert slots.max() < lds_slots
        for i in range(K_ROWS):
            r = tile * rows_wg + (wave * G + grp) * K_ROWS + i
            # one writer lane (j == 0) per row group and row; for split shapes
            # count each row once (the finishing WG writes the whole tile)
            w_rows = r[(j == 0) & (r < M)]
            if S == 1 or s == S - 1:
                np.add.at(written, l * M + w_rows, 1)
        if S > 1:
            assert n_tiles * L < 1024, "more tickets than the fixed ticket region holds"
            ws_part = cdiv(L * M * S * 4, 256) * 256
            assert g.nvfp4_gemv_workspace_bytes(M, K, L) == 4096 + ws_part
            rows = tile * rows_wg + np.arange(rows_wg)
            rows = rows[rows < M]
            assert ((l * M + rows) * S + s).max() < L * M * S
            assert l * n_tiles + tile < n_tiles * L
    assert np.all(written == 1), "some output row is written zero or several times"


SHAPES = sorted({(w.M, w.K, w.L) for w in synth.ALL} |
                {(1, 32, 1), (2, 64, 3), (31, 96, 2), (33, 160, 1), (129, 2080, 2), (300, 4128, 1),
                 (1, 16384, 1), (5, 32768, 1), (257, 7168, 2), (64, 224, 5), (1000, 1024, 1),
                 (3, 4096, 7), (16, 32, 1), (256, 32, 1), (2, 32, 256), (128, 128, 1),
                 (127, 16384, 3), (1000, 16384, 3), (7168, 2048, 4), (5, 32768, 2),
                 (33, 8192, 1), (1000, 4096, 3), (1000, 4096, 1), (256, 2048, 2), (4, 128, 16),
                 (7168, 32768, 1), (64, 65536, 1), (300, 20480, 2)})


@pytest.mark.parametrize("M,K,L", SHAPES)
@pytest.mark.parametrize("layout", [0, 1])
def test_kernel_addresses_in_bounds(M, K, L, layout):
    check_shape(M, K, L, layout)
