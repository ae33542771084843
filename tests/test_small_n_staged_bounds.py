"""CPU mirror of the staged matrix-core N-vector kernel's index arithmetic
(nvfp4_gemm_small_n_mfma_staged_kernel in nvfp4_gemm_small_n.hip), run over its
whole grid before it runs on a GPU. Block by block it replays the staging
wave's copies into a model of the block's LDS slot (which global byte each LDS
byte holds), then every LDS read the computing waves make in that block and
every global load of A (the first ring, the refills, the ragged last step),
and checks: loads inside their buffers,
copies and reads inside the slot, every LDS read returning exactly the scale
pair or chunk of B its MFMA step needs, every (row, chunk) of A taken exactly
once, every output written exactly once.

Keep in step with the kernel: wave 0 stages, waves 1..4 compute (cw = 0..3), 2
tiles of 16 rows; workgroup h of a 128-row block owns rows 8h + p + 32j (p < 8,
j < 4); MFMA row m of tile t is row 8h + (m & 7) + 32 (2 (m >> 3) + t);
computing wave cw takes the K-steps 4u + cw; block k is the K-steps 32k ..
32k+31 in slot k % 3 (each block is modelled in a fresh slot: the staging
wave's order is checked by the barrier count); lane group g = lane / 16 takes
chunk 4s + g of step s; copies whose K-steps all lie past the last are skipped;
the slot layout of MsSlot; the ragged last step by the last computing wave."""
import numpy as np
import pytest

import block_scaled_fp4_gemv_amd as g

CWAVES, RT, BLK, LOCAL, RING = 4, 2, 32, 8, 4


def slot_layout(N):
    NP = 4 if N <= 4 else 8
    kB, kSfa, kSfb = BLK * 64 * NP, BLK * 256, BLK * 8 * NP
    return NP, kB, kSfa, kSfb


def blocked_offset(r, kb, ncb):
    return ((r >> 7) * ncb + (kb >> 2)) * 512 + (r & 31) * 16 + ((r >> 5) & 3) * 4 + (kb & 3)


def emulate(M, N, K, L):
    plan = g.nvfp4_gemm_small_n_plan(M, N, K, L, "blocked")
    NP, kB, kSfa, kSfb = slot_layout(N)
    slot_bytes = kB + kSfa + kSfb
    assert plan["lds_bytes"] == 3 * slot_bytes
    P = -(-M // 128) * 4
    assert plan["workgroups"] == L * P
    nchunks, nkb = K // 32, K // 16
    ncb = (nkb + 3) // 4
    nfull = nchunks // 4
    nblk = -(-nfull // BLK)
    row_bytes = K // 2
    a_bytes, b_bytes = L * M * row_bytes, L * N * row_bytes
    sfa_batch, sfb_batch = -(-M // 128) * ncb * 512, ncb * 512
    taken = np.zeros((L, M, nchunks), np.int64)
    written = np.zeros((L, N, M), np.int64)
    lane = np.arange(64)
    grp, i16 = lane >> 4, lane & 15
    B0, SA0, SB0 = 0, 1 << 40, 2 << 40        # tags of the three global buffers
    n = np.minimum(i16, N - 1)
    n_live = i16 < N
    nus = [nfull // CWAVES + (1 if cw < nfull % CWAVES else 0) for cw in range(CWAVES)]
    for lid in range(L * P):
        wgb, l = lid % P, lid // P
        blk, h = wgb // 4, wgb % 4
        rbase = blk * 128 + 8 * h

        def rows_of(t):
            return rbase + (i16 & 7) + 32 * (2 * (i16 >> 3) + t)

        def a_load(addr):
            assert addr.min() >= 0 and (addr + 16).max() <= a_bytes

        # the first ring and the refills of every computing wave (global loads of A)
        for cw in range(CWAVES):
            nu = nus[cw]
            for t in range(RT):
                r = np.minimum(rows_of(t), M - 1)
                row0 = (l * M + r) * row_bytes
                for d in range(RING):
                    a_load(row0 + grp * 16 + cw * 64 + min(d, nu - 1) * 64 * CWAVES if nu > 0 else row0)
                for u in range(nu):
                    if u + RING < nu:
                        a_load(row0 + grp * 16 + cw * 64 + (u + RING) * 64 * CWAVES)
        for k in range(nblk):
            lds = np.full(slot_bytes, -1, np.int64)
            s0 = k * BLK

            def store(dst, src):
                assert dst.min() >= 0 and dst.max() < slot_bytes
                lds[dst] = src

            for i in range(kB // 1024):                # B: [sb][NP][4 chunks of 16 bytes]
                if s0 + (i * 64) // (4 * NP) >= nfull:
                    break                              # every K-step of the copy lies past the end
                e = 64 * i + lane
                s = np.minimum(s0 + e // (4 * NP), nfull - 1)
                nn = np.minimum((e >> 2) % NP, N - 1)
                src = (l * N + nn) * row_bytes + (4 * s + (e & 3)) * 16
                assert src.min() >= 0 and (src + 16).max() <= b_bytes
                for b in range(16):
                    store(i * 1024 + lane * 16 + b, B0 + src + b)
            for i in range(kSfa // 1024):              # SFA: [sb][2 groups][8 pieces of 16 bytes]
                if s0 + 4 * i >= nfull:
                    break
                e = 64 * i + lane
                s = np.minimum(s0 + (e >> 4), nfull - 1)
                q = 2 * s + ((e >> 3) & 1)
                src = l * sfa_batch + (blk * ncb + q) * 512 + (8 * h + (e & 7)) * 16
                assert src.min() >= 0 and (src + 16).max() <= L * sfa_batch
                for b in range(16):
                    store(kB + i * 1024 + lane * 16 + b, SA0 + src + b)
            for i in range(kSfb // 256):               # SFB: [sb][NP][2 groups][4 bytes]
                if s0 + (i * 64) // (2 * NP) >= nfull:
                    break
                e = 64 * i + lane
                s = np.minimum(s0 + e // (2 * NP), nfull - 1)
                nn = np.minimum((e >> 1) % NP, N - 1)
                q = 2 * s + (e & 1)
                src = l * sfb_batch + q * 512 + nn * 16
                assert src.min() >= 0 and (src + 4).max() <= L * sfb_batch
                for b in range(4):
                    store(kB + kSfa + i * 256 + lane * 4 + b, SB0 + src + b)

            def read(off, size):
                assert off.min() >= 0 and (off + size).max() <= slot_bytes
                return np.stack([lds[off + b] for b in range(size)], axis=1)

            for cw in range(CWAVES):
                nu = nus[cw]
                ob = (cw * NP + n) * 64 + grp * 16
                osfb = kB + kSfa + (cw * NP + n) * 8 + 2 * grp
                osfa = kB + cw * 256 + (grp >> 1) * 128 + (i16 & 7) * 16 + 8 * (i16 >> 3)
                for u in range(LOCAL * k, min(LOCAL * (k + 1), nu)):
                    d = u % LOCAL
                    s = 4 * u + cw
                    c = 4 * s + grp
                    got_b = read(ob + d * 4 * 64 * NP, 16)
                    want_b = B0 + ((l * N + n) * row_bytes + c * 16)[:, None] + np.arange(16)
                    assert np.array_equal(got_b, want_b)
                    got_sb = read(osfb + d * 4 * 8 * NP, 2)
                    for b in range(2):
                        want = SB0 + l * sfb_batch + blocked_offset(n, 2 * c + b, ncb)
                        assert np.array_equal(got_sb[n_live, b], want[n_live])
                    got_sa = read(osfa + d * 4 * 256, 8)
                    for t in range(RT):
                        r_real = rows_of(t)
                        for b in range(2):
                            # the pair of chunk c sits at bytes 4t + 2 (c & 1) of the 8-byte read
                            got = got_sa[lane, 4 * t + 2 * (c & 1) + b]
                            want = SA0 + l * sfa_batch + blocked_offset(r_real, 2 * c + b, ncb)
                            assert np.array_equal(got, want)
                        ok = r_real < M
                        np.add.at(taken, (l, r_real[ok], c[ok]), 1)
        if nchunks % 4:                                # ragged last step, from global memory
            c = np.minimum(4 * nfull + grp, nchunks - 1)
            live = 4 * nfull + grp < nchunks
            for t in range(RT):
                r_real = rows_of(t)
                r = np.minimum(r_real, M - 1)
                a_load((l * M + r) * row_bytes + c * 16)
                sa = l * sfa_batch + blocked_offset(r, 2 * c, ncb)
                assert sa.min() >= 0 and (sa + 2).max() <= L * sfa_batch
                ok = live & (r_real < M)
                np.add.at(taken, (l, r_real[ok], c[ok]), 1)
            bo = (l * N + n) * row_bytes + c * 16
            assert bo.min() >= 0 and (bo + 16).max() <= b_bytes
            sb = l * sfb_batch + blocked_offset(n, 2 * c, ncb)
            assert sb.min() >= 0 and (sb + 2).max() <= L * sfb_batch
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
                                     (40, 4, 4224, 1), (20, 8, 40960, 1), (64, 3, 512, 1),
                                     # N = 2 (blocked, K >= 4096, 128 workgroups or more)
                                     (4100, 2, 4224, 1), (2000, 2, 4224, 2),
                                     # wide grids, ragged last 128-row blocks, two batches
                                     (7168, 3, 256, 1), (5000, 5, 128, 1), (6000, 3, 224, 1),
                                     (3000, 8, 128, 2), (1000, 4, 4096, 3)])
def test_staged_kernel_indexing(M, N, K, L):
    taken, written = emulate(M, N, K, L)
    assert np.all(taken == 1), "each (row, chunk) of A is taken exactly once"
    assert np.all(written == 1), "each output is written exactly once"


def test_staged_kernel_applies():
    """Blocked scales with N >= 3 take this kernel for grids of up to 256
    workgroups at any K (its LDS does not depend on K), and past 256 where all
    of K does not fit the up-front kernel's LDS; plain scales never do."""
    for M, N, K, L in [(7168, 8, 16384, 1), (64, 3, 65536, 1), (1, 3, 32, 1), (7168, 4, 32768, 1),
                       (4096, 8, 65536, 8)]:
        NP, kB, kSfa, kSfb = slot_layout(N)
        assert g.nvfp4_gemm_small_n_plan(M, N, K, L, "blocked")["lds_bytes"] == 3 * (kB + kSfa + kSfb)
        assert g.nvfp4_gemm_small_n_plan(M, N, K, L, "plain")["lds_bytes"] == 0
    p2 = g.nvfp4_gemm_small_n_plan(7168, 2, 16384, 1, "blocked")
    assert p2["workgroups"] == 224 and p2["lds_bytes"] == 3 * sum(slot_layout(2)[1:])
    p2 = g.nvfp4_gemm_small_n_plan(127, 2, 16384, 3, "blocked")
    assert p2["workgroups"] == 192          # below 128 workgroups: the dot-product kernel's plan
