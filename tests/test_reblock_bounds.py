"""CPU mirror of the reblock kernel's index arithmetic (nvfp4_reblock.hip),
run over its whole grid before it runs on a GPU: every plain read and every
blocked write is inside its buffer, every blocked byte is written exactly once,
and the bytes written are the view chain's (padding 0). Keep in step with the
kernel: 256 threads, 16 or 32 tiles per workgroup (one word per tile and row in LDS), workgroup
ids remapped to contiguous ranges per XCD, rows read in 16-byte units when the row length is a multiple of 16 (and the input
16-byte aligned; every unit loads, clamped to a real unit past the matrix,
and writes zeros there), else in words or bytes."""
import numpy as np
import pytest

import block_scaled_fp4_gemv_amd as g
import synth

THREADS = 256


def tiles_of(rows, K, L):
    """The library's choice of tiles per workgroup: 32 where that grid reaches
    256 workgroups and pads a block row's last group by at most an eighth, else 16."""
    nrb, ncb = -(-rows // 128), -(-(K // 16) // 4)
    large = -(-ncb // 32)
    return 32 if L * nrb * large >= 256 and large * 32 - ncb <= ncb // 8 else 16


def emulate(plain, rows, K, L, aligned=True):
    cols = K // 16
    TILES = tiles_of(rows, K, L)
    uw = 4 if (aligned and cols % 16 == 0) else 1      # words per read unit
    upr = TILES // uw
    nrb, ncb = -(-rows // 128), -(-cols // 4)
    wg_per_rb = -(-ncb // TILES)
    out_batch = nrb * ncb * 512
    out = np.full(L * out_batch, 0xAB, np.uint8)
    writes = np.zeros(L * out_batch, np.int64)
    flat = plain.reshape(-1)
    t = np.arange(THREADS)
    nwg = L * nrb * wg_per_rb
    seen = set()
    for bid in range(nwg):
        x, j = bid % 8, bid // 8                            # contiguous logical ids per XCD
        lid = x * (nwg // 8) + min(x, nwg % 8) + j
        assert 0 <= lid < nwg and lid not in seen
        seen.add(lid)
        wg, rbl = lid % wg_per_rb, lid // wg_per_rb
        l, rb = rbl // nrb, rbl % nrb
        assert l < L
        cb0 = wg * TILES
        words = np.zeros((128, TILES), np.uint32)
        for i in range(128 * upr // THREADS):
            e = t + i * THREADS
            row, u = e // upr, e % upr
            r, cb = rb * 128 + row, cb0 + u * uw
            for rr, cc, rw, uu in zip(r, cb, row, u):
                if uw == 4:
                    # 16-byte units: every unit loads, from a clamped (real) unit past the matrix
                    src = l * rows * cols + min(rr, rows - 1) * cols + 4 * min(cc, cols // 4 - 4)
                    assert 0 <= src and src + 16 <= flat.size, "plain read outside the buffer"
                    assert src % 16 == 0, "16-byte read from an unaligned offset"
                if rr >= rows or 4 * cc >= cols:
                    continue
                n = 16 if uw == 4 else min(4, cols - 4 * cc)
                src = l * rows * cols + rr * cols + 4 * cc
                assert 0 <= src and src + n <= flat.size, "plain read outside the buffer"
                assert uw == 1 or src % 16 == 0, "16-byte read from an unaligned offset"
                got = np.zeros(4 * uw, np.uint8)
                got[:n] = flat[src:src + n]
                words[rw, uu * uw:uu * uw + uw] = got.view(np.uint32)
        for i in range(TILES * 32 // THREADS):
            e = t + i * THREADS
            tl, r32 = e // 32, e % 32
            for a, b in zip(tl, r32):
                if cb0 + a >= ncb:
                    continue
                dst = l * out_batch + (rb * ncb + cb0 + a) * 512 + b * 16
                assert 0 <= dst and dst + 16 <= out.size, "blocked write outside the buffer"
                v = np.array([words[b + 32 * i4, a] for i4 in range(4)], np.uint32)
                out[dst:dst + 16] = v.view(np.uint8)
                writes[dst:dst + 16] += 1
    return out.reshape(L, out_batch), writes


@pytest.mark.parametrize("rows,K,L", [(1, 32, 1), (1, 96, 2), (127, 4096, 1), (128, 2048, 2),
                                      (300, 4128, 1), (129, 32, 3), (7, 1056, 2), (130, 8192, 1),
                                      (5, 16640, 2),
                                      # 32 tiles per workgroup (grids of 256 and more)
                                      (129, 8192, 32), (1024, 16384, 4), (100, 15872, 64)])
@pytest.mark.parametrize("aligned", [True, False])
def test_reblock_kernel_indexing(rows, K, L, aligned):
    plain = np.random.default_rng(rows * K + L).integers(0, 256, (L, rows, K // 16), dtype=np.uint8)
    out, writes = emulate(plain, rows, K, L, aligned)
    assert np.all(writes == 1), "each blocked byte is written exactly once"
    np.testing.assert_array_equal(out, synth.to_blocked(plain, pad=0))
    assert out.size == g.nvfp4_blocked_scales_bytes(rows, K, L)


def test_tile_choice():
    """The workloads' reblocks: 32 tiles for the headline SFA, 16 where 32
    would leave CUs idle or pad a block row's last group by more than an eighth."""
    assert tiles_of(7168, 16384, 1) == 32
    assert tiles_of(7168, 2048, 4) == 16          # 224 workgroups with 32
    assert tiles_of(4096, 7168, 8) == 16          # 112 groups: 128 - 112 > 14
    assert tiles_of(129, 8192, 32) == 32 and tiles_of(100, 15872, 64) == 32
