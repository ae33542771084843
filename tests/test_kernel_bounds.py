"""CPU check of the GEMV kernel's address arithmetic, before it runs on a GPU.

This mirrors the index arithmetic of nvfp4_gemv.hip for the whole grid of each
tested shape, using the launch plan the library reports, and checks:
  * every A, B, SFA and SFB read is inside its buffer (A through a buffer
    resource: inside the resource's byte range),
  * the staging wave's LDS writes stay inside their areas (scales of A, B,
    blocked SFB), no two of them hit one byte, and what the computing waves
    read there (the scales of every real (row, chunk), each lane's B chunks
    and their SFB scales) is exactly what was staged, byte for byte; no real
    row reads padding of the blocked layout,
  * every output row is written exactly once, and split-K partial and ticket
    indices stay inside the workspace.
Keep it in step with the kernel's constants: 4 computing waves and one staging
wave, 4 chunks per lane, 8 chunk loads in flight, 1024 tickets.
"""
import numpy as np
import pytest

import block_scaled_fp4_gemv_amd as g
import synth

THREADS, CPL, PREFETCH, XCDS, MAX_TICKETS = 256, 4, 8, 8, 1024
LOADER = 64                 # threads of the staging wave
ROW_THREADS = 256           # the row kernel for small problems (4 waves, one row each)
DMA_BYTES = 64 * 16         # LDS bytes one wave-wide staging load fills
STAGE_B = True              # blocked layout: the staging wave stages B as well as SFB


def cdiv(a, b):
    return (a + b - 1) // b


def xcd_remap(i, n):
    x, j = i % XCDS, i // XCDS
    q, r = n // XCDS, n % XCDS
    return x * q + np.minimum(x, r) + j


def split_local_row(q, nslots):
    """Local row q of a workgroup -> (slot offset, 32-row group): run by run."""
    q = np.asarray(q)
    i4 = (q >= nslots).astype(np.int64) + (q >= 2 * nslots) + (q >= 3 * nslots)
    return q - i4 * nslots, i4


def slot_row(first, nslots, q):
    sl, i4 = split_local_row(q, nslots)
    s = first + sl
    return ((s >> 5) << 7) + (i4 << 5) + (s & 31)


def stage_bytes(lpr, spw):
    return cdiv(32 * lpr * spw, DMA_BYTES) * DMA_BYTES


def sf_offset(layout, r, kb, nkb, ncb):
    """Byte of scale (row r, block kb) inside one batch (numpy-vectorised)."""
    if layout == 0:
        return r * nkb + kb
    return ((r >> 7) * ncb + (kb >> 2)) * 512 + (r & 31) * 16 + ((r >> 5) & 3) * 4 + (kb & 3)


def check_row_shape(M, K, L, layout, p, ws_bytes, strides=None):
    """The row kernel (small problems): a workgroup of 4 waves owns one slot,
    wave w its sub-row w; lane j loads chunks j, j+64, ... (clamped), their B
    chunks, SFB pairs and SFA pairs; lane 63 writes the row's output."""
    nchunks, nkb = K // 32, K // 16
    ncb = cdiv(nkb, 4)
    ns = 32 * (M // 128) + min(32, M % 128)
    assert p["workgroups"] == L * ns and p["rows_per_wg"] == 4 and p["k_splits"] == 1
    assert p["lds_bytes"] == 0 and ws_bytes == 0
    assert nchunks <= 64 * 2 and (L * ns <= 256 or (nchunks <= 8 and L * ns <= 1024))
    cpl = 1
    while 64 * cpl < nchunks:
        cpl *= 2
    sd = strides or g.nvfp4_gemv_dense_strides(M, K, L, layout)
    a_row, a_bat, b_bat, c_bat = sd["a_row"], sd["a_batch"], sd["b_batch"], sd["c_batch"]
    sfa_row, sfa_bat, sfb_bat = sd["sfa_row"], sd["sfa_batch"], sd["sfb_batch"]
    a_bytes = (L - 1) * a_bat + (M - 1) * a_row + K // 2
    b_size = (L - 1) * b_bat + K // 2
    sfa_batch = M * nkb if layout == 0 else cdiv(M, 128) * ncb * 512
    sfb_batch = nkb if layout == 0 else ncb * 512
    sfa_size = (L - 1) * sfa_bat + ((M - 1) * sfa_row + nkb if layout == 0 else sfa_batch)
    sfb_size = (L - 1) * sfb_bat + sfb_batch
    n_wg = p["workgroups"]
    lids = xcd_remap(np.arange(n_wg), n_wg)
    assert np.array_equal(np.sort(lids), np.arange(n_wg)), "remap is not a bijection"
    lane = np.arange(64)
    written = np.zeros((L - 1) * c_bat + M, np.int64)
    taken = np.zeros((L, M, nchunks), np.int64)
    for lid in lids:
        slot, l = lid % ns, lid // ns
        assert l < L
        for w in range(4):
            r = ((slot >> 5) << 7) + (w << 5) + (slot & 31)
            if r >= M:
                continue
            for i in range(cpl):
                c = lane + 64 * i
                live = c < nchunks
                cc = np.minimum(c, nchunks - 1)
                a_off = l * a_bat + r * a_row + cc * 16
                assert a_off.min() >= 0 and (a_off + 16).max() <= a_bytes, "A read outside the tensor"
                b_off = l * b_bat + cc * 16
                assert b_off.min() >= 0 and (b_off + 16).max() <= b_size, "B read outside the tensor"
                sb = l * sfb_bat + sf_offset(layout, np.zeros_like(cc), 2 * cc, nkb, ncb)
                assert sb.min() >= 0 and (sb + 2).max() <= sfb_size and (sb % 2 == 0).all()
                if layout == 0:
                    sa = l * sfa_bat + r * sfa_row + 2 * cc
                else:
                    sa = l * sfa_bat + sf_offset(1, np.full_like(cc, r), 2 * cc, nkb, ncb)
                assert sa.min() >= 0 and (sa + 2).max() <= sfa_size and (sa % 2 == 0).all()
                # the pair is scales (r, 2c) and (r, 2c+1)
                for b in range(2):
                    want = l * sfa_bat + (r * sfa_row + 2 * cc + b if layout == 0
                                          else sf_offset(1, np.full_like(cc, r), 2 * cc + b, nkb, ncb))
                    assert np.array_equal(sa + b, want), "SFA pair is not the chunk's two scales"
                np.add.at(taken, (l, r, cc[live]), 1)
            written[l * c_bat + r] += 1
    assert (taken == 1).all(), "some (row, chunk) is taken zero or several times"
    expect = np.zeros_like(written)
    for l in range(L):
        expect[l * c_bat + np.arange(M)] += 1
    assert np.array_equal(written, expect), "some output row is written zero or several times"


def check_rows_shape(M, K, L, layout, p, ws_bytes, strides=None):
    """The multi-row kernel (many rows, K <= 4096): workgroup (batch l, block
    rb, line h) owns rows rb*128 + 8h + q + 32w (wave w, q < 8); lane j takes
    chunks j, j+64 (clamped) of each. Blocked scales: the waves copy line h of
    every tile of block rb into LDS (copy i: tiles 8i .. 8i+7, clamped) and
    each (row, chunk) reads its pair back from there; plain scales: each row's
    pairs from global memory. Lane 63 writes each live row's output."""
    nchunks, nkb = K // 32, K // 16
    ncb = cdiv(nkb, 4)
    P = cdiv(M, 128) * 4
    assert p["workgroups"] == L * P and p["rows_per_wg"] == 32 and p["k_splits"] == 1 and ws_bytes == 0
    nsc = cdiv(ncb, 8)
    assert p["lds_bytes"] == nsc * DMA_BYTES and nchunks <= 128
    cpl = 1 if nchunks <= 64 else 2
    sd = strides or g.nvfp4_gemv_dense_strides(M, K, L, layout)
    a_row, a_bat, b_bat, c_bat = sd["a_row"], sd["a_batch"], sd["b_batch"], sd["c_batch"]
    sfa_row, sfa_bat, sfb_bat = sd["sfa_row"], sd["sfa_batch"], sd["sfb_batch"]
    a_bytes = (L - 1) * a_bat + (M - 1) * a_row + K // 2
    b_size = (L - 1) * b_bat + K // 2
    sfa_batch = M * nkb if layout == 0 else cdiv(M, 128) * ncb * 512
    sfb_batch = nkb if layout == 0 else ncb * 512
    sfa_size = (L - 1) * sfa_bat + ((M - 1) * sfa_row + nkb if layout == 0 else sfa_batch)
    sfb_size = (L - 1) * sfb_bat + sfb_batch
    n_wg = p["workgroups"]
    lids = xcd_remap(np.arange(n_wg), n_wg)
    assert np.array_equal(np.sort(lids), np.arange(n_wg)), "remap is not a bijection"
    lane = np.arange(64)
    written = np.zeros((L - 1) * c_bat + M, np.int64)
    taken = np.zeros((L, M, nchunks), np.int64)
    for lid in lids:
        l, t = lid // P, lid % P
        rb, h = t >> 2, t & 3
        assert l < L
        lds = np.full(nsc * DMA_BYTES, -1, np.int64)   # global SFA byte each LDS byte holds
        if layout == 1:
            for w in range(4):
                for i in range(w, nsc, 4):
                    tile = np.minimum(8 * i + (lane >> 3), ncb - 1)
                    src = l * sfa_bat + (rb * ncb + tile) * 512 + h * 128 + (lane & 7) * 16
                    assert src.min() >= 0 and (src + 16).max() <= sfa_size, "SFA copy outside the tensor"
                    dst = i * DMA_BYTES + lane * 16
                    assert (dst + 16).max() <= lds.size, "SFA copy outside the LDS"
                    for b in range(16):
                        lds[dst + b] = src + b
        for w in range(4):
            for i in range(cpl):
                c = lane + 64 * i
                live = c < nchunks
                cc = np.minimum(c, nchunks - 1)
                b_off = l * b_bat + cc * 16
                assert b_off.min() >= 0 and (b_off + 16).max() <= b_size, "B read outside the tensor"
                sb = l * sfb_bat + sf_offset(layout, np.zeros_like(cc), 2 * cc, nkb, ncb)
                assert sb.min() >= 0 and (sb + 2).max() <= sfb_size and (sb % 2 == 0).all()
                for q in range(8):
                    r_real = rb * 128 + 8 * h + q + 32 * w
                    r = min(r_real, M - 1)
                    a_off = l * a_bat + r * a_row + cc * 16
                    assert a_off.min() >= 0 and (a_off + 16).max() <= a_bytes, "A read outside the tensor"
                    if layout == 0:
                        sa = l * sfa_bat + r * sfa_row + 2 * cc
                        assert sa.min() >= 0 and (sa + 2).max() <= sfa_size
                        got = [sa, sa + 1]
                    else:
                        off = (cc >> 1) * 128 + q * 16 + w * 4 + (cc & 1) * 2
                        assert (off + 2).max() <= lds.size, "SFA read outside the LDS"
                        got = [lds[off], lds[off + 1]]
                    if r_real < M:
                        for b in range(2):
                            want = l * sfa_bat + (r * sfa_row + 2 * cc + b if layout == 0
                                                  else sf_offset(1, np.full_like(cc, r), 2 * cc + b, nkb, ncb))
                            assert np.array_equal(got[b], want), "SFA pair is not the chunk's two scales"
                        np.add.at(taken, (l, r_real, cc[live]), 1)
                        if i == 0:
                            written[l * c_bat + r_real] += 1
    assert (taken == 1).all(), "some (row, chunk) is taken zero or several times"
    expect = np.zeros_like(written)
    for l in range(L):
        expect[l * c_bat + np.arange(M)] += 1
    assert np.array_equal(written, expect), "some output row is written zero or several times"


def check_wide_row_shape(M, K, L, layout, p, ws_bytes, strides=None):
    """The wide-row kernel (few rows, longer K): a workgroup of 4 waves owns
    one row (workgroup lid: row lid % M of batch lid // M); thread j loads
    chunks j, j+256, ... (clamped), their B chunks, SFB pairs and SFA pairs;
    thread 0 writes the row's output."""
    nchunks, nkb = K // 32, K // 16
    ncb = cdiv(nkb, 4)
    assert p["workgroups"] == L * M and p["rows_per_wg"] == 1 and p["k_splits"] == 1
    assert p["lds_bytes"] == 0 and ws_bytes == 0 and p["lanes_per_row"] == ROW_THREADS
    assert 64 * 2 < nchunks <= ROW_THREADS * 4 and L * M <= 400
    cpl = 1
    while ROW_THREADS * cpl < nchunks:
        cpl *= 2
    sd = strides or g.nvfp4_gemv_dense_strides(M, K, L, layout)
    a_row, a_bat, b_bat, c_bat = sd["a_row"], sd["a_batch"], sd["b_batch"], sd["c_batch"]
    sfa_row, sfa_bat, sfb_bat = sd["sfa_row"], sd["sfa_batch"], sd["sfb_batch"]
    a_bytes = (L - 1) * a_bat + (M - 1) * a_row + K // 2
    b_size = (L - 1) * b_bat + K // 2
    sfa_batch = M * nkb if layout == 0 else cdiv(M, 128) * ncb * 512
    sfb_batch = nkb if layout == 0 else ncb * 512
    sfa_size = (L - 1) * sfa_bat + ((M - 1) * sfa_row + nkb if layout == 0 else sfa_batch)
    sfb_size = (L - 1) * sfb_bat + sfb_batch
    n_wg = p["workgroups"]
    lids = xcd_remap(np.arange(n_wg), n_wg)
    assert np.array_equal(np.sort(lids), np.arange(n_wg)), "remap is not a bijection"
    j = np.arange(ROW_THREADS)
    written = np.zeros((L - 1) * c_bat + M, np.int64)
    taken = np.zeros((L, M, nchunks), np.int64)
    for lid in lids:
        r, l = lid % M, lid // M
        assert l < L
        for i in range(cpl):
            c = j + ROW_THREADS * i
            live = c < nchunks
            cc = np.minimum(c, nchunks - 1)
            a_off = l * a_bat + r * a_row + cc * 16
            assert a_off.min() >= 0 and (a_off + 16).max() <= a_bytes, "A read outside the tensor"
            b_off = l * b_bat + cc * 16
            assert b_off.min() >= 0 and (b_off + 16).max() <= b_size, "B read outside the tensor"
            sb = l * sfb_bat + sf_offset(layout, np.zeros_like(cc), 2 * cc, nkb, ncb)
            assert sb.min() >= 0 and (sb + 2).max() <= sfb_size and (sb % 2 == 0).all()
            if layout == 0:
                sa = l * sfa_bat + r * sfa_row + 2 * cc
            else:
                sa = l * sfa_bat + sf_offset(1, np.full_like(cc, r), 2 * cc, nkb, ncb)
            assert sa.min() >= 0 and (sa + 2).max() <= sfa_size and (sa % 2 == 0).all()
            for b in range(2):
                want = l * sfa_bat + (r * sfa_row + 2 * cc + b if layout == 0
                                      else sf_offset(1, np.full_like(cc, r), 2 * cc + b, nkb, ncb))
                assert np.array_equal(sa + b, want), "SFA pair is not the chunk's two scales"
            np.add.at(taken, (l, r, cc[live]), 1)
        written[l * c_bat + r] += 1
    assert (taken == 1).all(), "some (row, chunk) is taken zero or several times"
    expect = np.zeros_like(written)
    for l in range(L):
        expect[l * c_bat + np.arange(M)] += 1
    assert np.array_equal(written, expect), "some output row is written zero or several times"


def two_vector_strides(M, K, L, layout):
    """The operands of the GEMV kernel with two vectors (nvfp4_gemm_small_n,
    N = 2): B [L][2][K/2], SFB per vector a row (plain) or the next 16-byte line
    of each tile (blocked), C [L][2][M]; plus the offsets between the vectors."""
    sd = g.nvfp4_gemv_dense_strides(M, K, L, layout)
    nkb = K // 16
    sd.update(b_batch=K, c_batch=2 * M, b_vec=K // 2, c_vec=M,
              sfb_vec=nkb if layout == 0 else 16)
    if layout == 0:
        sd["sfb_batch"] = 2 * nkb
    return sd


def check_shape(M, K, L, layout, plan=None, workspace_bytes=None, threads=THREADS, cpl=CPL,
                prefetch=PREFETCH, max_tickets=MAX_TICKETS, strides=None, nv=1):
    """Walk the whole grid of one launch. ``plan``/``workspace_bytes`` default
    to the built library's; the constants can be overridden to check a variant.
    ``strides`` (nvfp4_strides_t fields) default to the dense layout. ``nv`` = 2:
    the main kernel with two right-hand vectors, as the N-vector GEMM runs it."""
    THREADS, CPL, PREFETCH = threads, cpl, prefetch
    if nv == 2:
        p = (plan or g.nvfp4_gemv_two_vectors_plan)(M, K, L)
        ws_bytes = 0
        strides = strides or two_vector_strides(M, K, L, layout)
    else:
        p = (plan or g.nvfp4_gemv_plan)(M, K, L)
        ws_bytes = (workspace_bytes or g.nvfp4_gemv_workspace_bytes)(M, K, L)
    if p["threads_per_wg"] == ROW_THREADS and p["rows_per_wg"] == 32:
        return check_rows_shape(M, K, L, layout, p, ws_bytes, strides)
    if p["threads_per_wg"] == ROW_THREADS and p["rows_per_wg"] == 1:
        return check_wide_row_shape(M, K, L, layout, p, ws_bytes, strides)
    if p["threads_per_wg"] == ROW_THREADS:
        return check_row_shape(M, K, L, layout, p, ws_bytes, strides)
    lpr, spw, S = p["lanes_per_row"], p["rows_per_wg"] // 4, p["k_splits"]
    kc, n_wg, lds_bytes = p["k_per_split"] // 32, p["workgroups"], p["lds_bytes"]
    assert p["threads_per_wg"] == THREADS + LOADER
    nchunks, nkb = K // 32, K // 16
    ncb = cdiv(nkb, 4)
    ns = 32 * (M // 128) + min(32, M % 128)
    P = cdiv(ns, spw)
    assert n_wg == P * L * S
    SEG, G, WPG = lpr * CPL, THREADS // lpr, max(1, lpr // 64)
    stb = stage_bytes(lpr, spw)
    bstb = cdiv(64 * lpr, DMA_BYTES) * DMA_BYTES if STAGE_B else 0
    sfbb = cdiv(32 * lpr, DMA_BYTES) * DMA_BYTES
    assert lds_bytes == stb + nv * (bstb + sfbb) + 4 * spw * nv * WPG * 4
    assert lds_bytes <= 159 * 1024            # a workgroup fits the CU's 160 KiB of LDS
    sd = strides or g.nvfp4_gemv_dense_strides(M, K, L, layout)
    a_row, a_bat, b_bat, c_bat = sd["a_row"], sd["a_batch"], sd["b_batch"], sd["c_batch"]
    sfa_row, sfa_bat, sfb_bat = sd["sfa_row"], sd["sfa_batch"], sd["sfb_batch"]
    b_vec, sfb_vec, c_vec = sd.get("b_vec", 0), sd.get("sfb_vec", 0), sd.get("c_vec", 0)
    assert nv == 1 or S == 1, "several vectors only without a K-split"
    wide_plain = nchunks % 8 == 0 and kc % 8 == 0 and sfa_row % 16 == 0 and sfa_bat % 16 == 0
    direct = layout == 0 and not wide_plain
    # extents: one past the last byte each operand's strides address
    a_bytes = (L - 1) * a_bat + (M - 1) * a_row + K // 2
    b_size = (L - 1) * b_bat + (nv - 1) * b_vec + K // 2
    sfa_batch = M * nkb if layout == 0 else cdiv(M, 128) * ncb * 512     # dense bytes of one batch
    sfb_batch = nkb if layout == 0 else ncb * 512
    sfa_size = (L - 1) * sfa_bat + ((M - 1) * sfa_row + nkb if layout == 0 else sfa_batch)
    sfb_size = (L - 1) * sfb_bat + (nv - 1) * (sfb_vec if layout == 0 else 0) + sfb_batch

    def sfa_addr(l, r, kb):                     # global byte of scale (r, kb) of batch l
        if layout == 0:
            return l * sfa_bat + r * sfa_row + kb
        return l * sfa_bat + sf_offset(1, r, kb, nkb, ncb)
    valid_sfa = np.zeros(sfa_batch, bool)       # bytes that hold a real scale (dense batch)
    rr, kk = np.meshgrid(np.arange(M), np.arange(nkb), indexing="ij")
    valid_sfa[sf_offset(layout, rr, kk, nkb, ncb)] = True
    valid_sfb = np.zeros(sfb_batch + (nv - 1) * sfb_vec, bool)   # vector v's scale (kb) at v * sfb_vec + ...
    for v in range(nv):
        valid_sfb[v * sfb_vec + sf_offset(layout, np.zeros(nkb, np.int64), np.arange(nkb), nkb, ncb)] = True

    written = np.zeros((L - 1) * c_bat + (nv - 1) * c_vec + M, np.int64)
    lids = xcd_remap(np.arange(n_wg), n_wg)
    assert np.array_equal(np.sort(lids), np.arange(n_wg)), "remap is not a bijection"
    tid = np.arange(THREADS)
    grp, j = tid // lpr, tid % lpr
    lane = np.arange(LOADER)
    for lid in lids:
        s, t2 = lid % S, lid // S
        tile, l = t2 % P, t2 // P
        assert l < L
        first = tile * spw
        nslots = min(spw, ns - first)
        assert nslots >= 1
        nq = 4 * nslots
        assert stb + bstb + sfbb + nq * WPG * 4 <= lds_bytes
        c_begin, c_end = s * kc, min(s * kc + kc, nchunks)
        assert c_end > c_begin
        row_base = (first >> 5) << 7
        a_begin = l * a_bat + row_base * a_row
        num_records = min(a_bytes - a_begin, 2 ** 31 - 1)
        nsteps = cdiv(nq, G) * CPL
        rows_all = slot_row(first, nslots, np.arange(nq))
        for c0 in range(c_begin, c_end, SEG):
            nck = min(SEG, c_end - c0)
            # ---- A: every step, including the prefetch issued past the end
            last = cdiv(nsteps, PREFETCH) * PREFETCH + PREFETCH
            for t in range(last):
                q = np.minimum(grp + G * (t // CPL), nq - 1)
                r = np.minimum(slot_row(first, nslots, q), M - 1)
                ci = c0 + np.minimum(j + (t % CPL) * lpr, nck - 1)
                off = (r - row_base) * a_row + ci * 16
                assert off.min() >= 0 and (off + 16).max() <= num_records, "A read outside the resource"
                assert (off + 16).max() < 2 ** 31, "A offset beyond 32 bits"
            # ---- staging wave: LDS byte -> global scale byte
            ncb_seg, cb0, units = (nck + 1) >> 1, c0 >> 1, nck >> 3
            lds_src = np.full(stb, -1, np.int64)
            if not direct:
                items = nslots * ncb_seg if layout == 1 else nq * units
                assert layout == 1 or nck % 8 == 0
                nload = cdiv(items, 64)
                dst_all, src_all = [], []
                for i in range(nload):
                    it = i * 64 + lane              # past the end: the major index is clamped
                    if layout == 1:
                        sg, cb = first + it % nslots, np.minimum(it // nslots, ncb_seg - 1)
                        src = l * sfa_bat + ((sg >> 5) * ncb + cb0 + cb) * 512 + (sg & 31) * 16
                    else:
                        q, u = np.minimum(it // units, nq - 1), it % units
                        r = np.minimum(slot_row(first, nslots, q), M - 1)
                        assert (2 * c0 + 16 * u + 16).max() <= nkb
                        src = l * sfa_bat + r * sfa_row + 2 * c0 + 16 * u
                        assert (src % 16 == 0).all(), "16-byte staging copy from an unaligned address"
                    assert src.min() >= 0 and (src + 16).max() <= sfa_size, "SFA read outside the tensor"
                    dst = i * DMA_BYTES + lane * 16
                    assert (dst + 16).max() <= stb, "staged item outside the staging area"
                    for b in range(16):
                        dst_all.append(dst + b)
                        src_all.append(src + b)
                dst_cat = np.concatenate(dst_all)
                assert np.unique(dst_cat).size == dst_cat.size, "two staging lanes write one LDS byte"
                lds_src[dst_cat] = np.concatenate(src_all)
            else:
                it = np.arange(nq * nck)
                q, c = it // nck, it % nck
                r = np.minimum(slot_row(first, nslots, q), M - 1)
                src = l * sfa_bat + r * sfa_row + 2 * (c0 + c)
                assert src.min() >= 0 and (src + 2).max() <= sfa_size
                assert (src % 2 == 0).all()
                assert (2 * it + 2).max() <= stb
                lds_src[2 * it] = src
                lds_src[2 * it + 1] = src + 1
            # ---- b' inputs staged by the staging wave (blocked layout): B
            # chunks, then the 16-byte line of each 4-block SFB group that holds row 0
            stage_b = layout == 1 and STAGE_B
            b_src = np.full(nv * bstb, -1, np.int64)                # vector v's B at v * bstb
            for v in range(nv):
                for i in range(cdiv(nck, 64) if stage_b else 0):
                    src = l * b_bat + v * b_vec + (c0 + np.minimum(i * 64 + lane, nck - 1)) * 16
                    assert src.min() >= 0 and (src + 16).max() <= b_size and (src % 16 == 0).all()
                    dst = v * bstb + i * DMA_BYTES + lane * 16
                    assert (dst + 16).max() <= (v + 1) * bstb, "staged B outside its area"
                    for b in range(16):
                        b_src[dst + b] = src + b
            sfb_src = np.full(nv * sfbb, -1, np.int64)              # vector v's SFB lines at v * sfbb
            if layout == 1:
                for v in range(nv):
                    for i in range(cdiv(ncb_seg, 64)):
                        src = l * sfb_bat + v * sfb_vec + (cb0 + np.minimum(i * 64 + lane, ncb_seg - 1)) * 512
                        assert src.min() >= 0 and (src + 16).max() <= sfb_size and (src % 16 == 0).all()
                        dst = v * sfbb + i * DMA_BYTES + lane * 16
                        assert (dst + 16).max() <= (v + 1) * sfbb, "staged SFB outside its area"
                        for b in range(16):
                            sfb_src[dst + b] = src + b
            # ---- b': each lane's B chunk and its two SFB scales, per vector
            for v in range(nv):
                for k in range(CPL):
                    cc = np.minimum(j + k * lpr, nck - 1)
                    ci = c0 + cc
                    if stage_b:
                        for b in range(16):
                            assert np.array_equal(b_src[v * bstb + cc * 16 + b], l * b_bat + v * b_vec + ci * 16 + b), \
                                "staged B mismatch"
                    else:
                        boff = l * b_bat + v * b_vec + ci * 16
                        assert boff.min() >= 0 and (boff + 16).max() <= b_size and (boff % 16 == 0).all()
                    so = v * sfb_vec + sf_offset(layout, np.zeros_like(ci), 2 * ci, nkb, ncb)
                    assert (so + 1).max() < valid_sfb.size and (l * sfb_bat + so + 2).max() <= sfb_size
                    assert valid_sfb[so].all() and valid_sfb[so + 1].all()
                    if layout == 1:
                        at = v * sfbb + (cc >> 1) * 16 + (cc & 1) * 2
                        assert (at + 2).max() <= (v + 1) * sfbb
                        assert np.array_equal(sfb_src[at], l * sfb_bat + so), "staged SFB mismatch"
                        assert np.array_equal(sfb_src[at + 1], l * sfb_bat + so + 1), "staged SFB mismatch"

            # ---- computing waves: lane j reads, for its chunk k and round row q,
            # the 2 bytes at sfoff(c) + rowpart(q) (c, q clamped as in the kernel)
            def staged_at(q, c):
                if layout == 1:
                    sl, i4 = split_local_row(q, nslots)
                    return (c >> 1) * nslots * 16 + (c & 1) * 2 + sl * 16 + i4 * 4
                return (q * nck + c) * 2
            for k in range(CPL):
                cc = np.minimum(j + k * lpr, nck - 1)
                for n in range(cdiv(nq, G) + 1):            # one round of read-ahead past the end
                    q = np.minimum(grp + G * n, nq - 1)
                    at = staged_at(q, cc)
                    assert at.min() >= 0 and (at + 2).max() <= stb, "scale read outside the staging area"
            qs = np.arange(nq)[rows_all < M]
            if qs.size:
                qq, cl, b = np.meshgrid(qs, np.arange(nck), np.arange(2), indexing="ij")
                rq = rows_all[qq]
                want = sfa_addr(l, rq, 2 * (c0 + cl) + b)
                got = lds_src[staged_at(qq, cl) + b]
                assert np.array_equal(got, want), "staged scales do not match what the compute reads"
                assert valid_sfa[sf_offset(layout, rq, 2 * (c0 + cl) + b, nkb, ncb)].all()
        # ---- outputs
        real = rows_all[rows_all < M]
        if S == 1 or s == S - 1:
            for v in range(nv):
                np.add.at(written, l * c_bat + v * c_vec + real, 1)
        if S > 1:
            assert P * L <= max_tickets, "more tickets than the ticket region holds"
            ws_part = cdiv(L * M * S * 4, 256) * 256
            assert ws_bytes == 4 * max_tickets + ws_part
            assert ((l * M + real) * S + s).max() < L * M * S
            assert l * P + tile < P * L
    expect = np.zeros_like(written)
    for l in range(L):
        for v in range(nv):
            expect[l * c_bat + v * c_vec + np.arange(M)] += 1
    assert np.array_equal(written, expect), "some output row is written zero or several times"


SHAPES = sorted({(w.M, w.K, w.L) for w in synth.ALL} |
                {(1, 32, 1), (2, 64, 3), (31, 96, 2), (33, 160, 1), (129, 2080, 2), (300, 4128, 1),
                 (1, 16384, 1), (5, 32768, 1), (257, 7168, 2), (64, 224, 5), (1000, 1024, 1),
                 (3, 4096, 7), (16, 32, 1), (256, 32, 1), (2, 32, 256), (128, 128, 1),
                 (127, 16384, 3), (1000, 16384, 3), (7168, 2048, 4), (5, 32768, 2),
                 (33, 8192, 1), (1000, 4096, 3), (1000, 4096, 1), (256, 2048, 2), (4, 128, 16),
                 (7168, 32768, 1), (64, 65536, 1), (300, 20480, 2), (16, 256, 256), (2, 16384, 16),
                 (1, 352, 1), (1, 384, 1), (1, 320, 1), (128, 256, 1), (300, 4128, 1),
                 (127, 65536, 3), (121, 65536, 2), (16, 32768, 1), (1, 1 << 22, 1),
                 # wide-row kernel: K between 4096 and 32768, at most 400 rows
                 (127, 32768, 3), (33, 4160, 2), (100, 8256, 3), (400, 20480, 1), (33, 4128, 2),
                 # multi-row kernel: K <= 4096, grids of 192 .. 256 workgroups (ragged M and
                 # K, a partial last copy of SFA lines, rows past M in the last block)
                 (6017, 2048, 1), (3072, 4096, 2), (7168, 96, 1), (8100, 1056, 1), (2000, 3104, 3)})


@pytest.mark.parametrize("M,K,L", SHAPES)
@pytest.mark.parametrize("layout", [0, 1])
def test_kernel_addresses_in_bounds(M, K, L, layout):
    check_shape(M, K, L, layout)


# the main kernel with two vectors (the N-vector GEMM's N = 2 without a K-split)
TWO_VECTORS = [(1, 32, 1), (33, 160, 5), (1000, 4096, 3), (300, 20480, 2), (127, 16384, 1), (4100, 256, 1),
               (1012, 4352, 3), (7168, 2048, 1), (129, 2080, 2), (7168, 16384, 1)]


@pytest.mark.parametrize("M,K,L", TWO_VECTORS)
@pytest.mark.parametrize("layout", [0, 1])
def test_two_vector_kernel_addresses_in_bounds(M, K, L, layout):
    check_shape(M, K, L, layout, nv=2)


def strided(M, K, L, layout, **over):
    sd = g.nvfp4_gemv_dense_strides(M, K, L, layout)
    sd.update(over)
    return sd


STRIDED = [  # (M, K, L, layout, stride overrides)
    (300, 4128, 2, 0, dict(a_row=2080, a_batch=300 * 2080 + 48, b_batch=128 * 2064, sfa_row=272,
                           sfa_batch=300 * 272 + 16, sfb_batch=272, c_batch=301)),
    (300, 4128, 2, 0, dict(sfa_row=260, sfa_batch=300 * 260 + 2, sfb_batch=258)),   # odd-16 rows: 2-byte path
    (1000, 4096, 3, 1, dict(a_row=2048 + 512, a_batch=0, b_batch=0, sfa_batch=0, c_batch=1000)),
    (127, 16384, 3, 1, dict(a_batch=127 * 8192 + 4096, b_batch=64 * 8192, sfa_batch=4 * 131072 + 512,
                            sfb_batch=131072 + 1024, c_batch=200)),
    (7168, 2048, 4, 1, dict(b_batch=128 * 1024, c_batch=8192)),
    (33, 8192, 2, 0, dict(a_row=4096 + 16, sfa_row=512 + 32, sfa_batch=33 * 544, c_batch=40)),
    # the row kernel with the caller's strides (dense strides take its preloaded-argument variant)
    (127, 4096, 3, 1, dict(a_row=2048 + 256, a_batch=127 * 2304 + 512, b_batch=2048 + 64,
                           sfa_batch=32768 + 512, sfb_batch=32768 + 1024, c_batch=130)),
    (100, 2048, 2, 0, dict(a_row=1024 + 32, a_batch=100 * 1056 + 16, b_batch=1024 + 16, sfa_row=128 + 16,
                           sfa_batch=100 * 144 + 32, sfb_batch=160, c_batch=104)),
    # the multi-row kernel with the caller's strides
    (7000, 2048, 1, 1, dict(a_row=1024 + 48, c_batch=7000)),
    (3000, 2048, 2, 0, dict(a_row=1024 + 16, a_batch=3000 * 1040 + 32, b_batch=1024 + 32, sfa_row=128 + 32,
                            sfa_batch=3000 * 160 + 16, sfb_batch=144, c_batch=3008)),
]


@pytest.mark.parametrize("M,K,L,layout,over", STRIDED)
def test_kernel_addresses_in_bounds_strided(M, K, L, layout, over):
    check_shape(M, K, L, layout, strides=strided(M, K, L, layout, **over))
