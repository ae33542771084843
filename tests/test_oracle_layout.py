"""Pins for the oracle's 128x4 blocked scale index map (bit-exact, brute force).

The oracle's closed-form offset is compared with three descriptions of the
same layout on the pages, each executed as written there:
  1. the view/permute/reshape chain of submission 69953 `to_blocked_batch`
     (run in torch on a tensor of position labels, after padding),
  2. the index arithmetic of submission 69575 `blocked_transform_kernel`
     (tile-major permutation, then the 512-byte chunk split into d1/d2/d3),
  3. the 6-D pre-permuted tensor [32, 4, rest_m, 4, rest_k] of submission
     103289 `permuted_to_blocked` with its permute(2, 4, 0, 1, 3) and reshape.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

SHAPES = [(1, 2), (1, 4), (1, 6), (1, 1024), (127, 4), (128, 16), (129, 6), (256, 8),
          (1000, 256), (7168, 4), (300, 3), (5, 1), (128, 448)]


def cdiv(a, b):
    return (a + b - 1) // b


def oracle_offsets(layout, rows, nkb):
    out = np.empty((rows, nkb), dtype=np.int64)
    for r in range(rows):
        for kb in range(nkb):
            out[r, kb] = oracle.sf_offset(layout, r, kb, rows, nkb)
    return out


def labels_view_chain(rows, nkb):
    """Page 3's chain on labels r*nkb+kb (padding = -1), flattened."""
    nrb, ncb = cdiv(rows, 128), cdiv(nkb, 4)
    lab = torch.full((nrb * 128, ncb * 4), -1, dtype=torch.int64)
    lab[:rows, :nkb] = torch.arange(rows * nkb, dtype=torch.int64).view(rows, nkb)
    blocks = lab.view(nrb, 128, ncb, 4).permute(0, 2, 1, 3)
    rearranged = blocks.reshape(-1, 4, 32, 4).transpose(1, 2).reshape(-1, 32, 16)
    return rearranged.flatten().numpy()


def p2_out_index(i, j, M, K):
    """Page 2's index arithmetic (K = number of scale columns there)."""
    ncb = (K + 3) // 4
    rb, ri = i // 128, i % 128
    cb, ci = j // 4, j % 4
    perm = rb * ncb * 128 * 4 + cb * 128 * 4 + ri * 4 + ci
    chunk = perm // 512
    in_chunk = perm % 512
    d1 = in_chunk // 128
    rest = in_chunk % 128
    d2 = rest // 4
    d3 = rest % 4
    return chunk * 512 + d2 * 16 + d1 * 4 + d3


@pytest.mark.parametrize("rows,nkb", SHAPES)
def test_blocked_map_equals_view_chain(oracle_lib, rows, nkb):
    flat = labels_view_chain(rows, nkb)
    off = oracle_offsets(1, rows, nkb)
    assert flat.size == oracle.sf_batch_bytes(1, rows, nkb)
    labels = np.arange(rows * nkb).reshape(rows, nkb)
    np.testing.assert_array_equal(flat[off], labels)
    # every non-padding slot is hit exactly once (bijection onto the labels)
    assert np.unique(off).size == rows * nkb
    assert (flat >= 0).sum() == rows * nkb


@pytest.mark.parametrize("rows,nkb", SHAPES)
def test_blocked_map_equals_p2_index_formula(oracle_lib, rows, nkb):
    off = oracle_offsets(1, rows, nkb)
    i, j = np.meshgrid(np.arange(rows), np.arange(nkb), indexing="ij")
    np.testing.assert_array_equal(p2_out_index(i, j, rows, nkb), off)


@pytest.mark.parametrize("rows,nkb", [(128, 4), (256, 8), (384, 12), (1024, 64)])
def test_blocked_map_equals_p1_six_d_permute(oracle_lib, rows, nkb):
    # The 6-D tensor's modes are CuTe's scale-factor atom ((32,4),rest_m) x
    # ((4),rest_k): row r = i32 + 32*i4 + 128*rm, block kb = kbi + 4*rk.
    rest_m, rest_k = rows // 128, nkb // 4
    lab = np.arange(rows * nkb).reshape(rows, nkb)
    six = np.empty((32, 4, rest_m, 4, rest_k), dtype=np.int64)
    for i32 in range(32):
        for i4 in range(4):
            for rm in range(rest_m):
                r = i32 + 32 * i4 + 128 * rm
                for kbi in range(4):
                    six[i32, i4, rm, kbi, :] = lab[r, kbi::4]
    flat = torch.from_numpy(six).permute(2, 4, 0, 1, 3).reshape(-1, 32, 16).flatten().numpy()
    off = oracle_offsets(1, rows, nkb)
    np.testing.assert_array_equal(flat[off], lab)


@pytest.mark.parametrize("rows,nkb", [(127, 4), (1000, 256), (128, 16), (1, 1024), (7, 6)])
def test_generator_blocked_bytes_read_back_through_oracle_map(oracle_lib, rows, nkb):
    rng = np.random.default_rng([rows, nkb])
    plain = rng.integers(0, 0x7F, size=(2, rows, nkb), dtype=np.uint8)
    blk = synth.to_blocked(plain)
    off = oracle_offsets(1, rows, nkb)
    for l in range(2):
        np.testing.assert_array_equal(blk[l][off], plain[l])
    # padding holds the NaN code only
    mask = np.ones(blk.shape[1], bool)
    mask[off.ravel()] = False
    assert np.all(blk[:, mask] == 0x7F)


def test_plain_map(oracle_lib):
    for rows, nkb in [(3, 5), (128, 16)]:
        off = oracle_offsets(0, rows, nkb)
        np.testing.assert_array_equal(off, np.arange(rows * nkb).reshape(rows, nkb))
        assert oracle.sf_batch_bytes(0, rows, nkb) == rows * nkb


def test_blocked_sizes(oracle_lib):
    assert oracle.sf_batch_bytes(1, 1000, 256) == 8 * 64 * 512 == 262144
    assert oracle.sf_batch_bytes(1, 7168, 1024) == 7168 * 1024
    assert oracle.sf_batch_bytes(1, 1, 1024) == 256 * 512
    assert oracle.sf_batch_bytes(1, 1, 6) == 2 * 512
