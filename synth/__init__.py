"""Seeded synthetic NVFP4 GEMV inputs, shared by the oracle side and the HIP side.

This module draws random E2M1 codes and E4M3 scale codes and lays the bytes out
in the formats the GEMV consumes. It holds none of the GEMV's arithmetic: it
never decodes a code to a value and never multiplies or sums anything. The only
value-level step is turning the drawn scale magnitudes 2^u into E4M3 codes, and
that is done by torch's float32 -> float8_e4m3fn conversion (round to nearest
even), a library routine.

Memory order (batch outermost, as in the CuTe layouts of the 103289 submission,
`cute_jit_kernel`, whose A stride is (k, 1, m*k) and C stride (1, 1, m)):

    a          uint8 [L][M][K/2]   two E2M1 codes per byte, low nibble = even k
    b          uint8 [L][K/2]      same packing, one row per batch
    sfa_plain  uint8 [L][M][K/16]  one E4M3 code per 16 consecutive k
    sfb_plain  uint8 [L][K/16]
    sfa_blocked uint8 [L][ceil(M/128)*ceil(K/64)*512]   128x4 blocked form
    sfb_blocked uint8 [L][ceil(K/64)*512]               (B padded to 128 rows)

The 128x4 blocked form is built exactly as the 69953 submission's
`to_blocked_batch` builds it: view the (rows, cols) scale matrix as
(row_blocks, 128, col_blocks, 4), permute to (row_blocks, col_blocks, 128, 4),
regroup each 128x4 tile as (4, 32, 4), swap the first two axes and flatten.
Rows are padded to a multiple of 128 and columns to a multiple of 4 first;
the padding is filled with ``pad`` (0x7F, the E4M3 NaN code, by default) so
that any read of padding shows up as NaN in the result.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

E4M3_NAN_CODE = 0x7F


def ceil_div(a: int, b: int) -> int:
    return (a + b - 1) // b


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class Workload:
    """One GEMV problem: M rows, K reduction length, L batches (N is always 1)."""
    name: str
    M: int
    K: int
    L: int
    dist: str = "uniform"      # "uniform" or "edge"
    cfg_id: int = 0

    @property
    def ideal_bytes(self) -> int:
        """Bytes a perfect kernel moves: A, SFA, B, SFB read once, C written once."""
        M, K, L = self.M, self.K, self.L
        return L * (M * K // 2 + M * K // 16 + K // 2 + K // 16 + 2 * M)

    @property
    def ideal_read_bytes(self) -> int:
        M, K, L = self.M, self.K, self.L
        return L * (M * K // 2 + M * K // 16 + K // 2 + K // 16)


def _edge_workloads():
    out = []
    for M in (127, 1000, 7168):
        for K in (64, 4096, 16384):
            for L in (1, 3):
                out.append(Workload(f"edge_{M}x{K}x{L}", M, K, L, "edge", 4))
    return out


TINY = Workload("tiny_128x256x1", 128, 256, 1, "uniform", 0)
BALANCED = Workload("balanced_7168x2048x4", 7168, 2048, 4, "uniform", 1)
BATCHED = Workload("batched_4096x7168x8", 4096, 7168, 8, "uniform", 2)
HEADLINE = Workload("headline_7168x16384x1", 7168, 16384, 1, "uniform", 3)
EDGE = _edge_workloads()
# one GPU's share of the headline split 8 ways along M (whole 128-row blocks)
SHARD = Workload("shard_896x16384x1", 896, 16384, 1, "uniform", 5)
ALL = [TINY, BALANCED, BATCHED, HEADLINE] + EDGE + [SHARD]


def rng_for(w: Workload, set_idx: int = 0, seed: int = 0) -> np.random.Generator:
    return np.random.default_rng([w.cfg_id, w.M, w.K, w.L, set_idx, seed])


# --------------------------------------------------------------------------
# code draws
# --------------------------------------------------------------------------

def e2m1_codes(rng: np.random.Generator, shape, dist: str = "uniform") -> np.ndarray:
    """Random 4-bit E2M1 codes (0..15, -0 included).

    uniform: every code equally likely.
    edge:    code 0 with probability 1/2, otherwise uniform over all 16.
    """
    codes = rng.integers(0, 16, size=shape, dtype=np.uint8)
    if dist == "edge":
        zero = rng.integers(0, 2, size=shape, dtype=np.uint8) == 0
        codes[zero] = 0
    elif dist != "uniform":
        raise ValueError(dist)
    return codes


def e4m3_codes_of(values: np.ndarray) -> np.ndarray:
    """E4M3 codes of finite float values, via torch's float8_e4m3fn cast (RNE)."""
    t = torch.from_numpy(np.ascontiguousarray(values, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def scale_codes(rng: np.random.Generator, shape, dist: str = "uniform") -> np.ndarray:
    """Random E4M3 scale codes.

    uniform: 2^u, u ~ U[-3, 3], rounded to E4M3 (all such values are normals).
    edge:    10% code 0x00 (zero), 10% a subnormal code 0x01..0x07,
             10% 0x7E (448, the largest finite value), 70% as uniform.
    """
    u = rng.uniform(-3.0, 3.0, size=shape)
    codes = e4m3_codes_of(np.exp2(u))
    if dist == "edge":
        pick = rng.integers(0, 10, size=shape, dtype=np.uint8)
        sub = rng.integers(1, 8, size=shape, dtype=np.uint8)
        codes = np.where(pick == 0, np.uint8(0x00), codes)
        codes = np.where(pick == 1, sub, codes)
        codes = np.where(pick == 2, np.uint8(0x7E), codes)
        codes = codes.astype(np.uint8)
    elif dist != "uniform":
        raise ValueError(dist)
    return codes


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """Pack 4-bit codes along the last axis, two per byte, low nibble = even index."""
    assert codes.shape[-1] % 2 == 0
    lo = codes[..., 0::2].astype(np.uint8) & 0xF
    hi = codes[..., 1::2].astype(np.uint8) & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """Inverse of pack_nibbles."""
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out


# --------------------------------------------------------------------------
# 128x4 blocked scale layout
# --------------------------------------------------------------------------

def blocked_bytes_per_batch(rows: int, cols: int) -> int:
    return ceil_div(rows, 128) * ceil_div(cols, 4) * 512


def to_blocked(plain: np.ndarray, pad: int = E4M3_NAN_CODE) -> np.ndarray:
    """Plain scales [L][rows][cols] -> blocked bytes [L][nrb*ncb*512].

    The view / permute / reshape chain of the 69953 submission's
    `to_blocked_batch`, applied per batch after padding rows to 128*nrb and
    columns to 4*ncb with ``pad``.
    """
    L, rows, cols = plain.shape
    nrb, ncb = ceil_div(rows, 128), ceil_div(cols, 4)
    padded = np.full((L, nrb * 128, ncb * 4), pad, dtype=np.uint8)
    padded[:, :rows, :cols] = plain
    out = np.empty((L, nrb * ncb * 512), dtype=np.uint8)
    for l in range(L):
        blocks = padded[l].reshape(nrb, 128, ncb, 4).transpose(0, 2, 1, 3)
        rearranged = blocks.reshape(-1, 4, 32, 4).transpose(0, 2, 1, 3).reshape(-1, 32, 16)
        out[l] = rearranged.reshape(-1)
    return out


# --------------------------------------------------------------------------
# full input sets
# --------------------------------------------------------------------------

@dataclass
class Inputs:
    w: Workload
    a: np.ndarray            # [L][M][K/2]
    b: np.ndarray            # [L][K/2]
    sfa_plain: np.ndarray    # [L][M][K/16]
    sfb_plain: np.ndarray    # [L][K/16]
    sfa_blocked: np.ndarray  # [L][nrb*ncb*512]
    sfb_blocked: np.ndarray  # [L][ncb*512]
    extra: dict = field(default_factory=dict)

    def sfa(self, layout: str) -> np.ndarray:
        return self.sfa_plain if layout == "plain" else self.sfa_blocked

    def sfb(self, layout: str) -> np.ndarray:
        return self.sfb_plain if layout == "plain" else self.sfb_blocked


def make_inputs(w: Workload, set_idx: int = 0, seed: int = 0,
                blocked: bool = True, pad: int = E4M3_NAN_CODE) -> Inputs:
    """Seeded inputs for workload ``w`` (input set ``set_idx``)."""
    M, K, L = w.M, w.K, w.L
    if K % 32 != 0:
        raise ValueError("K must be a multiple of 32")
    rng = rng_for(w, set_idx, seed)
    a_codes = e2m1_codes(rng, (L, M, K), w.dist)
    b_codes = e2m1_codes(rng, (L, K), w.dist)
    sfa = scale_codes(rng, (L, M, K // 16), w.dist)
    sfb = scale_codes(rng, (L, K // 16), w.dist)
    a = pack_nibbles(a_codes)
    b = pack_nibbles(b_codes)
    if blocked:
        sfa_b = to_blocked(sfa, pad)
        sfb_b = to_blocked(sfb.reshape(L, 1, K // 16), pad)
    else:
        sfa_b = np.zeros((L, 0), np.uint8)
        sfb_b = np.zeros((L, 0), np.uint8)
    return Inputs(w, a, b, sfa, sfb, sfa_b, sfb_b)


def from_codes(a_codes: np.ndarray, b_codes: np.ndarray, sfa: np.ndarray,
               sfb: np.ndarray, pad: int = E4M3_NAN_CODE, name: str = "custom") -> Inputs:
    """Build an input set from explicit codes: a_codes [L][M][K], b_codes [L][K],
    sfa [L][M][K/16], sfb [L][K/16]."""
    L, M, K = a_codes.shape
    w = Workload(name, M, K, L, "custom", -1)
    a = pack_nibbles(a_codes)
    b = pack_nibbles(b_codes)
    sfa = np.ascontiguousarray(sfa, dtype=np.uint8)
    sfb = np.ascontiguousarray(sfb, dtype=np.uint8)
    return Inputs(w, a, b, sfa, sfb, to_blocked(sfa, pad),
                  to_blocked(sfb.reshape(L, 1, K // 16), pad))


def random_inputs(M: int, K: int, L: int, seed: int, dist: str = "uniform",
                  pad: int = E4M3_NAN_CODE) -> Inputs:
    """Seeded inputs of an arbitrary shape (used for parity sweeps)."""
    w = Workload(f"random_{M}x{K}x{L}", M, K, L, dist, 99)
    return make_inputs(w, 0, seed, True, pad)
