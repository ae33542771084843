"""Seeded random strides (nvfp4_gemv_strided) on random shapes of every plan
branch: row pitches and batch strides padded by random multiples of their
alignment, batch stride 0 (one batch broadcast) now and then, gaps between the
output's batches. The CPU mirrors walk each launch with those strides; the
same cases run on the GPU in test_gpu_random_strided.py (bit-identical to the
dense call, gaps untouched, within the oracle's tolerance)."""
import numpy as np
import pytest

import block_scaled_fp4_gemv_amd as g
from test_kernel_bounds import check_shape
from test_random_shapes_bounds import random_shapes


def random_strided(seed=404, n=16):
    rng = np.random.default_rng(seed)
    shapes = [s for s in random_shapes(seed=seed, n=60) if s[0] * s[1] * s[2] <= 8_000_000][:n]
    out = []
    for i, (M, K, L) in enumerate(shapes):
        layout = i % 2
        nkb = K // 16
        pick = lambda: int(rng.integers(0, 5))
        over = dict(a_row=K // 2 + 16 * pick())
        over["a_batch"] = 0 if L > 1 and rng.random() < 0.2 else M * over["a_row"] + 16 * pick()
        over["b_batch"] = 0 if L > 1 and rng.random() < 0.2 else K // 2 + 16 * pick()
        if layout == 0:
            over["sfa_row"] = nkb + 2 * pick()
            over["sfa_batch"] = M * over["sfa_row"] + 2 * pick()
            over["sfb_batch"] = nkb + 2 * pick()
        else:
            over["sfa_batch"] = g.nvfp4_blocked_scales_bytes(M, K, 1) + 16 * pick()
            over["sfb_batch"] = g.nvfp4_blocked_scales_bytes(1, K, 1) + 16 * pick()
        over["c_batch"] = M + pick()
        out.append((M, K, L, layout, over))
    return out


CASES = random_strided()


def strided(M, K, L, layout, **over):
    sd = g.nvfp4_gemv_dense_strides(M, K, L, layout)
    sd.update(over)
    return sd


@pytest.mark.parametrize("M,K,L,layout,over", CASES)
def test_random_strided_addresses_in_bounds(M, K, L, layout, over):
    check_shape(M, K, L, layout, strides=strided(M, K, L, layout, **over))
