"""CPU checks of the C ABI: the library loads, exports every symbol the header
declares, validates arguments before any HIP call, and plans shapes sanely.
No compute call is made here (there is no GPU)."""
import ctypes
import os
import re

import pytest

import block_scaled_fp4_gemv_amd as g
import synth
from conftest import no_gpu_only

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4_gemv.h")

A16 = 0x10000       # fake but aligned device addresses: validation never dereferences them.
# A call whose arguments all pass validation would launch on them, so such
# tests carry @no_gpu_only and skip wherever a GPU is visible.
OK_ARGS = dict(a=A16, b=A16 + 0x100, sfa=A16 + 0x200, sfb=A16 + 0x300, c=A16 + 0x400)


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nvfp4_\w+)\s*\(", text)))


def test_header_declares_what_binding_lists():
    assert header_functions() == sorted(g.EXPORTED_SYMBOLS)


def test_library_exports_every_header_symbol():
    lib = g.lib()
    for name in header_functions():
        assert hasattr(lib, name), name
    out = os.popen(f"nm -D --defined-only {g.LIB_PATH}").read()
    for name in header_functions():
        assert re.search(rf"\bT {name}$", out, re.M), name


def call(**kw):
    args = dict(OK_ARGS, M=128, K=256, L=1, layout=0)
    args.update(kw)
    return g.lib().nvfp4_gemv(args["a"], args["b"], args["sfa"], args["sfb"], args["c"],
                              args["M"], args["K"], args["L"], args["layout"], None)


@pytest.mark.parametrize("ptr", ["a", "b", "sfa", "sfb", "c"])
def test_null_pointers(ptr):
    assert call(**{ptr: None}) == g.NVFP4_ERR_NULL_POINTER


@pytest.mark.parametrize("M,K,L", [(0, 256, 1), (128, 0, 1), (128, 256, 0), (-1, 256, 1),
                                   (128, 48, 1), (128, 16, 1), (128, 100, 1), (2 ** 40, 256, 1),
                                   (1, 2 ** 40, 1), (1 << 20, 1 << 20, 1 << 20)])
def test_bad_shapes(M, K, L):
    assert call(M=M, K=K, L=L) == g.NVFP4_ERR_INVALID_SHAPE


@pytest.mark.parametrize("ptr,off", [("a", 8), ("b", 4), ("sfa", 4), ("sfa", 8), ("sfb", 1), ("sfb", 2), ("c", 1)])
def test_misaligned(ptr, off):
    assert call(**{ptr: OK_ARGS[ptr] + off}) == g.NVFP4_ERR_MISALIGNED


@no_gpu_only
def test_alignment_minimums_accepted_by_validation():
    # 4-byte aligned sfb and 2-byte aligned c pass validation (they then
    # fail later only because there is no GPU here, never with MISALIGNED)
    st = call(sfb=OK_ARGS["sfb"] + 4, c=OK_ARGS["c"] + 2)
    assert st not in (g.NVFP4_ERR_MISALIGNED, g.NVFP4_ERR_NULL_POINTER, g.NVFP4_ERR_INVALID_SHAPE)


@pytest.mark.parametrize("layout", [2, -1, 99])
def test_bad_layout(layout):
    assert call(layout=layout) == g.NVFP4_ERR_INVALID_LAYOUT


def test_ex_workspace_errors():
    lib = g.lib()
    M, K, L = 16, 32768, 1                      # a shape the plan splits along K
    need = lib.nvfp4_gemv_workspace_bytes(M, K, L)
    assert need > 0
    base = (OK_ARGS["a"], OK_ARGS["b"], OK_ARGS["sfa"], OK_ARGS["sfb"], OK_ARGS["c"], M, K, L, 1)
    assert lib.nvfp4_gemv_ex(*base, None, need, None) == g.NVFP4_ERR_WORKSPACE
    assert lib.nvfp4_gemv_ex(*base, 0x200000, need - 1, None) == g.NVFP4_ERR_WORKSPACE
    assert lib.nvfp4_gemv_ex(*base, 0x200010, need, None) == g.NVFP4_ERR_WORKSPACE
    # shape errors take precedence and need no workspace
    assert lib.nvfp4_gemv_ex(*base[:5], M, 33, L, 1, None, 0, None) == g.NVFP4_ERR_INVALID_SHAPE


def scaled(alpha=1.0, ws=None, ws_bytes=0, M=128, K=256, L=1, **kw):
    args = dict(OK_ARGS)
    args.update(kw)
    return g.lib().nvfp4_gemv_scaled(args["a"], args["b"], args["sfa"], args["sfb"], args["c"],
                                     M, K, L, 1, alpha, ws, ws_bytes, None)


@pytest.mark.parametrize("alpha", [float("nan"), float("inf"), float("-inf")])
def test_scaled_rejects_non_finite_alpha(alpha):
    assert scaled(alpha) == g.NVFP4_ERR_INVALID_SCALE


def test_scaled_validation_order():
    # pointer, shape and alignment errors come before the scale check
    assert scaled(float("nan"), a=None) == g.NVFP4_ERR_NULL_POINTER
    assert scaled(float("nan"), K=48) == g.NVFP4_ERR_INVALID_SHAPE
    assert scaled(float("nan"), c=OK_ARGS["c"] + 1) == g.NVFP4_ERR_MISALIGNED


def test_scaled_workspace_errors():
    M, K, L = 16, 32768, 1                      # a shape the plan splits along K
    need = g.lib().nvfp4_gemv_workspace_bytes(M, K, L)
    assert need > 0
    assert scaled(0.5, None, need, M, K, L) == g.NVFP4_ERR_WORKSPACE       # NULL with a size
    assert scaled(0.5, 0x200000, need - 1, M, K, L) == g.NVFP4_ERR_WORKSPACE
    assert scaled(0.5, 0x200010, need, M, K, L) == g.NVFP4_ERR_WORKSPACE


def test_workspace_bytes():
    lib = g.lib()
    for w in (synth.BALANCED, synth.BATCHED, synth.HEADLINE, synth.TINY):
        assert lib.nvfp4_gemv_workspace_bytes(w.M, w.K, w.L) == 0, w.name
    assert lib.nvfp4_gemv_workspace_bytes(0, 256, 1) == 0
    assert lib.nvfp4_gemv_workspace_bytes(16, 32768, 1) % 256 == 0
    assert lib.nvfp4_gemv_workspace_bytes(127, 16384, 3) == 0    # a split would cost more than it saves


@pytest.mark.parametrize("w", synth.ALL, ids=lambda w: w.name)
def test_plans(w):
    p = g.nvfp4_gemv_plan(w.M, w.K, w.L)
    assert 1 <= p["lanes_per_row"] <= 256
    assert p["k_splits"] >= 1
    assert p["k_per_split"] % 32 == 0
    assert p["k_splits"] * p["k_per_split"] >= w.K > (p["k_splits"] - 1) * p["k_per_split"]
    ns = 32 * (w.M // 128) + min(32, w.M % 128)
    assert p["lds_bytes"] <= 159 * 1024       # a workgroup fits the CU's 160 KiB of LDS
    nchunks = w.K // 32
    if 128 < nchunks <= 1024 and w.M * w.L <= 400 and p["k_splits"] == 1:
        # few rows, longer K: the wide-row kernel, one row per workgroup of 4 waves
        assert p["threads_per_wg"] == 256 and p["rows_per_wg"] == 1 and p["lanes_per_row"] == 256
        assert p["workgroups"] == w.M * w.L and p["lds_bytes"] == 0
        return
    tiles = synth.ceil_div(ns, p["rows_per_wg"] // 4)
    assert p["workgroups"] == tiles * w.L * p["k_splits"]
    if w.K <= 4096 and (ns * w.L <= 256 or (w.K <= 256 and ns * w.L <= 1024)):
        # few rows: the row kernel, 4 waves of one row each, one slot per workgroup, no LDS
        assert p["threads_per_wg"] == 256 and p["rows_per_wg"] == 4 and p["lds_bytes"] == 0
        assert p["lanes_per_row"] == 64
    elif w.K <= 4096 and 192 <= w.L * synth.ceil_div(w.M, 128) * 4 <= 256:
        # short rows, a grid of about one workgroup per CU: the multi-row
        # kernel, 32 rows per workgroup of 4 waves, the blocked SFA lines in LDS
        assert p["threads_per_wg"] == 256 and p["rows_per_wg"] == 32 and p["lanes_per_row"] == 64
        assert p["lds_bytes"] == synth.ceil_div(synth.ceil_div(w.K // 16, 4), 8) * 1024
    else:
        assert p["threads_per_wg"] == 320      # 4 computing waves and the staging wave


def test_split_slices_start_on_scale_groups():
    """With a K-split, every slice is a multiple of 8 chunks (256 k), so each
    starts on a 4-block scale group, and the slices cover K."""
    for M, K, L in [(102, 55872, 2), (90, 46272, 1), (64, 65536, 1), (5, 32768, 2), (1, 1 << 22, 1),
                    (30, 60768, 2), (127, 65536, 3)]:
        p = g.nvfp4_gemv_plan(M, K, L)
        if p["k_splits"] > 1:
            assert p["k_per_split"] % 256 == 0, (M, K, L, p)
            assert p["k_splits"] * p["k_per_split"] >= K > (p["k_splits"] - 1) * p["k_per_split"]


def test_multi_row_kernel_boundaries():
    """The multi-row kernel takes short rows (K <= 4096, not the row kernel's)
    where its grid of 32-row workgroups is 192 to 256 workgroups; with more
    (several per CU) or fewer, and for longer K, the main kernel runs."""
    rows = lambda M, K, L: g.nvfp4_gemv_plan(M, K, L)["rows_per_wg"] == 32
    assert rows(7168, 64, 1) and rows(7168, 4096, 1) and rows(3072, 4096, 2) and rows(8192, 2048, 1)
    assert rows(6017, 2048, 1) and not rows(6016, 2048, 1)        # 192 workgroups; 188
    assert not rows(8193, 2048, 1)                                # 260 workgroups
    assert not rows(7168, 2048, 4) and not rows(7168, 4096, 3)    # several workgroups per CU
    assert not rows(7168, 4128, 1) and not rows(1000, 4096, 3)    # longer K; a small grid


def test_row_kernel_boundaries():
    """The row kernel takes K <= 4096 when the slots of all batches fit one
    workgroup per CU (four per CU with K <= 256); larger shapes, longer K and
    K-splits keep the main kernel."""
    row = lambda M, K, L: (g.nvfp4_gemv_plan(M, K, L)["threads_per_wg"] == 256
                           and g.nvfp4_gemv_plan(M, K, L)["rows_per_wg"] == 4)
    assert row(1024, 4096, 1) and not row(1025, 4096, 1)          # 256 slots; 257
    assert row(127, 4096, 3) and row(128, 256, 2) and row(1000, 64, 3) and row(4096, 256, 1)
    assert not row(4097, 256, 1) and not row(1000, 288, 3)        # 1025 slots; K above 256 with 750
    assert not row(7168, 16384, 1) and not row(1000, 4096, 3) and not row(896, 16384, 1)
    assert not row(127, 4128, 1)                                  # K above 64 lanes x 2 chunks
    assert not row(5, 32768, 1)                                   # long K (split)


def test_wide_row_kernel_boundaries():
    """The wide-row kernel takes 4096 < K <= 32768 for at most 400 rows over
    all batches, where the plan needs no K-split."""
    wide = lambda M, K, L: g.nvfp4_gemv_plan(M, K, L)["rows_per_wg"] == 1
    assert wide(127, 16384, 3) and wide(127, 16384, 1) and wide(400, 8192, 1) and wide(1, 16384, 1)
    assert not wide(401, 16384, 1) and not wide(896, 16384, 1) and not wide(1000, 16384, 1)
    assert not wide(127, 4096, 3)                                 # the row kernel
    assert wide(33, 4128, 2)                                      # K just past the row kernel's
    assert not wide(1, 65536, 1) and not wide(5, 32768, 2) and not wide(1, 32768, 1)   # K-splits


def test_long_k_is_segmented_not_split():
    # K beyond one segment (4 chunks x 256 lanes) is walked in segments, not split
    p = g.nvfp4_gemv_plan(7168, 65536, 1)
    assert p["k_splits"] == 1 and p["k_per_split"] == 65536 and p["lanes_per_row"] == 256


def test_split_only_for_small_grids():
    for M, K, L in [(127, 16384, 1), (1000, 4096, 3), (1, 32768, 1), (5, 65536, 2), (127, 65536, 3)]:
        p = g.nvfp4_gemv_plan(M, K, L)
        ns = 32 * (M // 128) + min(32, M % 128)
        if p["k_splits"] > 1:
            assert ns * L < 256 and p["k_per_split"] >= 256 * 32
            assert g.nvfp4_gemv_workspace_bytes(M, K, L) >= 4096


def test_headline_plan_has_no_split():
    p = g.nvfp4_gemv_plan(7168, 16384, 1)
    assert p["k_splits"] == 1 and p["lanes_per_row"] == 128
    assert p["workgroups"] == 256 and p["rows_per_wg"] == 28


def test_plan_rejects_bad_shape():
    with pytest.raises(g.Nvfp4Error):
        g.nvfp4_gemv_plan(128, 100, 1)


def test_status_strings():
    for st in range(0, 9):
        assert g.status_string(st)
    assert g.status_string(1234) == "unknown status"


def test_binding_checks_buffer_sizes():
    # size checks happen in the binding before the library is called
    class Fake:
        is_cuda = True

        def __init__(self, n):
            self.n = n

        def is_contiguous(self):
            return True

        def data_ptr(self):
            return A16

        def numel(self):
            return self.n

        def element_size(self):
            return 1

    with pytest.raises(ValueError, match="a holds"):
        g.nvfp4_gemv(Fake(10), Fake(128), Fake(2048), Fake(16), Fake(256), 128, 256, 1, "plain")


def test_blocked_scales_bytes():
    assert g.nvfp4_blocked_scales_bytes(7168, 16384, 1) == 56 * 256 * 512
    assert g.nvfp4_blocked_scales_bytes(1, 32, 3) == 3 * 512
    assert g.nvfp4_blocked_scales_bytes(129, 96, 2) == 2 * 2 * 2 * 512
    for bad in [(0, 32, 1), (1, 48, 1), (1, 32, 0), (1, 16, 1)]:
        assert g.nvfp4_blocked_scales_bytes(*bad) == 0


def test_reblock_validation_before_launch():
    lib = g.lib()
    assert lib.nvfp4_scales_to_blocked(None, A16, 128, 256, 1, None) == g.NVFP4_ERR_NULL_POINTER
    assert lib.nvfp4_scales_to_blocked(A16, None, 128, 256, 1, None) == g.NVFP4_ERR_NULL_POINTER
    assert lib.nvfp4_scales_to_blocked(A16, A16 + 0x1000, 128, 48, 1, None) == g.NVFP4_ERR_INVALID_SHAPE
    assert lib.nvfp4_scales_to_blocked(A16, A16 + 0x1000, 0, 256, 1, None) == g.NVFP4_ERR_INVALID_SHAPE
    assert lib.nvfp4_scales_to_blocked(A16, A16 + 0x1008, 128, 256, 1, None) == g.NVFP4_ERR_MISALIGNED


def strided_call(layout=1, M=1000, K=4096, L=3, **over):
    sd = g.nvfp4_gemv_dense_strides(M, K, L, layout)
    sd.update(over)
    st = g.Strides(**sd)
    return g.lib().nvfp4_gemv_strided(OK_ARGS["a"], OK_ARGS["b"], OK_ARGS["sfa"], OK_ARGS["sfb"],
                                      OK_ARGS["c"], M, K, L, layout, ctypes.byref(st), 1.0, None, 0, None)


def test_dense_strides():
    assert g.nvfp4_gemv_dense_strides(1000, 4096, 3, 0) == dict(
        a_row=2048, a_batch=1000 * 2048, b_batch=2048, sfa_row=256, sfa_batch=1000 * 256,
        sfb_batch=256, c_batch=1000)
    d = g.nvfp4_gemv_dense_strides(1000, 4096, 3, 1)
    assert d["sfa_batch"] == 8 * 64 * 512 and d["sfb_batch"] == 64 * 512


@pytest.mark.parametrize("layout,over", [
    (1, dict(a_row=2047)), (1, dict(a_row=2056)), (1, dict(a_batch=8)), (1, dict(b_batch=-16)),
    (1, dict(sfa_batch=8)), (1, dict(sfb_batch=4)), (1, dict(c_batch=999)),
    (0, dict(sfa_row=255)), (0, dict(sfa_row=257)), (0, dict(sfa_batch=3)), (0, dict(sfb_batch=1)),
    (1, dict(a_row=2 ** 24)), (1, dict(a_batch=2 ** 41))])
def test_strided_rejects_bad_strides(layout, over):
    assert strided_call(layout, **over) == g.NVFP4_ERR_INVALID_STRIDE


def test_strided_null_strides_and_order():
    lib = g.lib()
    args = (OK_ARGS["a"], OK_ARGS["b"], OK_ARGS["sfa"], OK_ARGS["sfb"], OK_ARGS["c"], 128, 256, 1, 0)
    assert lib.nvfp4_gemv_strided(*args, None, 1.0, None, 0, None) == g.NVFP4_ERR_NULL_POINTER
    # shape errors come first, then NULL strides
    bad = (OK_ARGS["a"], OK_ARGS["b"], OK_ARGS["sfa"], OK_ARGS["sfb"], OK_ARGS["c"], 128, 48, 1, 0)
    assert lib.nvfp4_gemv_strided(*bad, None, 1.0, None, 0, None) == g.NVFP4_ERR_INVALID_SHAPE


@no_gpu_only
def test_strided_cases_pass_validation():
    from test_kernel_bounds import STRIDED
    for M, K, L, layout, over in STRIDED:
        st = strided_call(layout, M, K, L, **over)
        assert st not in (g.NVFP4_ERR_INVALID_STRIDE, g.NVFP4_ERR_INVALID_SHAPE, g.NVFP4_ERR_MISALIGNED), \
            (M, K, L, layout, over)


def test_small_n_validation():
    lib = g.lib()
    base = (OK_ARGS["a"], OK_ARGS["b"], OK_ARGS["sfa"], OK_ARGS["sfb"], OK_ARGS["c"])
    assert lib.nvfp4_gemm_small_n(*base, 128, 0, 256, 1, 0, 1.0, None) == g.NVFP4_ERR_INVALID_SHAPE
    assert lib.nvfp4_gemm_small_n(*base, 128, 9, 256, 1, 0, 1.0, None) == g.NVFP4_ERR_INVALID_SHAPE
    assert lib.nvfp4_gemm_small_n(*base, 128, 2, 48, 1, 0, 1.0, None) == g.NVFP4_ERR_INVALID_SHAPE
    assert lib.nvfp4_gemm_small_n(*base, 128, 2, 256, 1, 5, 1.0, None) == g.NVFP4_ERR_INVALID_LAYOUT
    assert lib.nvfp4_gemm_small_n(*base, 128, 2, 256, 1, 0, float("nan"), None) == g.NVFP4_ERR_INVALID_SCALE
    bad = (OK_ARGS["a"] + 8,) + base[1:]
    assert lib.nvfp4_gemm_small_n(*bad, 128, 2, 256, 1, 0, 1.0, None) == g.NVFP4_ERR_MISALIGNED
    assert lib.nvfp4_gemm_small_n(None, *base[1:], 128, 2, 256, 1, 0, 1.0, None) == g.NVFP4_ERR_NULL_POINTER


def test_small_n_plan():
    # N <= 2 with plain scales: the dot-product kernel, one workgroup per CU
    p = g.nvfp4_gemm_small_n_plan(7168, 2, 16384, 1, "plain")
    assert p["workgroups"] == 256 and p["rows_per_wg"] == 28
    p = g.nvfp4_gemm_small_n_plan(100000, 2, 64, 1, "plain")
    assert p["lds_bytes"] <= 48 * 1024
    # N = 2 with blocked scales: the streamed matrix-core kernel from 128 workgroups on
    p = g.nvfp4_gemm_small_n_plan(7168, 2, 16384, 1, "blocked")
    assert p["workgroups"] == 224 and p["lds_bytes"] == 3 * 32 * (64 * 4 + 256 + 8 * 4)
    # below 128 workgroups N = 2 keeps the dot-product kernel's plan (R rows, N sums per wave in LDS)
    p = g.nvfp4_gemm_small_n_plan(127, 2, 16384, 3, "blocked")
    assert p["workgroups"] == 192 and p["lds_bytes"] == p["rows_per_wg"] * 2 * 4 * 4
    # N >= 3, plain scales: the matrix-core kernel, 32-row tiles per workgroup, static LDS only
    p = g.nvfp4_gemm_small_n_plan(7168, 8, 16384, 1, "plain")
    assert p["workgroups"] == 224 and p["rows_per_wg"] == 32 and p["lds_bytes"] == 0
    p = g.nvfp4_gemm_small_n_plan(7, 3, 96, 2, "plain")
    assert p["workgroups"] == 2 and p["rows_per_wg"] == 7
    # blocked scales: the staged kernel, 4 workgroups per 128-row block, B and the scales in LDS
    p = g.nvfp4_gemm_small_n_plan(7168, 8, 16384, 1, "blocked")
    assert p["workgroups"] == 224 and p["rows_per_wg"] == 32 and 0 < p["lds_bytes"] <= 96 * 1024
    p = g.nvfp4_gemm_small_n_plan(7, 3, 96, 2, "blocked")
    assert p["workgroups"] == 8 and p["rows_per_wg"] == 7 and p["lds_bytes"] > 0
    p = g.nvfp4_gemm_small_n_plan(1000, 4, 4096, 3, "blocked")
    assert p["workgroups"] == 3 * 8 * 4
    # the staged kernel's LDS does not depend on K: three slots of one block of 32 K-steps
    p = g.nvfp4_gemm_small_n_plan(300, 4, 40960, 1, "blocked")
    assert p["workgroups"] == 12 and p["lds_bytes"] == 3 * 32 * (64 * 4 + 256 + 8 * 4)
    p = g.nvfp4_gemm_small_n_plan(300, 5, 40960, 1, "blocked")
    assert p["lds_bytes"] == 3 * 32 * (64 * 8 + 256 + 8 * 8)
    with pytest.raises(g.Nvfp4Error):
        g.nvfp4_gemm_small_n_plan(128, 9, 256, 1)
    with pytest.raises(g.Nvfp4Error):
        g.nvfp4_gemm_small_n_plan(128, 4, 256, 1, 7)


def test_noalloc_validation_before_launch():
    lib = g.lib()
    args = [OK_ARGS["a"], OK_ARGS["b"], OK_ARGS["sfa"], OK_ARGS["sfb"], OK_ARGS["c"], 128, 256, 1, 0, None]
    bad = list(args)
    bad[0] = None
    assert lib.nvfp4_gemv_noalloc(*bad) == g.NVFP4_ERR_NULL_POINTER
    bad = list(args)
    bad[6] = 48
    assert lib.nvfp4_gemv_noalloc(*bad) == g.NVFP4_ERR_INVALID_SHAPE
    bad = list(args)
    bad[4] = OK_ARGS["c"] + 1
    assert lib.nvfp4_gemv_noalloc(*bad) == g.NVFP4_ERR_MISALIGNED
    bad = list(args)
    bad[8] = 7
    assert lib.nvfp4_gemv_noalloc(*bad) == g.NVFP4_ERR_INVALID_LAYOUT
    assert lib.nvfp4_gemv_noalloc_scratch_bytes() == 64 * 1024
