"""Python binding of the MI355X NVFP4 block-scaled batched GEMV (libnvfp4gemv.so).

Argument marshalling only: every step of the GEMV runs in the HIP library. The
names mirror the C ABI in include/nvfp4_gemv.h. torch provides device memory and
the stream; tensors are passed as raw device pointers.

    nvfp4_gemv(a, b, sfa, sfb, c, M, K, L, sf_layout, stream=None)
    nvfp4_gemv_scaled(..., sf_layout, alpha, workspace=None, stream=None)
    nvfp4_scales_to_blocked(plain, blocked, rows, K, L, stream=None)

    a   uint8 [L, M, K/2]   packed E2M1, low nibble = even k
    b   uint8 [L, K/2]
    sfa uint8 plain [L, M, K/16] or blocked [L, ceil(M/128)*ceil(K/64)*512]
    sfb uint8 plain [L, K/16]    or blocked [L, ceil(K/64)*512]
    c   float16 [L, M]          written

There is no fallback: if the library is missing the import fails.
"""
from __future__ import annotations

import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libnvfp4gemv.so")

NVFP4_SF_PLAIN = 0
NVFP4_SF_BLOCKED = 1
NVFP4_OK = 0
NVFP4_ERR_NULL_POINTER = 1
NVFP4_ERR_INVALID_SHAPE = 2
NVFP4_ERR_MISALIGNED = 3
NVFP4_ERR_INVALID_LAYOUT = 4
NVFP4_ERR_WORKSPACE = 5
NVFP4_ERR_HIP = 6
NVFP4_ERR_INVALID_SCALE = 7
NVFP4_ERR_INVALID_STRIDE = 8

EXPORTED_SYMBOLS = (
    "nvfp4_gemv",
    "nvfp4_gemv_noalloc",
    "nvfp4_gemv_noalloc_scratch_bytes",
    "nvfp4_gemv_workspace_bytes",
    "nvfp4_gemv_ex",
    "nvfp4_gemv_scaled",
    "nvfp4_gemv_strided",
    "nvfp4_gemv_dense_strides",
    "nvfp4_gemv_plan",
    "nvfp4_gemv_two_vectors_plan",
    "nvfp4_gemm_small_n",
    "nvfp4_gemm_small_n_plan",
    "nvfp4_scales_to_blocked",
    "nvfp4_blocked_scales_bytes",
    "nvfp4_status_string",
    "nvfp4_last_hip_error",
)


class Nvfp4Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = status_string(status)
        if status == NVFP4_ERR_HIP:
            msg += f" (hipError_t {lib().nvfp4_last_hip_error()})"
        super().__init__(f"{where}: {msg} [status {status}]")


class Strides(ctypes.Structure):
    """nvfp4_strides_t: byte strides (c_batch in float16 elements)."""
    _fields_ = [("a_row", ctypes.c_int64), ("a_batch", ctypes.c_int64),
                ("b_batch", ctypes.c_int64),
                ("sfa_row", ctypes.c_int64), ("sfa_batch", ctypes.c_int64),
                ("sfb_batch", ctypes.c_int64),
                ("c_batch", ctypes.c_int64)]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


class Plan(ctypes.Structure):
    _fields_ = [("lanes_per_row", ctypes.c_int32),
                ("rows_per_wg", ctypes.c_int32),
                ("k_splits", ctypes.c_int32),
                ("k_per_split", ctypes.c_int32),
                ("workgroups", ctypes.c_int64),
                ("threads_per_wg", ctypes.c_int32),
                ("lds_bytes", ctypes.c_int32)]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


_lib = None


def lib():
    """The loaded C library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m block_scaled_fp4_gemv_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.nvfp4_gemv.restype = i32
    L.nvfp4_gemv.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, vp]
    L.nvfp4_gemv_ex.restype = i32
    L.nvfp4_gemv_noalloc.restype = i32
    L.nvfp4_gemv_noalloc.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, vp]
    L.nvfp4_gemv_noalloc_scratch_bytes.restype = ctypes.c_size_t
    L.nvfp4_gemv_noalloc_scratch_bytes.argtypes = []
    L.nvfp4_gemv_ex.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, vp, ctypes.c_size_t, vp]
    L.nvfp4_gemv_scaled.restype = i32
    L.nvfp4_gemv_scaled.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, ctypes.c_float, vp,
                                    ctypes.c_size_t, vp]
    L.nvfp4_gemv_strided.restype = i32
    L.nvfp4_gemv_strided.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, ctypes.POINTER(Strides),
                                     ctypes.c_float, vp, ctypes.c_size_t, vp]
    L.nvfp4_gemv_dense_strides.restype = None
    L.nvfp4_gemv_dense_strides.argtypes = [i64, i64, i64, i32, ctypes.POINTER(Strides)]
    L.nvfp4_gemv_workspace_bytes.restype = ctypes.c_size_t
    L.nvfp4_gemv_workspace_bytes.argtypes = [i64, i64, i64]
    L.nvfp4_gemv_plan.restype = i32
    L.nvfp4_gemv_plan.argtypes = [i64, i64, i64, ctypes.POINTER(Plan)]
    L.nvfp4_gemv_two_vectors_plan.restype = i32
    L.nvfp4_gemv_two_vectors_plan.argtypes = [i64, i64, i64, ctypes.POINTER(Plan)]
    L.nvfp4_gemm_small_n.restype = i32
    L.nvfp4_gemm_small_n.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, ctypes.c_float, vp]
    L.nvfp4_gemm_small_n_plan.restype = i32
    L.nvfp4_gemm_small_n_plan.argtypes = [i64, i64, i64, i64, i32, ctypes.POINTER(ctypes.c_int32),
                                          ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int32)]
    L.nvfp4_scales_to_blocked.restype = i32
    L.nvfp4_scales_to_blocked.argtypes = [vp, vp, i64, i64, i64, vp]
    L.nvfp4_blocked_scales_bytes.restype = ctypes.c_size_t
    L.nvfp4_blocked_scales_bytes.argtypes = [i64, i64, i64]
    L.nvfp4_status_string.restype = ctypes.c_char_p
    L.nvfp4_status_string.argtypes = [i32]
    L.nvfp4_last_hip_error.restype = i32
    L.nvfp4_last_hip_error.argtypes = []
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().nvfp4_status_string(status).decode()


def layout_id(layout) -> int:
    if layout in (NVFP4_SF_PLAIN, "plain"):
        return NVFP4_SF_PLAIN
    if layout in (NVFP4_SF_BLOCKED, "blocked"):
        return NVFP4_SF_BLOCKED
    return int(layout)   # passed through; the library rejects unknown values


def cdiv(a: int, b: int) -> int:
    return (a + b - 1) // b


def operand_bytes(M: int, K: int, L: int, layout) -> dict:
    """Bytes each operand must hold for a shape."""
    lay = layout_id(layout)
    nkb = K // 16
    if lay == NVFP4_SF_BLOCKED:
        sfa = L * cdiv(M, 128) * cdiv(nkb, 4) * 512
        sfb = L * cdiv(nkb, 4) * 512
    else:
        sfa, sfb = L * M * nkb, L * nkb
    return {"a": L * M * K // 2, "b": L * K // 2, "sfa": sfa, "sfb": sfb, "c": 2 * L * M}


def _ptr_and_bytes(x):
    """(device pointer, byte size) of a torch tensor, or (x, None) for a raw int."""
    if x is None:
        return None, None
    if isinstance(x, int):
        return x, None
    if not x.is_cuda:
        raise ValueError("operands must be device tensors")
    if not x.is_contiguous():
        raise ValueError("operands must be contiguous")
    return x.data_ptr(), x.numel() * x.element_size()


def _stream_handle(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check_sizes(M, K, L, layout, **ops):
    if M < 1 or K < 1 or L < 1 or K % 32:
        return   # the library reports shape errors itself
    need = operand_bytes(M, K, L, layout)
    for name, nbytes in ops.items():
        if nbytes is not None and nbytes < need[name]:
            raise ValueError(f"{name} holds {nbytes} bytes, the shape needs {need[name]}")


def nvfp4_gemv(a, b, sfa, sfb, c, M: int, K: int, L: int, sf_layout, stream=None) -> None:
    """Enqueue c = GEMV(a, b, sfa, sfb) on ``stream`` (default: torch's current stream)."""
    (pa, na), (pb, nb), (psa, nsa), (psb, nsb), (pc, nc) = map(_ptr_and_bytes, (a, b, sfa, sfb, c))
    lay = layout_id(sf_layout)
    _check_sizes(M, K, L, lay, a=na, b=nb, sfa=nsa, sfb=nsb, c=nc)
    st = lib().nvfp4_gemv(pa, pb, psa, psb, pc, M, K, L, lay, _stream_handle(stream))
    if st != NVFP4_OK:
        raise Nvfp4Error(st, "nvfp4_gemv")


def nvfp4_gemv_noalloc(a, b, sfa, sfb, c, M: int, K: int, L: int, sf_layout, stream=None) -> None:
    """As nvfp4_gemv, with the split-K workspace taken from the library's fixed
    per-device scratch array (no allocation; calls on one GPU must not overlap)."""
    (pa, na), (pb, nb), (psa, nsa), (psb, nsb), (pc, nc) = map(_ptr_and_bytes, (a, b, sfa, sfb, c))
    lay = layout_id(sf_layout)
    _check_sizes(M, K, L, lay, a=na, b=nb, sfa=nsa, sfb=nsb, c=nc)
    st = lib().nvfp4_gemv_noalloc(pa, pb, psa, psb, pc, M, K, L, lay, _stream_handle(stream))
    if st != NVFP4_OK:
        raise Nvfp4Error(st, "nvfp4_gemv_noalloc")


def nvfp4_gemv_noalloc_scratch_bytes() -> int:
    return int(lib().nvfp4_gemv_noalloc_scratch_bytes())


def nvfp4_gemv_workspace_bytes(M: int, K: int, L: int) -> int:
    return int(lib().nvfp4_gemv_workspace_bytes(M, K, L))


def nvfp4_gemv_ex(a, b, sfa, sfb, c, M: int, K: int, L: int, sf_layout, workspace,
                  workspace_bytes: int | None = None, stream=None) -> None:
    """As nvfp4_gemv with a caller-owned (zero-initialised) workspace."""
    (pa, na), (pb, nb), (psa, nsa), (psb, nsb), (pc, nc) = map(_ptr_and_bytes, (a, b, sfa, sfb, c))
    pw, nw = _ptr_and_bytes(workspace)
    if workspace_bytes is None:
        workspace_bytes = nw or 0
    lay = layout_id(sf_layout)
    _check_sizes(M, K, L, lay, a=na, b=nb, sfa=nsa, sfb=nsb, c=nc)
    st = lib().nvfp4_gemv_ex(pa, pb, psa, psb, pc, M, K, L, lay, pw, workspace_bytes,
                             _stream_handle(stream))
    if st != NVFP4_OK:
        raise Nvfp4Error(st, "nvfp4_gemv_ex")


def nvfp4_gemv_scaled(a, b, sfa, sfb, c, M: int, K: int, L: int, sf_layout, alpha: float,
                      workspace=None, workspace_bytes: int | None = None, stream=None) -> None:
    """Enqueue c = fp16(alpha * GEMV(a, b, sfa, sfb)); ``workspace`` None uses
    the library-owned one, else a caller-owned (zero-initialised) workspace."""
    (pa, na), (pb, nb), (psa, nsa), (psb, nsb), (pc, nc) = map(_ptr_and_bytes, (a, b, sfa, sfb, c))
    pw, nw = _ptr_and_bytes(workspace)
    if workspace_bytes is None:
        workspace_bytes = nw or 0
    lay = layout_id(sf_layout)
    _check_sizes(M, K, L, lay, a=na, b=nb, sfa=nsa, sfb=nsb, c=nc)
    st = lib().nvfp4_gemv_scaled(pa, pb, psa, psb, pc, M, K, L, lay, float(alpha), pw,
                                 workspace_bytes, _stream_handle(stream))
    if st != NVFP4_OK:
        raise Nvfp4Error(st, "nvfp4_gemv_scaled")


def nvfp4_gemv_dense_strides(M: int, K: int, L: int, sf_layout) -> dict:
    st = Strides()
    lib().nvfp4_gemv_dense_strides(M, K, L, layout_id(sf_layout), ctypes.byref(st))
    return st.as_dict()


def _raw_ptr(x):
    """Device pointer of a torch tensor (any strides: the library reads through
    the strides it is given), or a raw int."""
    if x is None or isinstance(x, int):
        return x
    if not x.is_cuda:
        raise ValueError("operands must be device tensors")
    return x.data_ptr()


def nvfp4_gemv_strided(a, b, sfa, sfb, c, M: int, K: int, L: int, sf_layout, strides: dict,
                       alpha: float = 1.0, workspace=None, workspace_bytes: int | None = None,
                       stream=None) -> None:
    """Enqueue c = fp16(alpha * GEMV) over strided operands: ``strides`` holds
    the fields of nvfp4_strides_t (bytes; c_batch in elements). The tensors
    are passed by base pointer: the library reads and writes through the
    strides, so each tensor must cover what they address."""
    st = Strides(**strides)
    pw, nw = _ptr_and_bytes(workspace)
    if workspace_bytes is None:
        workspace_bytes = nw or 0
    rc = lib().nvfp4_gemv_strided(_raw_ptr(a), _raw_ptr(b), _raw_ptr(sfa), _raw_ptr(sfb), _raw_ptr(c),
                                  M, K, L, layout_id(sf_layout), ctypes.byref(st), float(alpha), pw,
                                  workspace_bytes, _stream_handle(stream))
    if rc != NVFP4_OK:
        raise Nvfp4Error(rc, "nvfp4_gemv_strided")


def nvfp4_gemv_plan(M: int, K: int, L: int) -> dict:
    plan = Plan()
    st = lib().nvfp4_gemv_plan(M, K, L, ctypes.byref(plan))
    if st != NVFP4_OK:
        raise Nvfp4Error(st, "nvfp4_gemv_plan")
    return plan.as_dict()


def nvfp4_gemv_two_vectors_plan(M: int, K: int, L: int) -> dict:
    plan = Plan()
    st = lib().nvfp4_gemv_two_vectors_plan(M, K, L, ctypes.byref(plan))
    if st != NVFP4_OK:
        raise Nvfp4Error(st, "nvfp4_gemv_two_vectors_plan")
    return plan.as_dict()


def nvfp4_gemm_small_n_plan(M: int, N: int, K: int, L: int, layout="blocked") -> dict:
    r, wg, lds = ctypes.c_int32(), ctypes.c_int64(), ctypes.c_int32()
    st = lib().nvfp4_gemm_small_n_plan(M, N, K, L, layout_id(layout), ctypes.byref(r), ctypes.byref(wg),
                                       ctypes.byref(lds))
    if st != NVFP4_OK:
        raise Nvfp4Error(st, "nvfp4_gemm_small_n_plan")
    return {"rows_per_wg": r.value, "workgroups": wg.value, "lds_bytes": lds.value}


def small_n_operand_bytes(M: int, N: int, K: int, L: int, layout) -> dict:
    """Bytes each operand of nvfp4_gemm_small_n must hold."""
    lay = layout_id(layout)
    nkb = K // 16
    if lay == NVFP4_SF_BLOCKED:
        sfa, sfb = L * cdiv(M, 128) * cdiv(nkb, 4) * 512, L * cdiv(N, 128) * cdiv(nkb, 4) * 512
    else:
        sfa, sfb = L * M * nkb, L * N * nkb
    return {"a": L * M * K // 2, "b": L * N * K // 2, "sfa": sfa, "sfb": sfb, "c": 2 * L * N * M}


def nvfp4_gemm_small_n(a, b, sfa, sfb, c, M: int, N: int, K: int, L: int, sf_layout,
                       alpha: float = 1.0, stream=None) -> None:
    """Enqueue c[l][n][m] = fp16(alpha * sum_k A*SFA*B_n*SFB_n) for N = 1..8 vectors."""
    (pa, na), (pb, nb), (psa, nsa), (psb, nsb), (pc, nc) = map(_ptr_and_bytes, (a, b, sfa, sfb, c))
    lay = layout_id(sf_layout)
    if M >= 1 and K >= 32 and K % 32 == 0 and L >= 1 and 1 <= N <= 8:
        need = small_n_operand_bytes(M, N, K, L, lay)
        for name, nbytes in dict(a=na, b=nb, sfa=nsa, sfb=nsb, c=nc).items():
            if nbytes is not None and nbytes < need[name]:
                raise ValueError(f"{name} holds {nbytes} bytes, the shape needs {need[name]}")
    st = lib().nvfp4_gemm_small_n(pa, pb, psa, psb, pc, M, N, K, L, lay, float(alpha), _stream_handle(stream))
    if st != NVFP4_OK:
        raise Nvfp4Error(st, "nvfp4_gemm_small_n")


def nvfp4_blocked_scales_bytes(rows: int, K: int, L: int) -> int:
    return int(lib().nvfp4_blocked_scales_bytes(rows, K, L))


def nvfp4_scales_to_blocked(plain, blocked, rows: int, K: int, L: int, stream=None) -> None:
    """Enqueue the plain -> 128x4 blocked reblock of a scale tensor.
    plain uint8 [L, rows, K/16]; blocked uint8 of nvfp4_blocked_scales_bytes bytes."""
    (pp, npb), (pb, nbb) = _ptr_and_bytes(plain), _ptr_and_bytes(blocked)
    need = nvfp4_blocked_scales_bytes(rows, K, L)
    if need and npb is not None and npb < L * rows * (K // 16):
        raise ValueError(f"plain holds {npb} bytes, the shape needs {L * rows * (K // 16)}")
    if need and nbb is not None and nbb < need:
        raise ValueError(f"blocked holds {nbb} bytes, the shape needs {need}")
    st = lib().nvfp4_scales_to_blocked(pp, pb, rows, K, L, _stream_handle(stream))
    if st != NVFP4_OK:
        raise Nvfp4Error(st, "nvfp4_scales_to_blocked")


def nvfp4_status_string(status: int) -> str:
    return status_string(status)


def nvfp4_last_hip_error() -> int:
    return int(lib().nvfp4_last_hip_error())
