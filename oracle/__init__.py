"""CPU oracle for the NVFP4 block-scaled batched GEMV.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
baseline import this package. The GPU library and its Python binding never
import, load or call it, and it shares no code with them (the seeded input
generator in ``synth`` is the only module both sides use).

The arithmetic lives in ``nvfp4_oracle.c`` (plain C, pthreads), built here with
gcc into ``liboracle.so``. This module is a ctypes wrapper plus the parity
tolerance:

    |gpu - oracle| <= 1e-3 * sum_k |a*sfa*b*sfb| + 1 fp16 ulp(oracle)

with the float16 overflow edge handled as described in ``check``.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

PLAIN, BLOCKED = 0, 1
REL_TOL = 1e-3
FP16_MAX = 65504.0
FP16_OVERFLOW_EDGE = 65520.0   # |S| >= this rounds to inf under RNE


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into oracle/liboracle.so."""
    global _lib
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-pthread", "-shared", "-fPIC",
               _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
        _lib = None
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    i64, u8p, vp = ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p
    lib.nvo_e2m1.restype = ctypes.c_double
    lib.nvo_e2m1.argtypes = [ctypes.c_uint]
    lib.nvo_e4m3.restype = ctypes.c_double
    lib.nvo_e4m3.argtypes = [ctypes.c_uint]
    lib.nvo_tables.restype = None
    lib.nvo_tables.argtypes = [vp, vp]
    for name in ("nvo_sf_offset_plain", "nvo_sf_offset_blocked"):
        f = getattr(lib, name)
        f.restype = i64
        f.argtypes = [i64, i64, i64, i64]
    lib.nvo_sf_offset.restype = i64
    lib.nvo_sf_offset.argtypes = [ctypes.c_int, i64, i64, i64, i64]
    lib.nvo_sf_batch_bytes.restype = i64
    lib.nvo_sf_batch_bytes.argtypes = [ctypes.c_int, i64, i64]
    lib.nvo_fp16_round.restype = ctypes.c_uint16
    lib.nvo_fp16_round.argtypes = [ctypes.c_int, ctypes.c_uint64, ctypes.c_int]
    lib.nvo_fp16_from_double.restype = ctypes.c_uint16
    lib.nvo_fp16_from_double.argtypes = [ctypes.c_double]
    lib.nvo_fp16_from_double_n.restype = None
    lib.nvo_fp16_from_double_n.argtypes = [vp, vp, i64]
    lib.nvo_fp16_to_double.restype = ctypes.c_double
    lib.nvo_fp16_to_double.argtypes = [ctypes.c_uint16]
    lib.nvo_gemv.restype = ctypes.c_int
    lib.nvo_gemv.argtypes = [u8p, u8p, u8p, u8p, i64, i64, i64, ctypes.c_int, ctypes.c_float,
                             ctypes.c_int, vp, vp, vp, vp, vp]
    lib.nvo_gemv_rows.restype = ctypes.c_int
    lib.nvo_gemv_rows.argtypes = [u8p, u8p, u8p, u8p, i64, i64, i64, ctypes.c_int, ctypes.c_float,
                                  vp, i64, ctypes.c_int, vp, vp, vp, vp, vp]
    lib.nvo_reblock.restype = ctypes.c_int
    lib.nvo_reblock.argtypes = [vp, i64, i64, i64, vp]
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


# ---------------------------------------------------------------- decode

def e2m1(code: int) -> float:
    return _load().nvo_e2m1(code)


def e4m3(code: int) -> float:
    return _load().nvo_e4m3(code)


def tables():
    """(e2m1 values of codes 0..15, e4m3 values of codes 0..255) as float64."""
    t2 = np.zeros(16, np.float64)
    t8 = np.zeros(256, np.float64)
    _load().nvo_tables(_ptr(t2), _ptr(t8))
    return t2, t8


# ---------------------------------------------------------------- layout

def sf_offset(layout: int, r: int, kb: int, rows: int, nkb: int) -> int:
    return _load().nvo_sf_offset(layout, r, kb, rows, nkb)


def sf_batch_bytes(layout: int, rows: int, nkb: int) -> int:
    return _load().nvo_sf_batch_bytes(layout, rows, nkb)


def gemm_small_n(a, b, sfa, sfb, M: int, N: int, K: int, L: int, nthreads: int = 0,
                 alpha: float = 1.0) -> Result:
    """Oracle of the N-vector skinny GEMM: column n is the GEMV of A against
    vector n. a [L][M][K/2], b [L][N][K/2], plain scales sfa [L][M][K/16],
    sfb [L][N][K/16]. Arrays of the result are [L][N][M]."""
    b = np.asarray(b, np.uint8).reshape(L, N, K // 2)
    sfb = np.asarray(sfb, np.uint8).reshape(L, N, K // 16)
    cols = [gemv_arrays(a, b[:, n], sfa, sfb[:, n], M, K, L, PLAIN, nthreads, alpha) for n in range(N)]
    st = lambda f: np.stack([getattr(r, f) for r in cols], axis=1)
    return Result(st("c"), st("s_f64"), st("s_abs"), st("s_exact"), st("nan"), _alpha32(alpha))


def reblock(plain, rows: int, K: int, L: int) -> np.ndarray:
    """Plain scales [L][rows][K/16] -> blocked bytes [L][per-batch bytes],
    padding 0 (the oracle of the device reblock)."""
    plain = np.ascontiguousarray(plain, dtype=np.uint8)
    if plain.size != L * rows * (K // 16):
        raise ValueError("plain size mismatch")
    per = sf_batch_bytes(BLOCKED, rows, K // 16)
    out = np.zeros(L * per, np.uint8)
    if _load().nvo_reblock(_ptr(plain), rows, K, L, _ptr(out)) != 0:
        raise ValueError("oracle rejected the arguments")
    return out.reshape(L, per)


# ---------------------------------------------------------------- fp16

def fp16_round(neg: bool, mag: int, e2: int) -> int:
    return _load().nvo_fp16_round(int(neg), mag, e2)


def fp16_from_double(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.zeros(x.shape, np.uint16)
    _load().nvo_fp16_from_double_n(_ptr(x), _ptr(out), x.size)
    return out


def fp16_bits_to_double(bits) -> np.ndarray:
    """Decode float16 bit patterns (uint16) to float64 (exact)."""
    bits = np.asarray(bits, dtype=np.uint16)
    return bits.view(np.float16).astype(np.float64)


# ---------------------------------------------------------------- GEMV

@dataclass
class Result:
    c: np.ndarray        # uint16 fp16 bits of alpha * sum, [L][M] (or [n] for row subsets)
    s_f64: np.ndarray    # plain fp64 sum, times alpha
    s_abs: np.ndarray    # fp64 sum of |a*sfa*b*sfb|, times |alpha|
    s_exact: np.ndarray  # exact unscaled sum in units of 2^-20 (int64)
    nan: np.ndarray      # 1 where a NaN scale was met
    alpha: float = 1.0   # global float32 scale the call used

    @property
    def value(self) -> np.ndarray:
        return fp16_bits_to_double(self.c)


def _layout_id(layout) -> int:
    if layout in (PLAIN, "plain"):
        return PLAIN
    if layout in (BLOCKED, "blocked"):
        return BLOCKED
    raise ValueError(layout)


def _alpha32(alpha) -> float:
    """alpha as the float32 the library takes (finite)."""
    with np.errstate(over="ignore"):
        a32 = np.float32(alpha)
    if not np.isfinite(a32):
        raise ValueError("alpha must be a finite float32")
    return float(a32)


def gemv_arrays(a, b, sfa, sfb, M: int, K: int, L: int, layout, nthreads: int = 0,
                alpha: float = 1.0) -> Result:
    """Oracle GEMV on raw byte arrays (batch-outermost layouts, see synth).
    ``alpha`` is the global float32 scale: c = fp16(alpha * sum)."""
    lay = _layout_id(layout)
    alpha = _alpha32(alpha)
    a, b, sfa, sfb = (np.ascontiguousarray(x, dtype=np.uint8) for x in (a, b, sfa, sfb))
    if a.size != L * M * K // 2 or b.size != L * K // 2:
        raise ValueError("A/B size mismatch")
    if sfa.size != L * sf_batch_bytes(lay, M, K // 16) or sfb.size != L * sf_batch_bytes(lay, 1, K // 16):
        raise ValueError("scale size mismatch")
    n = L * M
    c = np.zeros(n, np.uint16)
    s = np.zeros(n, np.float64)
    sa = np.zeros(n, np.float64)
    se = np.zeros(n, np.int64)
    nan = np.zeros(n, np.uint8)
    nth = nthreads if nthreads > 0 else (os.cpu_count() or 1)
    rc = _load().nvo_gemv(_ptr(a), _ptr(b), _ptr(sfa), _ptr(sfb), M, K, L, lay, alpha, nth,
                          _ptr(c), _ptr(s), _ptr(sa), _ptr(se), _ptr(nan))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    shp = (L, M)
    return Result(c.reshape(shp), s.reshape(shp), sa.reshape(shp), se.reshape(shp),
                  nan.reshape(shp), alpha)


def gemv(inp, layout="plain", nthreads: int = 0, alpha: float = 1.0) -> Result:
    """Oracle GEMV of a ``synth.Inputs`` set, reading the scales in ``layout``."""
    w = inp.w
    return gemv_arrays(inp.a, inp.b, inp.sfa(layout), inp.sfb(layout), w.M, w.K, w.L,
                       layout, nthreads, alpha)


def gemv_rows(inp, rows, layout="plain", nthreads: int = 0, alpha: float = 1.0) -> Result:
    """Oracle values of selected flattened rows (l*M + m) only."""
    w = inp.w
    lay = _layout_id(layout)
    alpha = _alpha32(alpha)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    a, b = np.ascontiguousarray(inp.a), np.ascontiguousarray(inp.b)
    sfa, sfb = np.ascontiguousarray(inp.sfa(layout)), np.ascontiguousarray(inp.sfb(layout))
    n = rows.size
    c = np.zeros(n, np.uint16)
    s = np.zeros(n, np.float64)
    sa = np.zeros(n, np.float64)
    se = np.zeros(n, np.int64)
    nan = np.zeros(n, np.uint8)
    nth = nthreads if nthreads > 0 else (os.cpu_count() or 1)
    rc = _load().nvo_gemv_rows(_ptr(a), _ptr(b), _ptr(sfa), _ptr(sfb), w.M, w.K, w.L, lay, alpha,
                               _ptr(rows), n, nth, _ptr(c), _ptr(s), _ptr(sa), _ptr(se), _ptr(nan))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return Result(c, s, sa, se, nan, alpha)


# ---------------------------------------------------------------- tolerance

def ulp16(x) -> np.ndarray:
    """One float16 ulp at the (finite) float16 value x: 2^(floor(log2|x|) - 10)
    for |x| >= 2^-14, else the subnormal spacing 2^-24."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    out = np.full(ax.shape, 2.0 ** -24)
    norm = np.isfinite(ax) & (ax >= 2.0 ** -14)
    out[norm] = np.exp2(np.floor(np.log2(ax[norm])) - 10)
    return out


def check(gpu_bits, ref: Result, rel_tol: float = REL_TOL):
    """Element-wise parity check of GPU float16 bits against the oracle.

    Finite oracle value o: the GPU value g must be finite with
        |g - o| <= rel_tol * s_abs + ulp16(o).
    Overflow edge: the GPU accumulates in fp32, so when the exact (scaled) sum S is
    within rel_tol * s_abs of 65520 (where float16 rounding switches between
    65504 and inf) either +-65504 or +-inf of the sign of S is accepted.
    Infinite oracle value: the GPU must give the same infinity (or the edge
    case above). NaN oracle value (a NaN scale): the GPU must give NaN.
    Signed zeros compare equal.
    Returns a boolean array (True = within tolerance).
    """
    g = fp16_bits_to_double(np.asarray(gpu_bits, dtype=np.uint16).reshape(ref.c.shape))
    o = fp16_bits_to_double(ref.c)
    S = ref.s_exact.astype(np.float64) * 2.0 ** -20 * ref.alpha
    tol = rel_tol * ref.s_abs + ulp16(np.where(np.isfinite(o), o, 0.0))
    ok = np.zeros(o.shape, dtype=bool)

    o_nan = np.isnan(o)
    ok |= o_nan & np.isnan(g)

    edge = (~o_nan) & (np.abs(np.abs(S) - FP16_OVERFLOW_EDGE) <= rel_tol * ref.s_abs)
    same_sign = np.signbit(g) == np.signbit(S)
    edge_ok = edge & same_sign & (np.isinf(g) | (np.abs(g) == FP16_MAX))
    ok |= edge_ok

    fin = (~o_nan) & np.isfinite(o) & np.isfinite(g)
    with np.errstate(invalid="ignore"):
        ok |= fin & (np.abs(g - o) <= tol)
    inf = (~o_nan) & np.isinf(o) & np.isinf(g) & (np.sign(g) == np.sign(o))
    ok |= inf
    return ok


def check_report(gpu_bits, ref: Result, rel_tol: float = REL_TOL, max_show: int = 8) -> str:
    """Human-readable summary of the failures of ``check`` (empty if none)."""
    ok = check(gpu_bits, ref, rel_tol)
    if ok.all():
        return ""
    g = fp16_bits_to_double(np.asarray(gpu_bits, dtype=np.uint16).reshape(ref.c.shape))
    o = fp16_bits_to_double(ref.c)
    bad = np.argwhere(~ok)
    lines = [f"{len(bad)} of {ok.size} outputs outside tolerance"]
    for idx in bad[:max_show]:
        idx = tuple(idx)
        lines.append(f"  at {idx}: gpu={g[idx]!r} oracle={o[idx]!r} "
                     f"S={ref.s_exact[idx] * 2.0 ** -20 * ref.alpha!r} s_abs={ref.s_abs[idx]!r}")
    return "\n".join(lines)
