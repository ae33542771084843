"""ctypes binding of libnvfp4bench.so, the measurement helper the bench uses
(a streaming read of a buffer in one of several read designs). It is not part
of the GEMV library or its C ABI."""
from __future__ import annotations

import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
BENCH_LIB_PATH = os.path.join(PKG_DIR, "libnvfp4bench.so")

# read designs of nvfp4bench_stream_read (see csrc/bench/stream_read.hip)
STREAM_READ_MODES = {
    0: "register ring, 4 waves x 8 x 16 B per lane, contiguous slice per workgroup",
    1: "register ring, 4 waves x 8 x 16 B per lane, 16 KiB units dealt round-robin",
    2: "direct-to-LDS copies, 4 waves x 8 in flight, contiguous slice per workgroup",
    3: "direct-to-LDS copies, 4 waves x 8 in flight, 16 KiB units dealt round-robin",
}
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(BENCH_LIB_PATH):
            raise ImportError(f"{BENCH_LIB_PATH} is missing: build it with python -m block_scaled_fp4_gemv_amd.build")
        L = ctypes.CDLL(BENCH_LIB_PATH)
        L.nvfp4bench_stream_read_unit.restype = ctypes.c_size_t
        L.nvfp4bench_stream_read_unit.argtypes = [ctypes.c_int]
        L.nvfp4bench_stream_read.restype = ctypes.c_int
        L.nvfp4bench_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                             ctypes.c_void_p]
        _lib = L
    return _lib


def stream_read_unit(mode: int) -> int:
    """Byte granularity of the read in design ``mode``."""
    return int(lib().nvfp4bench_stream_read_unit(mode))


def stream_read(src, nbytes: int, sink, mode: int, stream=None) -> None:
    """Enqueue one streaming read of the first ``nbytes`` bytes of the device
    tensor ``src``; ``sink`` is a device tensor of at least 1024 bytes."""
    if src.numel() * src.element_size() < nbytes:
        raise ValueError(f"src holds fewer than {nbytes} bytes")
    if sink.numel() * sink.element_size() < 1024:
        raise ValueError("sink needs 1024 bytes")
    if stream is None:
        import torch
        stream = torch.cuda.current_stream().cuda_stream
    elif not isinstance(stream, int):
        stream = stream.cuda_stream
    rc = lib().nvfp4bench_stream_read(src.data_ptr(), nbytes, sink.data_ptr(), mode, stream)
    if rc != 0:
        raise RuntimeError(f"nvfp4bench_stream_read returned {rc}")
