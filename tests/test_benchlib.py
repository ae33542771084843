"""CPU checks of the bench's measurement library: it loads, exports its two
symbols, and rejects bad arguments before any HIP call."""
from block_scaled_fp4_gemv_amd import benchlib

A16 = 0x10000


def test_exports_and_unit():
    L = benchlib.lib()
    assert hasattr(L, "nvfp4bench_stream_read") and hasattr(L, "nvfp4bench_stream_read_unit")
    assert [benchlib.stream_read_unit(m) for m in range(4)] == [2 ** 20, 4 * 2 ** 20, 2 ** 20, 4 * 2 ** 20]


def test_validation_before_launch():
    L = benchlib.lib()
    mode = 1
    u = benchlib.stream_read_unit(mode)
    assert L.nvfp4bench_stream_read(None, u, A16, mode, None) == 1
    assert L.nvfp4bench_stream_read(A16, u, None, mode, None) == 1
    for bad in (0, u - 16, u + 4096, u + 2 ** 20):
        assert L.nvfp4bench_stream_read(A16, bad, A16, mode, None) == 2
    assert L.nvfp4bench_stream_read(A16, u, A16, 4, None) == 2
    assert L.nvfp4bench_stream_read(A16, u, A16, -1, None) == 2
    assert L.nvfp4bench_stream_read(A16 + 8, u, A16, mode, None) == 3
    assert L.nvfp4bench_stream_read(A16, u, A16 + 2, mode, None) == 3
