/*
 * nvfp4_bench.h -- measurement helper library (libnvfp4bench.so), not part of
 * the GEMV library or its C ABI.
 *
 * nvfp4bench_stream_read: one streaming read of `bytes` device bytes at `src`
 * (16-byte aligned), a multiple of nvfp4bench_stream_read_unit(mode); `sink` is a
 * device array of 256 uint32 that the kernel writes only in a data-dependent
 * case that zero or random data practically never meets. `mode` picks the
 * read design (0..3, see stream_read.hip). Only enqueues on `stream`.
 * Returns 0, or 1 (NULL pointer), 2 (size or mode), 3 (alignment), 4 (launch).
 */
#ifndef NVFP4_BENCH_H
#define NVFP4_BENCH_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

size_t nvfp4bench_stream_read_unit(int mode);
int nvfp4bench_stream_read(const void *src, size_t bytes, void *sink, int mode, void *stream);

#ifdef __cplusplus
}
#endif

#endif
