// Streaming-read reference kernel for MI355X (gfx950): reads a buffer once,
// in the same access pattern as the GEMV's A stream and with nothing else to
// do, so that the bench can state how far the GEMV is from what a plain read
// of the same byte count attains on the same machine (launch and ramp costs
// included). It computes nothing that anyone uses.
//
// 256 workgroups of 4 waves; workgroup w reads the w-th of 256 equal slices.
// Inside a slice the four waves take 1 KiB pieces in turn (wave v: pieces v,
// v+4, ...), every lane 16 bytes per piece, with a ring of 8 non-temporal
// loads in flight per lane (32 KiB per workgroup), the depth that measured
// best for this pattern.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "nvfp4_gemv.h"
#include "nvfp4_internal.h"
#include "nvfp4_device.h"

namespace {

constexpr int kReadWGs = 256;
constexpr int kReadThreads = 256;
constexpr int kReadDepth = 8;
constexpr int kPiece = 1024;                  // bytes one wave-wide 16-byte load covers
constexpr uint32_t kMagic = 0x9E3779B9u;      // the sink is written only if a lane's XOR equals this

__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const uint8_t *__restrict__ src,
                                                                   int32_t slice_bytes,
                                                                   uint32_t *__restrict__ sink)
{
    const uint32_t w = xcd_remap(blockIdx.x, kReadWGs);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(src + (int64_t)w * slice_bytes), (short)0, slice_bytes, 0x00020000);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int npieces = slice_bytes / kPiece;
    constexpr int nw = kReadThreads / 64;
    uint4_t ring[kReadDepth];
    uint4_t acc = {0u, 0u, 0u, 0u};
    int p = wave;
#pragma unroll
    for (int d = 0; d < kReadDepth; ++d) {
        ring[d] = __builtin_amdgcn_raw_buffer_load_b128(rs, min(p, npieces - 1) * kPiece + lane * 16, 0, 2);
        p += nw;
    }
    for (int it = 0; it < npieces; it += nw * kReadDepth) {
#pragma unroll
        for (int d = 0; d < kReadDepth; ++d) {
            acc ^= ring[d];
            __builtin_amdgcn_sched_barrier(0);
            ring[d] = __builtin_amdgcn_raw_buffer_load_b128(rs, min(p, npieces - 1) * kPiece + lane * 16, 0, 2);
            p += nw;
        }
    }
#pragma unroll
    for (int d = 0; d < kReadDepth; ++d)
        acc ^= ring[d];
    const uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (x == kMagic)
        sink[blockIdx.x] = x;
}

} // namespace

extern "C" nvfp4_status_t nvfp4_stream_read(const void *src, size_t bytes, void *sink, void *stream)
{
    if (!src || !sink)
        return NVFP4_ERR_NULL_POINTER;
    const size_t unit = (size_t)kReadWGs * kPiece;
    if (bytes == 0 || bytes % unit != 0 || bytes / kReadWGs > (size_t)INT32_MAX)
        return NVFP4_ERR_INVALID_SHAPE;
    if (((uintptr_t)src & 15) != 0 || ((uintptr_t)sink & 3) != 0)
        return NVFP4_ERR_MISALIGNED;
    hipLaunchKernelGGL(stream_read_kernel, dim3(kReadWGs), dim3(kReadThreads), 0, (hipStream_t)stream,
                       (const uint8_t *)src, (int32_t)(bytes / kReadWGs), (uint32_t *)sink);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        nvfp4_record_hip_error((int)e);
        return NVFP4_ERR_HIP;
    }
    return NVFP4_OK;
}
