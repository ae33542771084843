// Streaming-read reference for MI355X (gfx950): reads a buffer once and
// computes nothing anyone uses, so that the bench can state what a plain read
// of a given byte count attains on the same machine, with the same launch and
// timing method as the GEMV (launch and ramp costs included). Measurement
// only: this is libnvfp4bench.so, not part of the GEMV library or its C ABI.
//
// 256 workgroups of 4 waves (one per CU). A "step" is 4 KiB: each wave reads
// 1 KiB of it, 16 bytes per lane. Designs (mode):
//   0  register ring, 8 steps in flight per wave; workgroup w reads the w-th
//      of 256 contiguous slices
//   1  register ring as 0; 16 KiB units dealt round-robin to the workgroups,
//      so that the whole chip reads one window of the buffer at a time
//   2  direct-to-LDS copies (global_load_lds_dwordx4), 8 in flight per wave
//      (a ring of 8 KiB of LDS per wave, never read); contiguous slices
//   3  direct-to-LDS copies as 2; 16 KiB units dealt round-robin
// All loads are non-temporal. Every wave issues exactly its own steps: the
// register ring clamps its last prefetches onto its last step (an L2 hit).

#include <hip/hip_runtime.h>

#include <cstdint>

#include "nvfp4_bench.h"

namespace {

constexpr int kWGs = 256;
constexpr int kWaves = 4;
constexpr int kDepth = 8;                     // steps in flight per wave
constexpr int kStep = kWaves * 1024;          // bytes of one step
constexpr int kUnitSteps = 4;                 // 16 KiB units in the round-robin designs
constexpr uint32_t kMagic = 0x9E3779B9u;      // the sink is written only if a lane's XOR equals this

typedef uint32_t u4 __attribute__((ext_vector_type(4)));

// Contiguous ids per XCD: hardware id i runs on XCD i % 8.
__device__ inline uint32_t xcd_remap(uint32_t i, uint32_t n)
{
    const uint32_t x = i % 8, j = i / 8, q = n / 8, r = n % 8;
    return x * q + min(x, r) + j;
}

// Byte offset of step i (0 <= i < n) of workgroup w.
template <bool RR>
__device__ inline int64_t step_offset(uint32_t w, int32_t i, int32_t per_wg)
{
    if (RR)
        return ((int64_t)(w + (uint32_t)(i / kUnitSteps) * kWGs) * kUnitSteps + i % kUnitSteps) * kStep;
    return ((int64_t)w * per_wg + i) * kStep;
}

template <bool LDS, bool RR>
__global__ __launch_bounds__(kWaves * 64) void stream_read_kernel(const uint8_t *__restrict__ src, int32_t per_wg,
                                                                  uint32_t *__restrict__ sink)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const uint32_t w = xcd_remap(blockIdx.x, kWGs);
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int lane = (int)(threadIdx.x & 63);
    const uint8_t *base = src + wave * 1024 + lane * 16;
    const int32_t n = per_wg;                      // steps of this workgroup (every workgroup has as many;
                                                   // a multiple of kUnitSteps in the round-robin designs)
    if (LDS) {
        const uint32_t ring = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds) + wave * (kDepth * 1024);
        for (int32_t i = 0; i < n; ++i) {
            if (i >= kDepth)
                asm volatile("s_waitcnt vmcnt(%0)" : : "n"(kDepth - 1) : "memory");
            const uint8_t *p = base + step_offset<RR>(w, i, per_wg);
            asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt" : : "v"(p),
                         "s"(ring + (uint32_t)(i % kDepth) * 1024u) : "memory", "m0");
        }
        asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
        return;
    }
    u4 ring[kDepth];
    u4 acc = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int d = 0; d < kDepth; ++d)
        ring[d] = __builtin_nontemporal_load((const u4 *)(base + step_offset<RR>(w, min(d, n - 1), per_wg)));
    for (int32_t i = 0; i < n; i += kDepth) {
#pragma unroll
        for (int d = 0; d < kDepth; ++d) {
            acc ^= ring[d];
            __builtin_amdgcn_sched_barrier(0);
            ring[d] = __builtin_nontemporal_load(
                (const u4 *)(base + step_offset<RR>(w, min(i + kDepth + d, n - 1), per_wg)));
        }
    }
#pragma unroll
    for (int d = 0; d < kDepth; ++d)
        acc ^= ring[d];
    const uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (x == kMagic)
        sink[blockIdx.x] = x;
}

} // namespace

extern "C" {

size_t nvfp4bench_stream_read_unit(int mode)
{
    // one step per workgroup (contiguous designs), one 16 KiB unit per workgroup (round-robin)
    return (size_t)kWGs * kStep * ((mode & 1) ? kUnitSteps : 1);
}

int nvfp4bench_stream_read(const void *src, size_t bytes, void *sink, int mode, void *stream)
{
    if (!src || !sink)
        return 1;
    if (mode < 0 || mode > 3)
        return 2;
    const size_t unit = nvfp4bench_stream_read_unit(mode);
    if (bytes == 0 || bytes % unit != 0 || bytes / kWGs > (size_t)INT32_MAX)
        return 2;
    if (((uintptr_t)src & 15) != 0 || ((uintptr_t)sink & 3) != 0)
        return 3;
    const int32_t per_wg = (int32_t)(bytes / kWGs / kStep);
    const hipStream_t st = (hipStream_t)stream;
    const dim3 grid(kWGs), block(kWaves * 64);
    const uint8_t *s = (const uint8_t *)src;
    uint32_t *k = (uint32_t *)sink;
    switch (mode) {
    case 0: hipLaunchKernelGGL((stream_read_kernel<false, false>), grid, block, 0, st, s, per_wg, k); break;
    case 1: hipLaunchKernelGGL((stream_read_kernel<false, true>), grid, block, 0, st, s, per_wg, k); break;
    case 2: hipLaunchKernelGGL((stream_read_kernel<true, false>), grid, block, kWaves * kDepth * 1024, st, s, per_wg, k); break;
    default: hipLaunchKernelGGL((stream_read_kernel<true, true>), grid, block, kWaves * kDepth * 1024, st, s, per_wg, k); break;
    }
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

} // extern "C"
