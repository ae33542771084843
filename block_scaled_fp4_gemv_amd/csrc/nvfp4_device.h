// Device helpers shared by the HIP kernels of libnvfp4gemv.so: E2M1/E4M3
// conversions with gfx950's conversion instructions, DPP lane sums, float16
// rounding and the workgroup-id remap for the 8 XCDs. Internal header.
#ifndef NVFP4_DEVICE_H
#define NVFP4_DEVICE_H

#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

constexpr int kXcdCount = 8;              // MI355X: 8 XCDs, workgroup ids dealt round-robin

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef uint32_t uint4_t __attribute__((ext_vector_type(4)));
typedef uint32_t uint2_t __attribute__((ext_vector_type(2)));

// Contiguous logical ids per XCD: hardware id i runs on XCD i % 8.
__device__ inline uint32_t xcd_remap(uint32_t i, uint32_t n)
{
    const uint32_t x = i % kXcdCount, j = i / kXcdCount;
    const uint32_t q = n / kXcdCount, r = n % kXcdCount;
    return x * q + min(x, r) + j;
}

// Reinterpretation helpers. They take their operand by value on purpose:
// applying __builtin_bit_cast to an ext-vector element such as `v.y` directly
// read the vector's first element with this compiler.
__device__ __attribute__((always_inline)) inline half2_t as_h2(uint32_t v)
{
    return __builtin_bit_cast(half2_t, v);
}
__device__ __attribute__((always_inline)) inline uint32_t as_u32(half2_t v)
{
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __attribute__((always_inline)) inline float as_f32(int v)
{
    return __builtin_bit_cast(float, v);
}
__device__ __attribute__((always_inline)) inline int as_i32(float v)
{
    return __builtin_bit_cast(int, v);
}

// two E2M1 codes (byte SEL of w, low nibble first) -> two float16 values
template <int SEL>
__device__ __attribute__((always_inline)) inline half2_t fp4x2(uint32_t w)
{
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL);
}

// float32 -> float16 bits, round to nearest even, overflow to +-inf
__device__ __attribute__((always_inline)) inline uint16_t f16_bits(float v)
{
    return __builtin_bit_cast(uint16_t, (_Float16)v);
}

// Sum over aligned groups of RED lanes (RED = 1..64, a power of two) with DPP.
// The group's sum ends in its last lane: row_shr accumulates a window of RED
// lanes inside each 16-lane row, row_bcast15 / row_bcast31 carry the row sums
// across rows.
template <int RED>
__device__ __attribute__((always_inline)) inline float group_sum(float v)
{
    if (RED >= 2)
        v += as_f32(__builtin_amdgcn_update_dpp(0, as_i32(v), 0x111, 0xF, 0xF, true));  // row_shr:1
    if (RED >= 4)
        v += as_f32(__builtin_amdgcn_update_dpp(0, as_i32(v), 0x112, 0xF, 0xF, true));  // row_shr:2
    if (RED >= 8)
        v += as_f32(__builtin_amdgcn_update_dpp(0, as_i32(v), 0x114, 0xF, 0xF, true));  // row_shr:4
    if (RED >= 16)
        v += as_f32(__builtin_amdgcn_update_dpp(0, as_i32(v), 0x118, 0xF, 0xF, true));  // row_shr:8
    if (RED >= 32)
        v += as_f32(__builtin_amdgcn_update_dpp(0, as_i32(v), 0x142, 0xA, 0xF, false)); // row_bcast:15
    if (RED >= 64)
        v += as_f32(__builtin_amdgcn_update_dpp(0, as_i32(v), 0x143, 0xC, 0xF, false)); // row_bcast:31
    return v;
}

// b' of one chunk: 16 bytes of packed B (32 codes) times its two SFB scales.
__device__ __attribute__((always_inline)) inline void make_bprime(uint4_t b, uint32_t sfb2,
                                                                  uint4_t (&out)[4])
{
    const half2_t sf = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sfb2, 1.0f, false);
    const half2_t s0 = {sf.x, sf.x}, s1 = {sf.y, sf.y};
    const uint32_t w[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const half2_t sc = d < 2 ? s0 : s1;
        out[d] = {as_u32(fp4x2<0>(w[d]) * sc), as_u32(fp4x2<1>(w[d]) * sc),
                  as_u32(fp4x2<2>(w[d]) * sc), as_u32(fp4x2<3>(w[d]) * sc)};
    }
}

} // namespace

#endif
