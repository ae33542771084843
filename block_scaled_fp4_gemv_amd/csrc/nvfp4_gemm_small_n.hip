// NVFP4 block-scaled skinny GEMM for a few right-hand vectors (N = 1..8) on
// MI355X (gfx950).
//
// c[l][n][m] = fp16( alpha * sum_k e2m1(A[l][m][k]) e4m3(SFA[l][m][k/16])
//                                 * e2m1(B[l][n][k]) e4m3(SFB[l][n][k/16]) )
// the general case of the product kernelbot NVFP4 GEMV submission 103289 hands
// to `torch._scaled_mm` (a @ b^T with block scales, float16 out); the GEMV is
// its N = 1 column. A is streamed once for all N vectors, so each chunk of A
// is decoded once and dotted with N vectors of b'.
//
// Work split. A workgroup (4 waves, 256 lanes) owns a contiguous range of R
// rows of one batch. Lane j owns chunk c0 + j of every K-segment of 256
// chunks (8192 k) and keeps b'_n = e2m1(B_n) * e4m3(SFB_n) of that chunk for
// all N vectors in registers (16 VGPRs each, exact float16). It walks the
// rows with a ring of kSnRing rows of A and SFA loads in flight, decodes the
// row's chunk once (v_cvt_scalef32_pk_f16_fp4), forms the two exact 16-element
// block sums against each b'_n (v_dot2_f32_f16), applies the SFA pair, and
// sums the wave's lanes with DPP; per-wave sums go to LDS and are added in a
// fixed order at the end, then rounded once to float16.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>

#include "nvfp4_device.h"
#include "nvfp4_gemv.h"
#include "nvfp4_internal.h"

namespace {

constexpr int kSnThreads = 256;               // 4 waves, all on one row
constexpr int kSnWaves = kSnThreads / 64;
constexpr int kSnRing = 8;                    // rows of A in flight per lane
constexpr int kSnMaxN = 8;
constexpr int kSnPartBudget = 48 * 1024;      // LDS bytes of per-wave row sums
// Workgroups to aim for: one per CU for N <= 2; two per CU from N = 3, where
// the per-row lane reductions (dependent DPP chains) need a second wave per
// SIMD to hide their latency (headline A, N = 4 / 8: 40.9 -> 35.7 / 68.8 ->
// 54.0 us; N = 2: 27.8 -> 30.9, so it keeps one).
constexpr int64_t kSnTargetWGsFew = 256;
constexpr int64_t kSnTargetWGsMany = 512;

struct SnParams {
    int32_t M, K, L;
    int32_t R;                                // rows per workgroup (at most)
    int32_t P;                                // workgroups per batch
    int64_t sfa_batch, sfb_batch;             // bytes per batch of SFA / SFB
    float alpha;
};

// Byte offset of the two scales of chunk c (blocks 2c, 2c+1) of row r of a
// scale matrix with nkb columns (ncb groups of 4 in the blocked layout).
template <int LAYOUT>
__device__ inline int64_t sn_pair_offset(int64_t r, int32_t c, int32_t nkb, int32_t ncb)
{
    if (LAYOUT == NVFP4_SF_PLAIN)
        return r * nkb + 2 * c;
    return ((r >> 7) * ncb + (c >> 1)) * 512 + (r & 31) * 16 + ((r >> 5) & 3) * 4 + (c & 1) * 2;
}

template <int LAYOUT, int N>
__global__ __launch_bounds__(kSnThreads) void nvfp4_gemm_small_n_kernel(
    const uint8_t *__restrict__ A, const uint8_t *__restrict__ B, const uint8_t *__restrict__ SFA,
    const uint8_t *__restrict__ SFB, uint16_t *__restrict__ C, SnParams p)
{
    extern __shared__ __attribute__((aligned(16))) float sn_part[];   // [R][N][kSnWaves]
    const uint32_t lid = xcd_remap(blockIdx.x, gridDim.x);
    const int32_t tile = (int32_t)(lid % (uint32_t)p.P), l = (int32_t)(lid / (uint32_t)p.P);
    const int32_t M = p.M, K = p.K;
    const int32_t nchunks = K >> 5, nkb = K >> 4, ncb = (nkb + 3) >> 2;
    const int32_t r0 = tile * p.R;
    const int32_t nr = min(p.R, M - r0);                              // >= 1 by the plan
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    const uint8_t *a_l = A + (int64_t)l * M * (K >> 1);
    const uint8_t *b_l = B + (int64_t)l * N * (K >> 1);
    const uint8_t *sfa_l = SFA + (int64_t)l * p.sfa_batch;
    const uint8_t *sfb_l = SFB + (int64_t)l * p.sfb_batch;

    for (int32_t c0 = 0; c0 < nchunks; c0 += kSnThreads) {
        const bool first_seg = c0 == 0;
        const int32_t cl = c0 + tid;
        const bool live = cl < nchunks;
        const int32_t c = min(cl, nchunks - 1);                       // clamped: every load is real
        if (!first_seg)
            __syncthreads();    // not needed for the sums (each slot has one writer); keeps waves together

        // the ring: row i's chunk of A and its SFA pair
        auto load_row = [&](int32_t i, uint4_t &a, uint32_t &s) {
            const int32_t r = r0 + min(i, nr - 1);
            a = __builtin_nontemporal_load((const uint4_t *)(a_l + (int64_t)r * (K >> 1) + (int64_t)c * 16));
            s = *(const uint16_t *)(sfa_l + sn_pair_offset<LAYOUT>(r, c, nkb, ncb));
        };
        uint4_t abuf[kSnRing];
        uint32_t sbuf[kSnRing];
#pragma unroll
        for (int d = 0; d < kSnRing; ++d)
            load_row(d, abuf[d], sbuf[d]);
        __builtin_amdgcn_sched_barrier(0);

        // b'_n of this lane's chunk for all N vectors
        uint4_t bp[N][4];
#pragma unroll
        for (int n = 0; n < N; ++n) {
            const uint4_t braw = *(const uint4_t *)(b_l + ((int64_t)n * (K >> 1)) + (int64_t)c * 16);
            const uint32_t sb = *(const uint16_t *)(sfb_l + sn_pair_offset<LAYOUT>(n, c, nkb, ncb));
            make_bprime(braw, sb, bp[n]);
        }

        // N <= 4: the lane sums of a whole ring come after its dot products, as
        // independent DPP chains (N = 2: 27.8 -> 25.5 us on the headline A). With
        // more vectors the extra live values cost more than they hide.
        if constexpr (N <= 4) {
            for (int32_t i0 = 0; i0 < nr; i0 += kSnRing) {
                // per row of the ring: decode once, dot with every vector, refill;
                // the lane sums of all kSnRing * N (row, vector) values come after,
                // as independent DPP chains the scheduler can interleave
                float vr[kSnRing][N];
#pragma unroll
                for (int d = 0; d < kSnRing; ++d) {
                    const int32_t i = i0 + d;
                    const uint4_t a = abuf[d];
                    const uint32_t s = sbuf[d];
                    __builtin_amdgcn_sched_barrier(0);
                    load_row(i + kSnRing, abuf[d], sbuf[d]);              // refill after the last use
                    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
                    half2_t h[16];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        h[4 * q + 0] = fp4x2<0>(w[q]);
                        h[4 * q + 1] = fp4x2<1>(w[q]);
                        h[4 * q + 2] = fp4x2<2>(w[q]);
                        h[4 * q + 3] = fp4x2<3>(w[q]);
                    }
                    const float2_t sf = __builtin_amdgcn_cvt_pk_f32_fp8(s, false);
#pragma unroll
                    for (int n = 0; n < N; ++n) {
                        float lo = 0.0f, hi = 0.0f;
#pragma unroll
                        for (int q = 0; q < 2; ++q) {
                            const uint4_t bl = bp[n][q], bh = bp[n][2 + q];
                            lo = __builtin_amdgcn_fdot2(h[4 * q + 0], as_h2(bl.x), lo, false);
                            lo = __builtin_amdgcn_fdot2(h[4 * q + 1], as_h2(bl.y), lo, false);
                            lo = __builtin_amdgcn_fdot2(h[4 * q + 2], as_h2(bl.z), lo, false);
                            lo = __builtin_amdgcn_fdot2(h[4 * q + 3], as_h2(bl.w), lo, false);
                            hi = __builtin_amdgcn_fdot2(h[8 + 4 * q + 0], as_h2(bh.x), hi, false);
                            hi = __builtin_amdgcn_fdot2(h[8 + 4 * q + 1], as_h2(bh.y), hi, false);
                            hi = __builtin_amdgcn_fdot2(h[8 + 4 * q + 2], as_h2(bh.z), hi, false);
                            hi = __builtin_amdgcn_fdot2(h[8 + 4 * q + 3], as_h2(bh.w), hi, false);
                        }
                        const float v = __builtin_fmaf(hi, sf.y, lo * sf.x);
                        vr[d][n] = live ? v : 0.0f;
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int d = 0; d < kSnRing; ++d) {
#pragma unroll
                    for (int n = 0; n < N; ++n)
                        vr[d][n] = group_sum<64>(vr[d][n]);
                }
                if (lane == 63) {
#pragma unroll
                    for (int d = 0; d < kSnRing; ++d) {
                        const int32_t i = i0 + d;
                        if (i < nr) {
#pragma unroll
                            for (int n = 0; n < N; ++n) {
                                float *dst = sn_part + ((int64_t)i * N + n) * kSnWaves + wave;
                                *dst = first_seg ? vr[d][n] : *dst + vr[d][n];
                            }
                        }
                    }
                }
            }
        } else {
            for (int32_t i0 = 0; i0 < nr; i0 += kSnRing) {
#pragma unroll
                for (int d = 0; d < kSnRing; ++d) {
                    const int32_t i = i0 + d;
                    const uint4_t a = abuf[d];
                    const uint32_t s = sbuf[d];
                    __builtin_amdgcn_sched_barrier(0);
                    load_row(i + kSnRing, abuf[d], sbuf[d]);              // refill after the last use
                    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
                    half2_t h[16];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        h[4 * q + 0] = fp4x2<0>(w[q]);
                        h[4 * q + 1] = fp4x2<1>(w[q]);
                        h[4 * q + 2] = fp4x2<2>(w[q]);
                        h[4 * q + 3] = fp4x2<3>(w[q]);
                    }
                    const float2_t sf = __builtin_amdgcn_cvt_pk_f32_fp8(s, false);
#pragma unroll
                    for (int n = 0; n < N; ++n) {
                        float lo = 0.0f, hi = 0.0f;
#pragma unroll
                        for (int q = 0; q < 2; ++q) {
                            const uint4_t bl = bp[n][q], bh = bp[n][2 + q];
                            lo = __builtin_amdgcn_fdot2(h[4 * q + 0], as_h2(bl.x), lo, false);
                            lo = __builtin_amdgcn_fdot2(h[4 * q + 1], as_h2(bl.y), lo, false);
                            lo = __builtin_amdgcn_fdot2(h[4 * q + 2], as_h2(bl.z), lo, false);
                            lo = __builtin_amdgcn_fdot2(h[4 * q + 3], as_h2(bl.w), lo, false);
                            hi = __builtin_amdgcn_fdot2(h[8 + 4 * q + 0], as_h2(bh.x), hi, false);
                            hi = __builtin_amdgcn_fdot2(h[8 + 4 * q + 1], as_h2(bh.y), hi, false);
                            hi = __builtin_amdgcn_fdot2(h[8 + 4 * q + 2], as_h2(bh.z), hi, false);
                            hi = __builtin_amdgcn_fdot2(h[8 + 4 * q + 3], as_h2(bh.w), hi, false);
                        }
                        float v = __builtin_fmaf(hi, sf.y, lo * sf.x);
                        v = live ? v : 0.0f;
                        v = group_sum<64>(v);
                        if (lane == 63 && i < nr) {
                            float *dst = sn_part + ((int64_t)i * N + n) * kSnWaves + wave;
                            *dst = first_seg ? v : *dst + v;
                        }
                    }
                }
            }
        }
    }
    __syncthreads();
    for (int32_t e = tid; e < nr * N; e += kSnThreads) {
        const int32_t i = e / N, n = e % N;
        const float *src = sn_part + (int64_t)e * kSnWaves;
        float v = src[0];
#pragma unroll
        for (int w = 1; w < kSnWaves; ++w)
            v += src[w];
        C[((int64_t)l * N + n) * M + r0 + i] = f16_bits(v * p.alpha);
    }
}

template <int LAYOUT, int N>
hipError_t sn_launch(int64_t grid, int lds, const void *a, const void *b, const void *sfa, const void *sfb,
                     void *c, const SnParams &p, hipStream_t st)
{
    hipLaunchKernelGGL((nvfp4_gemm_small_n_kernel<LAYOUT, N>), dim3((uint32_t)grid), dim3(kSnThreads), lds, st,
                       (const uint8_t *)a, (const uint8_t *)b, (const uint8_t *)sfa, (const uint8_t *)sfb,
                       (uint16_t *)c, p);
    return hipGetLastError();
}

template <int LAYOUT>
hipError_t sn_dispatch(int64_t N, int64_t grid, int lds, const void *a, const void *b, const void *sfa,
                       const void *sfb, void *c, const SnParams &p, hipStream_t st)
{
    switch (N) {
    case 1: return sn_launch<LAYOUT, 1>(grid, lds, a, b, sfa, sfb, c, p, st);
    case 2: return sn_launch<LAYOUT, 2>(grid, lds, a, b, sfa, sfb, c, p, st);
    case 3: return sn_launch<LAYOUT, 3>(grid, lds, a, b, sfa, sfb, c, p, st);
    case 4: return sn_launch<LAYOUT, 4>(grid, lds, a, b, sfa, sfb, c, p, st);
    case 5: return sn_launch<LAYOUT, 5>(grid, lds, a, b, sfa, sfb, c, p, st);
    case 6: return sn_launch<LAYOUT, 6>(grid, lds, a, b, sfa, sfb, c, p, st);
    case 7: return sn_launch<LAYOUT, 7>(grid, lds, a, b, sfa, sfb, c, p, st);
    default: return sn_launch<LAYOUT, 8>(grid, lds, a, b, sfa, sfb, c, p, st);
    }
}

bool sn_aligned(const void *q, uintptr_t a) { return ((uintptr_t)q & (a - 1)) == 0; }

} // namespace

extern "C" {

nvfp4_status_t nvfp4_gemm_small_n_plan(int64_t M, int64_t N, int64_t K, int64_t L, int32_t *rows_per_wg,
                                       int64_t *workgroups, int32_t *lds_bytes)
{
    if (M < 1 || N < 1 || N > kSnMaxN || L < 1 || K < 32 || K % 32 != 0 || K > (INT64_C(1) << 22) ||
        M > INT32_MAX / 2 || L > INT32_MAX / 2 || L * M > (INT64_C(1) << 62) / K)
        return NVFP4_ERR_INVALID_SHAPE;
    // about the target number of workgroups, each a contiguous row range of one batch,
    // with the per-wave row sums inside the LDS budget
    const int64_t rmax = kSnPartBudget / (N * kSnWaves * (int64_t)sizeof(float));
    const int64_t target = N <= 2 ? kSnTargetWGsFew : kSnTargetWGsMany;
    int64_t P = std::min<int64_t>(M, std::max<int64_t>(1, target / L));
    P = std::max<int64_t>(P, (M + rmax - 1) / rmax);
    const int64_t R = (M + P - 1) / P;
    P = (M + R - 1) / R;                                              // every workgroup has a row
    if (L * P > INT32_MAX)
        return NVFP4_ERR_INVALID_SHAPE;
    if (rows_per_wg)
        *rows_per_wg = (int32_t)R;
    if (workgroups)
        *workgroups = L * P;
    if (lds_bytes)
        *lds_bytes = (int32_t)(R * N * kSnWaves * sizeof(float));
    return NVFP4_OK;
}

nvfp4_status_t nvfp4_gemm_small_n(const void *a, const void *b, const void *sfa, const void *sfb, void *c,
                                  int64_t M, int64_t N, int64_t K, int64_t L, int sf_layout, float alpha,
                                  void *stream)
{
    if (!a || !b || !sfa || !sfb || !c)
        return NVFP4_ERR_NULL_POINTER;
    int32_t R = 0, lds = 0;
    int64_t grid = 0;
    nvfp4_status_t st = nvfp4_gemm_small_n_plan(M, N, K, L, &R, &grid, &lds);
    if (st != NVFP4_OK)
        return st;
    if (sf_layout != NVFP4_SF_PLAIN && sf_layout != NVFP4_SF_BLOCKED)
        return NVFP4_ERR_INVALID_LAYOUT;
    if (!sn_aligned(a, 16) || !sn_aligned(b, 16) || !sn_aligned(sfa, 16) || !sn_aligned(sfb, 4) ||
        !sn_aligned(c, 2))
        return NVFP4_ERR_MISALIGNED;
    if (!std::isfinite(alpha))
        return NVFP4_ERR_INVALID_SCALE;
    // One vector is the GEMV, whose kernel streams A faster (several chunks
    // per lane and row, one reduction per row): use it whenever its plan needs
    // no split-K workspace, so that this entry point still allocates nothing.
    // The operand layouts for N = 1 are the GEMV's.
    if (N == 1 && nvfp4_gemv_workspace_bytes(M, K, L) == 0)
        return nvfp4_gemv_scaled(a, b, sfa, sfb, c, M, K, L, sf_layout, alpha, nullptr, 0, stream);
    // Two vectors: the GEMV kernel with b' of both in registers, where it needs no K-split.
    if (N == 2 && nvfp4_gemv_workspace_bytes(M, K, L) == 0) {
        const nvfp4_status_t st2 = nvfp4_gemv_two_vectors(a, b, sfa, sfb, c, M, K, L, sf_layout, alpha, stream);
        if (st2 != NVFP4_ERR_INVALID_SHAPE)
            return st2;
    }
    SnParams p{};
    p.M = (int32_t)M;
    p.K = (int32_t)K;
    p.L = (int32_t)L;
    p.R = R;
    p.P = (int32_t)(grid / L);
    p.alpha = alpha;
    const int64_t nkb = K / 16, ncb = (nkb + 3) / 4;
    if (sf_layout == NVFP4_SF_PLAIN) {
        p.sfa_batch = M * nkb;
        p.sfb_batch = N * nkb;
    } else {
        p.sfa_batch = ((M + 127) / 128) * ncb * 512;
        p.sfb_batch = ((N + 127) / 128) * ncb * 512;
    }
    const hipError_t e = sf_layout == NVFP4_SF_PLAIN
                             ? sn_dispatch<NVFP4_SF_PLAIN>(N, grid, lds, a, b, sfa, sfb, c, p, (hipStream_t)stream)
                             : sn_dispatch<NVFP4_SF_BLOCKED>(N, grid, lds, a, b, sfa, sfb, c, p,
                                                             (hipStream_t)stream);
    if (e != hipSuccess) {
        nvfp4_record_hip_error((int)e);
        return NVFP4_ERR_HIP;
    }
    return NVFP4_OK;
}

} // extern "C"
