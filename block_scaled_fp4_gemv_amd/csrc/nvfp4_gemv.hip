// NVFP4 block-scaled batched GEMV for MI355X (gfx950, CDNA4).
//
// c[l][m] = fp16( sum_k e2m1(A[l][m][k]) e4m3(SFA[l][m][k/16]) e2m1(B[l][k]) e4m3(SFB[l][k/16]) )
// (kernelbot NVFP4 GEMV, submission 103289, `cute_kernel`: the per-k product of
// the four decoded operands, float32 accumulation, float16 cast.)
//
// With N = 1 this is a stream over A (8/9 of the bytes) and SFA (1/9): HBM
// bound, not a dense contraction, so it runs on the vector ALUs:
//   * Each workgroup owns `rows_per_wg` output rows of one batch and one K-slice.
//     It first converts its K-slice of B into b'[k] = e2m1(B[k]) * e4m3(SFB[k/16])
//     as float16 in LDS (exact: at most 6 significant bits, 2^-10 <= |b'| <= 2688).
//   * A 16-byte chunk of A (32 elements, two scale blocks) is the unit of work of
//     one lane. `LPR` lanes share a row and walk its K-slice in passes of LPR
//     consecutive chunks, so a group's loads are contiguous 16-byte vectors.
//   * Decode: v_cvt_scalef32_pk_f16_fp4 turns one byte (two E2M1 codes) into two
//     float16 values; v_dot2_f32_f16 multiplies them with two b' values and
//     accumulates in float32. Sums over one 16-element block are exact in float32
//     (they are multiples of sfb/4 below 2^12 * sfb), then one FMA applies the
//     SFA scale (decoded with v_cvt_pk_f32_fp8).
//   * The lanes of a row are reduced with cross-lane shuffles; a float16 result
//     is written, or for K-split problems a float32 partial, and the last
//     workgroup of a row tile (atomic ticket) sums the partials in slice order.
//   * Workgroup ids are remapped so that each XCD (own L2) gets a contiguous
//     range of row tiles: blocked-layout scale lines are shared by rows r, r+32,
//     r+64, r+96 of a 128-row block, which then stay in one L2.
//   * The batch index is part of the grid: one launch covers all L.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <vector>

#include "nvfp4_gemv.h"

namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef uint32_t uint4_t __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;                 // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 2;                  // rows per lane group
constexpr int kPrefetch = 4;              // passes of A kept in flight per lane
constexpr int kMaxChunksPerWG = 512;      // b' segment in LDS: 512 chunks = 16384 k = 32 KiB
constexpr int64_t kTargetWGs = 512;       // split K until the grid reaches ~2 WGs per CU
constexpr int kXcds = 8;                  // MI355X: 8 XCDs, WG ids dealt round-robin

struct Params {
    int32_t M, K, L;
    int32_t S;            // K-slices
    int32_t kc_split;     // 32-element chunks per K-slice
    int32_t n_row_tiles;
    int64_t sfa_batch;    // bytes per batch of SFA
    int64_t sfb_batch;    // bytes per batch of SFB
    float *partials;      // [L*M][S] when S > 1
    uint32_t *counters;   // tickets [L][n_row_tiles] when S > 1
};

// Contiguous logical ids per XCD: hardware id i runs on XCD i % 8.
__device__ inline uint32_t xcd_remap(uint32_t i, uint32_t n)
{
    const uint32_t x = i % kXcds, j = i / kXcds;
    const uint32_t q = n / kXcds, r = n % kXcds;
    return x * q + min(x, r) + j;
}

// Byte offset of scale (row r, block kb) inside one batch of the scale matrix.
// Blocked: the 128x4 tiling of submission 69953 `to_blocked_batch` (tile
// (r/128, kb/4) of 512 bytes; inside it row r%32 selects a 16-byte line, and
// (r%128)/32 and kb%4 the byte within it).
template <int LAYOUT>
__device__ inline int64_t sf_row_offset(int64_t r, int32_t nkb, int32_t ncb)
{
    if (LAYOUT == NVFP4_SF_PLAIN)
        return r * nkb;
    return (r >> 7) * (int64_t)ncb * 512 + (r & 31) * 16 + ((r >> 5) & 3) * 4;
}

// Offset of the two scales of chunk c (blocks 2c and 2c+1) relative to the row.
template <int LAYOUT>
__device__ inline int32_t sf_chunk_offset(int32_t c)
{
    if (LAYOUT == NVFP4_SF_PLAIN)
        return 2 * c;
    return (c >> 1) * 512 + (c & 1) * 2;
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

template <int LPR>
__device__ inline float group_sum(float v)
{
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1)
        v += __shfl_xor(v, off, 64);
    return v;
}

// LDS slot (16-byte units) of piece q (elements 8q..8q+7) of chunk ci. Pieces
// with the same q of 64 consecutive chunks are contiguous, so a pass's reads
// (consecutive lanes, consecutive chunks, same q) hit distinct banks.
__device__ inline int lds_slot(int ci, int q)
{
    return ((ci >> 6) << 8) + (q << 6) + (ci & 63);
}

// Sum over one 16-element scale block: dwords w0, w1 of A (8 codes each)
// against b' pieces b0, b1 (8 float16 each). Exact in float32 (see above).
__device__ inline float dot_block(uint32_t w0, uint32_t w1, const uint4_t &b0, const uint4_t &b1)
{
    float s = 0.0f;
    s = __builtin_amdgcn_fdot2(fp4x2<0>(w0), as_h2(b0.x), s, false);
    s = __builtin_amdgcn_fdot2(fp4x2<1>(w0), as_h2(b0.y), s, false);
    s = __builtin_amdgcn_fdot2(fp4x2<2>(w0), as_h2(b0.z), s, false);
    s = __builtin_amdgcn_fdot2(fp4x2<3>(w0), as_h2(b0.w), s, false);
    s = __builtin_amdgcn_fdot2(fp4x2<0>(w1), as_h2(b1.x), s, false);
    s = __builtin_amdgcn_fdot2(fp4x2<1>(w1), as_h2(b1.y), s, false);
    s = __builtin_amdgcn_fdot2(fp4x2<2>(w1), as_h2(b1.z), s, false);
    s = __builtin_amdgcn_fdot2(fp4x2<3>(w1), as_h2(b1.w), s, false);
    return s;
}

template <int LAYOUT, int LPR, bool SPLIT>
__global__ __launch_bounds__(kThreads) void nvfp4_gemv_kernel(
    const uint8_t *__restrict__ A, const uint8_t *__restrict__ B,
    const uint8_t *__restrict__ SFA, const uint8_t *__restrict__ SFB,
    uint16_t *__restrict__ C, Params p)
{
    constexpr int G = 64 / LPR;                  // row groups per wave
    constexpr int ROWS_WG = kWaves * G * kRows;
    constexpr int kStage = kMaxChunksPerWG * 4 / kThreads;   // b' pieces per thread
    extern __shared__ uint4_t lds_b[];           // b' as float16, see lds_slot

    const uint32_t lid = xcd_remap(blockIdx.x, gridDim.x);
    const int32_t s = (int32_t)(lid % (uint32_t)p.S);
    const uint32_t t2 = lid / (uint32_t)p.S;
    const int32_t tile = (int32_t)(t2 % (uint32_t)p.n_row_tiles);
    const int32_t l = (int32_t)(t2 / (uint32_t)p.n_row_tiles);

    const int32_t M = p.M, K = p.K;
    const int32_t nchunks = K >> 5, nkb = K >> 4, ncb = (nkb + 3) >> 2;
    const int32_t c_begin = s * p.kc_split;                  // this WG's K-slice, in chunks
    const int32_t c_end = min(c_begin + p.kc_split, nchunks);

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int grp = lane / LPR, j = lane % LPR;

    // ---- rows of this lane group; rows past M are clamped and not stored
    int32_t row[kRows];
    const uint8_t *arow[kRows];
    const uint8_t *srow[kRows];
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
        const int32_t r = tile * ROWS_WG + (wave * G + grp) * kRows + i;
        row[i] = r;
        const int64_t rc = min(r, M - 1);
        arow[i] = A + ((int64_t)l * M + rc) * (K >> 1);
        srow[i] = SFA + (int64_t)l * p.sfa_batch + sf_row_offset<LAYOUT>(rc, nkb, ncb);
    }
    const uint8_t *brow = B + (int64_t)l * (K >> 1);
    const uint8_t *sfbrow = SFB + (int64_t)l * p.sfb_batch;

    float acc[kRows];
#pragma unroll
    for (int i = 0; i < kRows; ++i)
        acc[i] = 0.0f;

    // The K-slice is walked in segments of at most kMaxChunksPerWG chunks, the
    // b' capacity of LDS (one segment unless K > 16384).
    for (int32_t c0 = c_begin; c0 < c_end; c0 += kMaxChunksPerWG) {
        const int32_t nck = min(kMaxChunksPerWG, c_end - c0);
        const int32_t npass = (nck + LPR - 1) / LPR;
        if (c0 != c_begin)
            __syncthreads();             // the previous segment's b' reads are done

        // ---- loads first, in this order: B and SFB for the b' staging, then
        // the first kPrefetch passes of A. Vector loads return in order, so
        // the staging waits only for its own (L2-resident) loads while A is in
        // flight. Every load is issued unconditionally (clamped to a valid
        // element) so that the wait counts stay exact; only real pieces are used.
        uint32_t bw[kStage], bs[kStage];
#pragma unroll
        for (int i = 0; i < kStage; ++i) {
            const int pc = min(threadIdx.x + i * kThreads, nck * 4 - 1);   // piece = 8 elements
            const int32_t kb = 2 * (c0 + (pc >> 2)) + ((pc & 3) >> 1);
            bw[i] = *(const uint32_t *)(brow + (int64_t)(c0 * 4 + pc) * 4);
            bs[i] = sfbrow[LAYOUT == NVFP4_SF_PLAIN ? kb : (kb >> 2) * 512 + (kb & 3)];
        }

        uint4_t abuf[kPrefetch][kRows];
        uint32_t sbuf[kPrefetch][kRows];
        auto load_pass = [&](int pass, uint4_t (&av)[kRows], uint32_t (&sv)[kRows]) {
            const int32_t ci = c0 + min(pass * LPR + j, nck - 1);
#pragma unroll
            for (int i = 0; i < kRows; ++i) {
                av[i] = __builtin_nontemporal_load((const uint4_t *)(arow[i] + (int64_t)ci * 16));
                sv[i] = *(const uint16_t *)(srow[i] + sf_chunk_offset<LAYOUT>(ci));
            }
        };
#pragma unroll
        for (int u = 0; u < kPrefetch; ++u)
            load_pass(u, abuf[u], sbuf[u]);     // passes past the end load a clamped chunk

        // ---- stage b' = e2m1(B) * e4m3(SFB) for this segment into LDS
#pragma unroll
        for (int i = 0; i < kStage; ++i) {
            const int pc = threadIdx.x + i * kThreads;
            if (pc < nck * 4) {
                const half2_t sf2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(bs[i], 1.0f, false);
                const half2_t sfv = {sf2.x, sf2.x};
                uint4_t v;
                v.x = as_u32(fp4x2<0>(bw[i]) * sfv);
                v.y = as_u32(fp4x2<1>(bw[i]) * sfv);
                v.z = as_u32(fp4x2<2>(bw[i]) * sfv);
                v.w = as_u32(fp4x2<3>(bw[i]) * sfv);
                lds_b[lds_slot(pc >> 2, pc & 3)] = v;
            }
        }
        __syncthreads();

        // ---- passes: no branches inside; passes past the end and lanes past
        // the segment read a clamped (valid) chunk and their contribution is
        // masked, so each pass waits only for its own data.
        for (int p0 = 0; p0 < npass; p0 += kPrefetch) {
#pragma unroll
            for (int u = 0; u < kPrefetch; ++u) {
                const int pass = p0 + u;
                const int32_t ci_raw = pass * LPR + j;
                const bool live = ci_raw < nck;
                const int32_t ci = min(ci_raw, nck - 1);
                const uint4_t b0 = lds_b[lds_slot(ci, 0)];
                const uint4_t b1 = lds_b[lds_slot(ci, 1)];
                const uint4_t b2 = lds_b[lds_slot(ci, 2)];
                const uint4_t b3 = lds_b[lds_slot(ci, 3)];
#pragma unroll
                for (int i = 0; i < kRows; ++i) {
                    const uint4_t a = abuf[u][i];
                    const float2_t sf = __builtin_amdgcn_cvt_pk_f32_fp8(sbuf[u][i], false);
                    const float lo = dot_block(a.x, a.y, b0, b1);
                    const float hi = dot_block(a.z, a.w, b2, b3);
                    const float nacc = __builtin_fmaf(hi, sf.y, __builtin_fmaf(lo, sf.x, acc[i]));
                    acc[i] = live ? nacc : acc[i];
                }
                load_pass(pass + kPrefetch, abuf[u], sbuf[u]);
            }
        }
    }

    // ---- reduce the LPR lanes of each row group and store
#pragma unroll
    for (int i = 0; i < kRows; ++i)
        acc[i] = group_sum<LPR>(acc[i]);

    if (!SPLIT) {
        if (j == 0) {
#pragma unroll
            for (int i = 0; i < kRows; ++i)
                if (row[i] < M)
                    C[(int64_t)l * M + row[i]] = f16_bits(acc[i]);
        }
        return;
    }

    // ---- K-split: float32 partial per (row, slice); the last WG of the tile
    // (atomic ticket) sums the partials in slice order and resets the ticket.
    if (j == 0) {
#pragma unroll
        for (int i = 0; i < kRows; ++i)
            if (row[i] < M)
                __hip_atomic_store(&p.partials[((int64_t)l * M + row[i]) * p.S + s], acc[i],
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __shared__ uint32_t is_last;
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t *ctr = &p.counters[(int64_t)l * p.n_row_tiles + tile];
        const uint32_t prev = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        const bool last = prev == (uint32_t)(p.S - 1);
        if (last)
            __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        is_last = last ? 1u : 0u;
    }
    __syncthreads();
    if (!is_last)
        return;
    __threadfence();
    for (int t = threadIdx.x; t < ROWS_WG; t += kThreads) {
        const int32_t r = tile * ROWS_WG + t;
        if (r >= M)
            break;
        const float *part = p.partials + ((int64_t)l * M + r) * p.S;
        float v = 0.0f;
        for (int k = 0; k < p.S; ++k)
            v += __hip_atomic_load(part + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        C[(int64_t)l * M + r] = f16_bits(v);
    }
}

// ------------------------------------------------------------------ host side

struct Plan {
    int lpr;
    int rows_wg;
    int S;
    int kc_split;         // chunks per slice
    int n_row_tiles;
    int64_t n_wg;
    int lds_bytes;
    size_t ws_partials;   // bytes of float32 partials (after the ticket region)
    size_t ws_total;
};

// Split-K workspace: a fixed ticket region first, then the partial sums. The
// tickets sit at the same place for every shape and each call leaves its own
// tickets at zero, so a zeroed workspace stays valid for any later shape.
constexpr size_t kWsAlign = 256;
constexpr int kMaxTickets = 1024;
constexpr size_t kCounterBytes = kMaxTickets * sizeof(uint32_t);
static_assert(kTargetWGs <= kMaxTickets, "split shapes need at most kTargetWGs tickets");

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int choose_lpr(int64_t nchunks)
{
    if (nchunks >= 64)
        return (nchunks % 64 == 0 || nchunks % 32 != 0) ? 64 : 32;
    int v = 1;
    while (v < nchunks)
        v <<= 1;
    return v;
}

nvfp4_status_t check_shape(int64_t M, int64_t K, int64_t L)
{
    if (M < 1 || K < 32 || L < 1 || K % 32 != 0)
        return NVFP4_ERR_INVALID_SHAPE;
    // int32 indices in the kernel; byte sizes well inside int64
    if (M > INT32_MAX / 2 || K > INT32_MAX / 2 || L > INT32_MAX / 2 || M * L > INT32_MAX / 2)
        return NVFP4_ERR_INVALID_SHAPE;
    if (L * M > (INT64_C(1) << 62) / K)
        return NVFP4_ERR_INVALID_SHAPE;
    return NVFP4_OK;
}

Plan make_plan(int64_t M, int64_t K, int64_t L)
{
    Plan pl{};
    const int64_t nchunks = K / 32;
    pl.lpr = choose_lpr(nchunks);
    pl.rows_wg = kWaves * (64 / pl.lpr) * kRows;
    pl.n_row_tiles = (int)cdiv(M, pl.rows_wg);
    const int64_t base = (int64_t)pl.n_row_tiles * L;
    // Split K only to fill the machine: S > 1 implies base < kTargetWGs, which
    // bounds the number of tickets. Each slice keeps at least one full pass.
    const int64_t s_max = std::max<int64_t>(1, nchunks / pl.lpr);
    int64_t S = std::min<int64_t>(cdiv(kTargetWGs, base), s_max);
    int64_t kc = cdiv(cdiv(nchunks, S), pl.lpr) * pl.lpr;
    S = cdiv(nchunks, kc);
    pl.S = (int)S;
    pl.kc_split = (int)kc;
    pl.n_wg = base * S;
    pl.lds_bytes = (int)(cdiv(std::min<int64_t>(kc, kMaxChunksPerWG), 64) * 64 * 4 * 16);
    if (S > 1) {
        pl.ws_partials = align_up((size_t)(L * M * S) * sizeof(float), kWsAlign);
        pl.ws_total = kCounterBytes + pl.ws_partials;
    }
    return pl;
}

thread_local int g_last_hip_error = 0;

template <int LAYOUT, int LPR>
hipError_t launch_lpr(const Plan &pl, const void *a, const void *b, const void *sfa, const void *sfb,
                      void *c, const Params &p, hipStream_t st)
{
    const dim3 grid((uint32_t)pl.n_wg), block(kThreads);
    if (pl.S > 1)
        hipLaunchKernelGGL((nvfp4_gemv_kernel<LAYOUT, LPR, true>), grid, block, pl.lds_bytes, st,
                           (const uint8_t *)a, (const uint8_t *)b, (const uint8_t *)sfa,
                           (const uint8_t *)sfb, (uint16_t *)c, p);
    else
        hipLaunchKernelGGL((nvfp4_gemv_kernel<LAYOUT, LPR, false>), grid, block, pl.lds_bytes, st,
                           (const uint8_t *)a, (const uint8_t *)b, (const uint8_t *)sfa,
                           (const uint8_t *)sfb, (uint16_t *)c, p);
    return hipGetLastError();
}

template <int LAYOUT>
hipError_t launch_layout(const Plan &pl, const void *a, const void *b, const void *sfa, const void *sfb,
                         void *c, const Params &p, hipStream_t st)
{
    switch (pl.lpr) {
    case 64: return launch_lpr<LAYOUT, 64>(pl, a, b, sfa, sfb, c, p, st);
    case 32: return launch_lpr<LAYOUT, 32>(pl, a, b, sfa, sfb, c, p, st);
    case 16: return launch_lpr<LAYOUT, 16>(pl, a, b, sfa, sfb, c, p, st);
    case 8: return launch_lpr<LAYOUT, 8>(pl, a, b, sfa, sfb, c, p, st);
    case 4: return launch_lpr<LAYOUT, 4>(pl, a, b, sfa, sfb, c, p, st);
    case 2: return launch_lpr<LAYOUT, 2>(pl, a, b, sfa, sfb, c, p, st);
    default: return launch_lpr<LAYOUT, 1>(pl, a, b, sfa, sfb, c, p, st);
    }
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

nvfp4_status_t validate(const void *a, const void *b, const void *sfa, const void *sfb, const void *c,
                        int64_t M, int64_t K, int64_t L, int sf_layout)
{
    if (!a || !b || !sfa || !sfb || !c)
        return NVFP4_ERR_NULL_POINTER;
    nvfp4_status_t st = check_shape(M, K, L);
    if (st != NVFP4_OK)
        return st;
    if (sf_layout != NVFP4_SF_PLAIN && sf_layout != NVFP4_SF_BLOCKED)
        return NVFP4_ERR_INVALID_LAYOUT;
    if (!aligned(a, 16) || !aligned(b, 16) || !aligned(sfa, 4) || !aligned(sfb, 4) || !aligned(c, 2))
        return NVFP4_ERR_MISALIGNED;
    return NVFP4_OK;
}

nvfp4_status_t launch(const void *a, const void *b, const void *sfa, const void *sfb, void *c,
                      int64_t M, int64_t K, int64_t L, int sf_layout, const Plan &pl,
                      void *ws, hipStream_t st)
{
    Params p{};
    p.M = (int32_t)M;
    p.K = (int32_t)K;
    p.L = (int32_t)L;
    p.S = pl.S;
    p.kc_split = pl.kc_split;
    p.n_row_tiles = pl.n_row_tiles;
    const int64_t nkb = K / 16, ncb = cdiv(nkb, 4);
    if (sf_layout == NVFP4_SF_PLAIN) {
        p.sfa_batch = M * nkb;
        p.sfb_batch = nkb;
    } else {
        p.sfa_batch = cdiv(M, 128) * ncb * 512;
        p.sfb_batch = ncb * 512;
    }
    if (pl.S > 1) {
        p.counters = (uint32_t *)ws;
        p.partials = (float *)((char *)ws + kCounterBytes);
    }
    hipError_t e = sf_layout == NVFP4_SF_PLAIN
                       ? launch_layout<NVFP4_SF_PLAIN>(pl, a, b, sfa, sfb, c, p, st)
                       : launch_layout<NVFP4_SF_BLOCKED>(pl, a, b, sfa, sfb, c, p, st);
    if (e != hipSuccess) {
        g_last_hip_error = (int)e;
        return NVFP4_ERR_HIP;
    }
    return NVFP4_OK;
}

// Library-owned split-K workspace, one per device, grown on demand.
struct DeviceWorkspace {
    void *ptr = nullptr;
    size_t bytes = 0;
};
std::mutex g_ws_mutex;
std::vector<DeviceWorkspace> g_ws;

nvfp4_status_t device_workspace(size_t need, void **out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        g_last_hip_error = (int)e;
        return NVFP4_ERR_HIP;
    }
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    if ((int)g_ws.size() <= dev)
        g_ws.resize(dev + 1);
    DeviceWorkspace &w = g_ws[dev];
    if (w.bytes < need) {
        size_t grow = std::max(need, w.bytes * 2);
        if (w.ptr) {
            // a kernel still in flight may be using the old buffer
            if ((e = hipDeviceSynchronize()) != hipSuccess || (e = hipFree(w.ptr)) != hipSuccess) {
                g_last_hip_error = (int)e;
                return NVFP4_ERR_HIP;
            }
            w.ptr = nullptr;
            w.bytes = 0;
        }
        void *p = nullptr;
        if ((e = hipMalloc(&p, grow)) != hipSuccess) {
            g_last_hip_error = (int)e;
            return NVFP4_ERR_HIP;
        }
        if ((e = hipMemset(p, 0, grow)) != hipSuccess || (e = hipDeviceSynchronize()) != hipSuccess) {
            g_last_hip_error = (int)e;
            (void)hipFree(p);
            return NVFP4_ERR_HIP;
        }
        w.ptr = p;
        w.bytes = grow;
    }
    *out = w.ptr;
    return NVFP4_OK;
}

} // namespace

extern "C" {

nvfp4_status_t nvfp4_gemv(const void *a, const void *b, const void *sfa, const void *sfb, void *c,
                          int64_t M, int64_t K, int64_t L, int sf_layout, void *stream)
{
    nvfp4_status_t st = validate(a, b, sfa, sfb, c, M, K, L, sf_layout);
    if (st != NVFP4_OK)
        return st;
    const Plan pl = make_plan(M, K, L);
    void *ws = nullptr;
    if (pl.ws_total > 0 && (st = device_workspace(pl.ws_total, &ws)) != NVFP4_OK)
        return st;
    return launch(a, b, sfa, sfb, c, M, K, L, sf_layout, pl, ws, (hipStream_t)stream);
}

size_t nvfp4_gemv_workspace_bytes(int64_t M, int64_t K, int64_t L)
{
    if (check_shape(M, K, L) != NVFP4_OK)
        return 0;
    return make_plan(M, K, L).ws_total;
}

nvfp4_status_t nvfp4_gemv_ex(const void *a, const void *b, const void *sfa, const void *sfb, void *c,
                             int64_t M, int64_t K, int64_t L, int sf_layout, void *workspace,
                             size_t workspace_bytes, void *stream)
{
    nvfp4_status_t st = validate(a, b, sfa, sfb, c, M, K, L, sf_layout);
    if (st != NVFP4_OK)
        return st;
    const Plan pl = make_plan(M, K, L);
    if (pl.ws_total > 0 &&
        (!workspace || workspace_bytes < pl.ws_total || !aligned(workspace, kWsAlign)))
        return NVFP4_ERR_WORKSPACE;
    return launch(a, b, sfa, sfb, c, M, K, L, sf_layout, pl, workspace, (hipStream_t)stream);
}

nvfp4_status_t nvfp4_gemv_plan(int64_t M, int64_t K, int64_t L, nvfp4_plan_t *plan)
{
    if (!plan)
        return NVFP4_ERR_NULL_POINTER;
    nvfp4_status_t st = check_shape(M, K, L);
    if (st != NVFP4_OK)
        return st;
    const Plan pl = make_plan(M, K, L);
    plan->lanes_per_row = pl.lpr;
    plan->rows_per_wg = pl.rows_wg;
    plan->k_splits = pl.S;
    plan->k_per_split = pl.kc_split * 32;
    plan->workgroups = pl.n_wg;
    plan->threads_per_wg = kThreads;
    plan->lds_bytes = pl.lds_bytes;
    return NVFP4_OK;
}

const char *nvfp4_status_string(int status)
{
    switch (status) {
    case NVFP4_OK: return "success";
    case NVFP4_ERR_NULL_POINTER: return "a required pointer is NULL";
    case NVFP4_ERR_INVALID_SHAPE: return "invalid shape (need M, K, L >= 1, K % 32 == 0, sizes in range)";
    case NVFP4_ERR_MISALIGNED: return "misaligned pointer (a, b: 16 B; sfa, sfb: 4 B; c: 2 B)";
    case NVFP4_ERR_INVALID_LAYOUT: return "invalid scale layout";
    case NVFP4_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case NVFP4_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
    }
}

int nvfp4_last_hip_error(void) { return g_last_hip_error; }

} // extern "C"
