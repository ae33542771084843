// NVFP4 block-scaled batched GEMV for MI355X (gfx950, CDNA4).
//
// c[l][m] = fp16( sum_k e2m1(A[l][m][k]) e4m3(SFA[l][m][k/16]) e2m1(B[l][k]) e4m3(SFB[l][k/16]) )
// (kernelbot NVFP4 GEMV, submission 103289, `cute_kernel`: the per-k product of
// the four decoded operands, float32 accumulation, float16 cast.)
//
// With N = 1 this is a stream over A (8/9 of the bytes) and SFA (1/9): HBM
// bound, not a dense contraction, so it runs on the vector ALUs.
//
// Work split. A "chunk" is 16 bytes of A: 32 elements, two scale blocks. A
// "slot" is one 16-byte line of the 128x4 blocked scale layout (submission
// 69953 `to_blocked_batch`): slot s of a batch holds, for every group of four
// scale blocks, the scales of the four rows 128*(s/32) + 32*i4 + s%32,
// i4 = 0..3. Each workgroup owns a contiguous range of slots of one batch,
// i.e. 4 rows per slot, and one K-slice. With that row set the workgroup's
// blocked scales are whole 16-byte vectors (neighbouring slots share lines),
// read once into LDS; plain scales are staged from their rows. Both layouts
// then run the same arithmetic and give bit-identical results.
//
// Roles. Four waves compute; a fifth (wave 0, the first one launched) stages
// the scales of the workgroup's rows into LDS with direct-to-LDS loads
// (global_load_lds), all in flight at once. A wave's vector loads complete in order, so scale loads issued by a
// computing wave would hold back every later A load of that wave; from a wave
// of their own they stream beside A. The computing waves start on A at once
// (or, in the BFIRST variant for workgroups with few row rounds, right after
// the copies of b's inputs are issued): the first rounds keep their exact
// block sums and take the scales after the barrier that publishes them.
//
// Inside a workgroup, LPR lanes share a row and the rows are taken run by
// run (consecutive rows of A at one time); lane j of a row group owns the
// chunks j, j+LPR, j+2*LPR, j+3*LPR of every K-segment (4*LPR chunks), so each
// wave-wide load is a contiguous run of 16-byte vectors. The lane converts its
// four chunks of B into b'[k] = e2m1(B[k]) * e4m3(SFB[k/16]) once (float16 in
// registers: exact, at most 6 significant bits, 2^-10 <= |b'| <= 2688) and
// reuses them for every row. Per chunk and row:
//   * v_cvt_scalef32_pk_f16_fp4 turns each byte (two E2M1 codes) into two
//     float16 values, v_dot2_f32_f16 multiplies them with two b' values and
//     accumulates in float32; sums over one 16-element block are exact in
//     float32 (multiples of sfb/4 below 2^12 * sfb);
//   * one FMA per block applies the SFA scale (v_cvt_pk_f32_fp8 decode).
// Rows follow each other without a break: the loads of the next kPrefetch
// chunk-steps are in flight until the last ring, which refills nothing. A row's lanes are summed with DPP and the
// per-wave sums are added in LDS in a fixed order; the result is rounded to
// float16 once, after one float32 multiply by the global scale alpha (1 for
// the unscaled entry points, where it changes nothing). K-split shapes (small
// M*L) write float32 partials and the last workgroup of a row range (atomic
// ticket) adds them in slice order.
//
// Workgroup ids are remapped so that each XCD (own L2) gets a contiguous range
// of slots; the batch index is part of the grid, so one launch covers all L.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <type_traits>
#include <vector>

#include "nvfp4_gemv.h"
#include "nvfp4_internal.h"
#include "nvfp4_device.h"

namespace {

constexpr int kWaves = 4;                 // compute waves per workgroup
constexpr int kThreads = 64 * kWaves;     // compute threads
constexpr int kBlock = kThreads + 64;     // plus one wave (wave 0) that stages the scales
constexpr int kCpl = 4;                   // chunks per lane per K-segment
constexpr int kPrefetch = 8;              // chunk loads in flight per lane (multiple of kCpl)
constexpr int kDeferRounds = 2;           // first row rounds that keep block sums (multiple of the ring's rounds)
constexpr int kMaxLpr = 256;              // lanes per row, at most the compute threads
constexpr int kLdsLimit = 159 * 1024;     // dynamic LDS of one workgroup (gfx950: 160 KiB per CU)
constexpr int kSfaLdsBudget = 36 * 1024;  // staged SFA bytes per workgroup
constexpr int kStageInFlight = 48;        // staging copies in flight at most (the counter holds 63)
constexpr int kDmaBytes = 64 * 16;        // LDS bytes one wave-wide 16-byte direct-to-LDS load fills
constexpr bool kStageB = true;            // blocked layout: B is staged with SFB (else the computing waves load it)
constexpr int kSfaAhead = 20;             // blocked: A-scale copies issued before the wait for b's inputs
constexpr int64_t kTargetWGs = 256;       // one workgroup per CU
constexpr int kBFirstMaxRounds = 8;       // b's inputs go first for workgroups of at most this many row rounds
constexpr int64_t kSplitCostBytes = 50 * 1024; // a K-split's partials, ticket and ordered sum, in bytes of
                                          // one workgroup's streaming (about 1.8 us at a CU's share)
constexpr int64_t kWgStartSlots = 7;      // start-up of one workgroup, in slots of streaming (measured: about
                                          // 1.7 us against 0.24 us per slot of 4 rows x 2 KiB)
constexpr int kWaitVmcnt0 = 0x0F70;       // s_waitcnt vmcnt(0) (expcnt, lgkmcnt unconstrained)
constexpr int kBufferFlags = 0x00020000;  // buffer resource word 3: 32-bit data format
constexpr int kCachePolicyNT = 2;         // buffer load cache policy: non-temporal
constexpr int64_t kMaxK = INT64_C(1) << 22; // keeps one workgroup's A offsets below 2^31
constexpr int kRowThreads = 256;          // row kernel: 4 waves, one row each
constexpr int kRowMaxCpl = 2;             // row kernel: chunks per lane, so K <= 64 * 2 * 32 = 4096
constexpr int64_t kRowMaxSlots = 256;     // row kernel when the slots of all batches fit one per CU,
constexpr int64_t kRowMaxSlotsShortK = 1024; // or four per CU with K <= 256
constexpr int kWideMaxCpl = 4;            // wide-row kernel: K <= 256 * 4 * 32 = 32768
constexpr int64_t kWideMaxRows = 400;     // wide-row kernel for at most this many rows (all batches)
constexpr int kRowsPerWave = 8;           // multi-row kernel: rows per wave (32 per workgroup)
constexpr int kRowsMaxCpl = 2;            // multi-row kernel: K <= 64 * 2 * 32 = 4096
constexpr int64_t kRowsMinGrid = 192;     // multi-row kernel: grids of 192 .. 256 workgroups

static_assert(kPrefetch % kCpl == 0, "a row's chunk-steps must not straddle the prefetch ring");
static_assert(kDeferRounds % (kPrefetch / kCpl) == 0, "deferred rounds end on a ring boundary");

struct Params {
    int32_t M, K, L;
    int32_t S;            // K-slices
    int32_t kc_split;     // chunks per K-slice
    int32_t P;            // workgroups per (batch, slice)
    int32_t spw;          // slots per workgroup (at most)
    int32_t ns;           // slots per batch that hold at least one row
    int32_t stage_bytes;  // LDS bytes for the staged scales (whole direct-to-LDS loads)
    int32_t wide_plain;   // plain scales staged in 16-byte units
    int32_t a_row;        // bytes between rows of A (a multiple of 16)
    int64_t a_batch;      // bytes between batches of A
    int64_t a_extent;     // bytes from A to one past its last byte
    int64_t b_batch;      // bytes between batches of B
    int64_t sfa_row;      // bytes between rows of plain SFA
    int64_t sfa_batch;    // bytes between batches of SFA
    int64_t sfb_batch;    // bytes between batches of SFB
    int64_t c_batch;      // float16 elements between batches of C
    int64_t b_vec;        // bytes between the vectors of B (NV > 1)
    int64_t sfb_vec;      // bytes between the vectors' scales in SFB (plain: a row; blocked: a 16-byte line)
    int64_t c_vec;        // float16 elements between the vectors' columns of C
    float alpha;          // global scale, applied to the float32 row sum before rounding
    uint32_t *counters;   // tickets [L][P] when S > 1
    float *partials;      // [L*M][S] when S > 1
};

// Local row q of a workgroup whose slots are first .. first+nslots-1: sub-row
// i4 = q / nslots (the 32-row group inside the 128-row block) of slot
// first + q % nslots. Consecutive q are consecutive rows of A, so the rows a
// workgroup streams at one time are neighbours in memory.
__device__ inline void split_local_row(int32_t q, int32_t nslots, int32_t &sl, int32_t &i4)
{
    i4 = (q >= nslots) + (q >= 2 * nslots) + (q >= 3 * nslots);   // q < 4 * nslots
    sl = q - i4 * nslots;
}
__device__ inline int32_t slot_row(int32_t first, int32_t nslots, int32_t q)
{
    int32_t sl, i4;
    split_local_row(q, nslots, sl, i4);
    const int32_t s = first + sl;
    return ((s >> 5) << 7) + (i4 << 5) + (s & 31);
}

// Byte offset of the two scales of chunk c (blocks 2c, 2c+1) of row r.
template <int LAYOUT>
__device__ inline int64_t sf_pair_offset(int64_t r, int32_t c, int32_t nkb, int32_t ncb)
{
    if (LAYOUT == NVFP4_SF_PLAIN)
        return r * nkb + 2 * c;
    return ((r >> 7) * ncb + (c >> 1)) * 512 + (r & 31) * 16 + ((r >> 5) & 3) * 4 + (c & 1) * 2;
}

// 16 bytes of A, streamed once: non-temporal
__device__ __attribute__((always_inline)) inline uint4_t load_a(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kCachePolicyNT);
}

// Sum over one 16-element scale block: dwords w0, w1 of A (8 codes each)
// against b' pieces b0, b1 (8 float16 each). Exact in float32 (see above).
__device__ __attribute__((always_inline)) inline float dot_block(uint32_t w0, uint32_t w1,
                                                                 const uint4_t &b0, const uint4_t &b1)
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

// s_waitcnt vmcnt(k) for a wave-uniform k (the count is an immediate; k
// above 63, the counter's limit, waits as 63 does)
template <int K0 = 0>
__device__ __attribute__((always_inline)) inline void wait_vmcnt(int k)
{
    if constexpr (K0 < 63) {
        if (k == K0) {
            __builtin_amdgcn_s_waitcnt((kWaitVmcnt0 & ~0xC00F) | (K0 & 15) | ((K0 >> 4) << 14));
            return;
        }
        wait_vmcnt<K0 + 1>(k);
    } else {
        __builtin_amdgcn_s_waitcnt((kWaitVmcnt0 & ~0xC00F) | 15 | (3 << 14));
    }
}

// 16 bytes per lane from global memory straight into LDS at lds_dst + lane*16
// (global_load_lds_dwordx4, LDS address from M0). Inline assembly so that the
// compiler does not track the copy: the staging wave orders its copies with
// its own vmcnt waits, and the compiler would otherwise wait for all of them
// before the first barrier. Nothing else in this file uses M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __attribute__((always_inline)) inline void copy16_to_lds(const void *src, const uint8_t *lds_dst)
{
    const uint32_t addr = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_dst);
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "s"(addr)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// The scalars that the first loads of A depend on lead the argument list as
// plain scalars: the build preloads the leading kernel arguments into SGPRs
// (kernarg preload), so the A stream does not wait for a kernarg read at wave
// start. Params repeats them for the host side; the kernel uses these copies.
// BFIRST: b's inputs are requested before the first ring of A (the staging
// wave's copies behind a barrier, or the computing waves' own loads). That
// pays when a workgroup has few row rounds, so the b' start-up is most of its
// time; with many rounds, A first streams better.
// ILV: the deferred rounds are finished one per following round instead of
// all at once after the publish barrier (measured faster for workgroups with
// many row rounds and LPR <= 64, slower with LPR = 128 or few rounds).
// NV: right-hand vectors (1, or 2 for the skinny GEMM): A is streamed and
// decoded once and dotted with each vector's b'.
template <int LAYOUT, int LPR, bool SPLIT, bool BFIRST, bool ILV, int NV>
__global__ __launch_bounds__(kBlock) void nvfp4_gemv_kernel(
    const uint8_t *__restrict__ A, uint32_t n_wg, int32_t M, int32_t K, int32_t nL, int32_t spw,
    int32_t ns, int32_t kc_split, int32_t a_row, int64_t a_extent, int32_t P, int32_t stage_bytes,
    const uint8_t *__restrict__ B, const uint8_t *__restrict__ SFA, const uint8_t *__restrict__ SFB,
    uint16_t *__restrict__ C, Params p)
{
    constexpr int SEG = LPR * kCpl;              // chunks per K-segment
    constexpr int G = kThreads / LPR;            // row groups (rows in flight) per workgroup
    constexpr int WPG = LPR > 64 ? LPR / 64 : 1; // waves per row group
    constexpr int RED = LPR < 64 ? LPR : 64;     // lanes summed inside one wave
    constexpr int PR = kPrefetch / kCpl;         // row rounds in the load ring
    constexpr int DR = kDeferRounds;             // first rounds that keep their block sums
    static_assert(NV == 1 || !SPLIT, "several vectors only without a K-split");
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    const uint32_t lid = xcd_remap(blockIdx.x, n_wg);
    const int32_t s = SPLIT ? (int32_t)(lid % (uint32_t)p.S) : 0;
    const uint32_t t2 = SPLIT ? lid / (uint32_t)p.S : lid;
    const int32_t tile = nL == 1 ? (int32_t)t2 : (int32_t)(t2 % (uint32_t)P);
    const int32_t l = nL == 1 ? 0 : (int32_t)(t2 / (uint32_t)P);

    const int32_t nchunks = K >> 5, nkb = K >> 4, ncb = (nkb + 3) >> 2;
    // Slots of this workgroup: a contiguous range, so that its blocked scales
    // are few whole lines per 512-byte tile (neighbouring slots share a line).
    const int32_t first = tile * spw;
    const int32_t nslots = min(spw, ns - first);
    const int32_t nq = 4 * nslots;                        // local rows (some may be >= M)
    const int32_t c_begin = s * kc_split;
    const int32_t c_end = min(c_begin + kc_split, nchunks);

    // One wave stages the scales, the others compute.
    // A wave's vector loads complete in order, so scale loads issued by a
    // computing wave would hold back every later A load of that wave; issued
    // by a wave of their own, they stream beside the A loads.
    // Wave 0 stages the scales (it is launched first), waves 1..4 compute.
    // The role is wave-uniform (scalar) so that the two roles are separate
    // paths, not one path with two lane masks whose registers would all be
    // live at once.
    const bool loader = __builtin_amdgcn_readfirstlane((int)threadIdx.x) < 64;
    const int tid = loader ? (int)threadIdx.x : (int)threadIdx.x - 64;
    const int grp = tid / LPR, j = tid % LPR;
    const int lane = tid & 63;
    const int wig = WPG > 1 ? j >> 6 : 0;                 // wave index inside the row group
    const bool leader = (lane % RED) == RED - 1;           // holds the group sum after group_sum

    const int64_t abatch = (int64_t)l * M;                 // row index base of the split-K partials
    const int64_t cbatch = (int64_t)l * p.c_batch;
    const uint8_t *sfa_l = SFA + (int64_t)l * p.sfa_batch;
    const uint8_t *sfb_l = SFB + (int64_t)l * p.sfb_batch;
    const uint8_t *b_l = B + (int64_t)l * p.b_batch;
    // Blocked layout: the staging wave stages b's inputs too, the 16-byte SFB
    // lines that hold row 0 (the scale pairs the lanes need sit 512 bytes
    // apart: one scattered 2-byte read each) and B. Plain: the computing waves
    // load them (one contiguous run each). The LDS areas are reserved either way.
    constexpr bool STAGE_SFB = LAYOUT == NVFP4_SF_BLOCKED;
    constexpr bool STAGE_B = STAGE_SFB && kStageB;
    constexpr int BSTB = kStageB ? (64 * LPR + kDmaBytes - 1) / kDmaBytes * kDmaBytes : 0;   // staged B bytes
    constexpr int SFBB = (32 * LPR + kDmaBytes - 1) / kDmaBytes * kDmaBytes;   // staged blocked SFB bytes
    uint8_t *stage = lds;                                  // staged SFA of the segment
    uint8_t *b_stage = lds + stage_bytes;                  // staged B of the segment: chunk c at c*16
    uint8_t *sfb_stage = b_stage + NV * BSTB;              // staged blocked SFB: 4-block group g at g*16 (per vector)
    float *part = (float *)(sfb_stage + NV * SFBB);        // [nq][NV][WPG] per-wave row sums

    // A through a buffer resource based at the first row of this workgroup's
    // first 128-row block: 32-bit lane offsets (the rows of one workgroup lie
    // within a few blocks).
    const int32_t row_base = (first >> 5) << 7;
    int64_t a_begin = (int64_t)row_base * a_row;
    if (nL != 1)                                           // one batch: no kernarg read here
        a_begin += (int64_t)l * p.a_batch;
    const __amdgpu_buffer_rsrc_t arsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(A + a_begin), (short)0, (int)min(a_extent - a_begin, (int64_t)0x7FFFFFFF),
        kBufferFlags);

    const int32_t NR = (nq + G - 1) / G;                   // row rounds per group
    const bool direct = LAYOUT == NVFP4_SF_PLAIN && !p.wide_plain;

    // Staged layout (bytes of LDS): blocked: item (slot sl, 4-block group cb)
    // = 16 bytes at (cb * nslots + sl) * 16, i.e. row 4 sl + i4 at +4 i4 and
    // chunk c of the group (2 scales) at +2 (c & 1); plain: the 2 scales of
    // (row q, chunk c) at (q * nck + c) * 2. Both roles pass the same barriers:
    // per segment one after the previous segment's staged bytes are read (not
    // before the first), (blocked, BFIRST) one after the copies of b's inputs
    // are issued, (blocked) one after b's inputs are staged, and one that
    // publishes the staged scales of A; then the ones of the epilogue. With
    // NV vectors, B and the SFB lines are staged per vector (B at
    // b_stage + v*BSTB, SFB at sfb_stage + v*SFBB).
    if (loader) {
        // raised issue priority: its copies gate the publish barrier, and the
        // computing waves' A loads would otherwise take every free issue slot
        __builtin_amdgcn_s_setprio(3);
        // nothing is in flight yet; saying so keeps the compiler from waiting
        // on the copies (it cannot see them) inside the issue loops below
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        for (int32_t c0 = c_begin; c0 < c_end; c0 += SEG) {
            const int32_t nck = min(SEG, c_end - c0);
            if (c0 != c_begin)
                __syncthreads();                           // the previous segment's staged bytes are read
            const int32_t ncb_seg = (nck + 1) >> 1, cb0 = c0 >> 1, units = nck >> 3;
            // b's inputs go first: b' waits for them, the scales of A only
            // for the deferred rounds' end. Past the end the index clamps.
            const int32_t nbc = STAGE_B ? (nck + 63) >> 6 : 0;
            const int32_t nsfb = STAGE_SFB ? (ncb_seg + 63) >> 6 : 0;
#pragma unroll
            for (int nv = 0; nv < NV; ++nv)
                for (int32_t i = 0; i < nbc; ++i)
                    copy16_to_lds(b_l + nv * p.b_vec + (int64_t)(c0 + min(i * 64 + lane, nck - 1)) * 16,
                                  b_stage + nv * BSTB + i * kDmaBytes);
#pragma unroll
            for (int nv = 0; nv < NV; ++nv)
                for (int32_t i = 0; i < nsfb; ++i)
                    copy16_to_lds(sfb_l + nv * p.sfb_vec + (int64_t)(cb0 + min(i * 64 + lane, ncb_seg - 1)) * 512,
                                  sfb_stage + nv * SFBB + i * kDmaBytes);
            if (BFIRST && STAGE_SFB)
                __syncthreads();                           // b's input copies are issued
            if (!direct) {
                // Wave-wide direct-to-LDS load i puts item i*64 + lane at
                // (i*64 + lane) * 16; all loads are in flight at once. Item it
                // is (minor, major) = (it % per, it / per) with per = nslots
                // (blocked: slot, 4-block group) or units (plain: 16-byte
                // unit, row). The lane steps its pair by 64 items per load
                // without dividing: issuing must be quick, or the scales land
                // late. Items past the end clamp the major index (in bounds;
                // those LDS bytes are never read).
                const int32_t per = LAYOUT == NVFP4_SF_BLOCKED ? nslots : units;
                const int32_t nmajor = LAYOUT == NVFP4_SF_BLOCKED ? ncb_seg : nq;
                const int32_t nload = (per * nmajor + 63) >> 6;
                const int32_t dmaj = 64 / per, dmin = 64 % per;
                int32_t mn = lane % per, mj = lane / per;
                // PACED: at most kStageInFlight copies in flight (b's inputs
                // count: they were issued first); only compiled in where the
                // copies could outnumber what the wait counter holds
                auto issue_loop = [&](auto paced, int32_t i0, int32_t i1) {
                    for (int32_t i = i0; i < i1; ++i) {
                        if (decltype(paced)::value && i + nbc * NV + nsfb * NV >= kStageInFlight)
                            __builtin_amdgcn_s_waitcnt((kWaitVmcnt0 & ~0xC00F) | ((kStageInFlight - 1) & 15) |
                                                       (((kStageInFlight - 1) >> 4) << 14));
                        const int32_t mjc = min(mj, nmajor - 1);
                        const uint8_t *src;
                        if (LAYOUT == NVFP4_SF_BLOCKED) {
                            const int32_t sg = first + mn;
                            src = sfa_l + ((int64_t)(sg >> 5) * ncb + cb0 + mjc) * 512 + (sg & 31) * 16;
                        } else {
                            const int32_t r = min(slot_row(first, nslots, mjc), M - 1);
                            src = sfa_l + (int64_t)r * p.sfa_row + 2 * c0 + 16 * mn;
                        }
                        copy16_to_lds(src, stage + i * kDmaBytes);
                        mn += dmin;
                        mj += dmaj;
                        if (mn >= per) {
                            mn -= per;
                            ++mj;
                        }
                    }
                };
                const bool many = NV * (nbc + nsfb) + nload > kStageInFlight;
                auto issue = [&](int32_t i0, int32_t i1) {
                    if (many)
                        issue_loop(std::true_type{}, i0, i1);
                    else
                        issue_loop(std::false_type{}, i0, i1);
                };
                if (STAGE_SFB) {
                    // A CU holds only so many loads in flight; issuing every
                    // copy before the wait would hold the computing waves at
                    // the b' barrier until the last one is issued. So: some
                    // copies, the wait for b's inputs, the barrier, the rest.
                    const int32_t na = min(nload, kSfaAhead);
                    issue(0, na);
                    wait_vmcnt(na);                        // the copies of b's inputs have landed
                    __syncthreads();                       // b' inputs are staged
                    issue(na, nload);
                } else {
                    issue(0, nload);
                }
                __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);   // the staged scales are in LDS
            } else {
                // plain scales whose rows are not 16-byte multiples: 2 bytes at a time
                for (int32_t it = lane; it < nq * nck; it += 64) {
                    const int32_t q = it / nck, c = it % nck;
                    const int32_t r = min(slot_row(first, nslots, q), M - 1);
                    *(uint16_t *)(stage + 2 * it) = *(const uint16_t *)(sfa_l + (int64_t)r * p.sfa_row + 2 * (c0 + c));
                }
            }
            __syncthreads();                               // publish the staged scales
        }
        __syncthreads();                                   // the epilogue's barriers
        if (SPLIT) {
            __syncthreads();
            __syncthreads();
        }
        return;
    }

    for (int32_t c0 = c_begin; c0 < c_end; c0 += SEG) {
        const int32_t nck = min(SEG, c_end - c0);
        const bool first_seg = c0 == c_begin;
        if (!first_seg)
            __syncthreads();                               // the previous segment's staged bytes are read

        auto row_off = [&](int32_t n) -> uint32_t {
            const int32_t q = min(grp + G * n, nq - 1);
            const int32_t r = min(slot_row(first, nslots, q), M - 1);
            return (uint32_t)(r - row_base) * (uint32_t)a_row;
        };
        // Step t = chunk t % kCpl of the group's row round t / kCpl; steps past
        // the end read a clamped (valid) chunk so that every load is
        // unconditional and the wait counts stay exact: round n of the group
        // reads row slot_row(q_n) (clamped to a real row), step k the lane's
        // chunk k (clamped to a real chunk; its contribution is masked by live[k]).
        uint32_t choff[kCpl];
        uint32_t sfoff[kCpl];                              // staged-scale byte of chunk k, row part excluded
        bool live[kCpl];
#pragma unroll
        for (int k = 0; k < kCpl; ++k) {
            const int32_t cl = j + k * LPR;
            const int32_t cc = min(cl, nck - 1);
            live[k] = cl < nck;
            choff[k] = (uint32_t)(c0 + cc) * 16u;
            sfoff[k] = LAYOUT == NVFP4_SF_BLOCKED ? (uint32_t)((cc >> 1) * nslots * 16 + (cc & 1) * 2)
                                                  : (uint32_t)(cc * 2);
        }
        auto sfa_of = [&](int32_t n) -> uint4_t {         // the lane's 4 scale pairs of round n
            const int32_t q = min(grp + G * n, nq - 1);
            int32_t sl, i4;
            split_local_row(q, nslots, sl, i4);
            const uint32_t rowpart = LAYOUT == NVFP4_SF_BLOCKED ? (uint32_t)(sl * 16 + i4 * 4)
                                                                : (uint32_t)(q * nck * 2);
            uint4_t w;
            w.x = *(const uint16_t *)(stage + sfoff[0] + rowpart);
            w.y = *(const uint16_t *)(stage + sfoff[1] + rowpart);
            w.z = *(const uint16_t *)(stage + sfoff[2] + rowpart);
            w.w = *(const uint16_t *)(stage + sfoff[3] + rowpart);
            return w;
        };
        auto decode_sfa = [&](uint4_t w, float2_t (&sfk)[kCpl]) {
            sfk[0] = __builtin_amdgcn_cvt_pk_f32_fp8(w.x, false);
            sfk[1] = __builtin_amdgcn_cvt_pk_f32_fp8(w.y, false);
            sfk[2] = __builtin_amdgcn_cvt_pk_f32_fp8(w.z, false);
            sfk[3] = __builtin_amdgcn_cvt_pk_f32_fp8(w.w, false);
        };
        auto store_row = [&](int32_t q, float acc, int nv) {
            const float v = group_sum<RED>(acc);
            if (leader && q < nq) {
                float *dst = part + (q * NV + nv) * WPG + wig;
                *dst = first_seg ? v : *dst + v;
            }
        };
        uint4_t abuf[kPrefetch];
        uint4_t bp[NV][kCpl][4];
        float2_t bsum[DR][kCpl][NV];                       // block sums of the first rounds
        uint4_t sf_next = {0u, 0u, 0u, 0u};
        // One round: block sums of the lane's chunks against b', then (SCALED)
        // the scales, the row sum and its store; the ring slot is refilled with
        // the step PR rounds ahead.
        auto round = [&](auto scaled, auto refill, int32_t n, int rr, int dn) {
            constexpr bool SCALED = decltype(scaled)::value;
            constexpr bool REFILL = decltype(refill)::value;      // the last rounds have nothing to load
            const uint32_t ro_refill = row_off(n + PR);
            float2_t sfk[kCpl];
            if (SCALED) {
                const uint4_t sfc = sf_next;
                sf_next = sfa_of(n + 1);
                decode_sfa(sfc, sfk);
            }
            float acc[NV];
#pragma unroll
            for (int nv = 0; nv < NV; ++nv)
                acc[nv] = 0.0f;
#pragma unroll
            for (int k = 0; k < kCpl; ++k) {
                const int u = rr * kCpl + k;
                const uint4_t a = abuf[u];
                if constexpr (NV == 1) {
                    // (one vector: the same code as a plain loop body, so the
                    // scheduler sees exactly the single-vector GEMV)
                    const float lo = dot_block(a.x, a.y, bp[0][k][0], bp[0][k][1]);
                    const float hi = dot_block(a.z, a.w, bp[0][k][2], bp[0][k][3]);
                    if (SCALED) {
                        const float nacc = __builtin_fmaf(hi, sfk[k].y, __builtin_fmaf(lo, sfk[k].x, acc[0]));
                        acc[0] = live[k] ? nacc : acc[0];
                    } else {
                        // computed here, as the data arrives, not sunk to their use
                        // after the staged scales
                        float l2 = lo, h2 = hi;
                        asm volatile("" : "+v"(l2), "+v"(h2));
                        bsum[dn][k][0] = (float2_t){l2, h2};
                    }
                } else {
#pragma unroll
                    for (int nv = 0; nv < NV; ++nv) {
                        const float lo = dot_block(a.x, a.y, bp[nv][k][0], bp[nv][k][1]);
                        const float hi = dot_block(a.z, a.w, bp[nv][k][2], bp[nv][k][3]);
                        if (SCALED) {
                            const float nacc = __builtin_fmaf(hi, sfk[k].y, __builtin_fmaf(lo, sfk[k].x, acc[nv]));
                            acc[nv] = live[k] ? nacc : acc[nv];
                        } else {
                            float l2 = lo, h2 = hi;
                            asm volatile("" : "+v"(l2), "+v"(h2));
                            bsum[dn][k][nv] = (float2_t){l2, h2};
                        }
                    }
                }
                // refill the slot only after its last use: a load hoisted above
                // the use would need a second register set and copies that wait
                __builtin_amdgcn_sched_barrier(0);
                if (REFILL)
                    abuf[u] = load_a(arsrc, ro_refill + choff[k]);
            }
            if (SCALED) {
#pragma unroll
                for (int nv = 0; nv < NV; ++nv)
                    store_row(grp + G * n, acc[nv], nv);
            }
        };

        // ---- the first kPrefetch steps of A and b's inputs, in the order
        // BFIRST picks (b' waits for its inputs either way)
        auto issue_ring = [&]() {
#pragma unroll
            for (int u = 0; u < kPrefetch; ++u)
                abuf[u] = load_a(arsrc, row_off(u / kCpl) + choff[u % kCpl]);
            __builtin_amdgcn_sched_barrier(0);
        };
        if (!BFIRST)
            issue_ring();
        uint4_t bload[NV][kCpl];
        uint32_t sload[NV][kCpl];
#pragma unroll
        for (int nv = 0; nv < NV; ++nv) {
#pragma unroll
            for (int k = 0; k < kCpl; ++k) {
                const int32_t ci = c0 + min(j + k * LPR, nck - 1);
                if (!STAGE_B)
                    bload[nv][k] = *(const uint4_t *)(b_l + nv * p.b_vec + (int64_t)ci * 16);
                if (!STAGE_SFB)
                    sload[nv][k] = *(const uint16_t *)(sfb_l + nv * p.sfb_vec + sf_pair_offset<LAYOUT>(0, ci, nkb, ncb));
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        if (BFIRST) {
            if (STAGE_SFB)
                __syncthreads();                           // b's input copies are issued
            issue_ring();
        }
        if (STAGE_SFB) {
            __syncthreads();                               // b' inputs are staged
#pragma unroll
            for (int nv = 0; nv < NV; ++nv) {
#pragma unroll
                for (int k = 0; k < kCpl; ++k) {
                    const int32_t cc = min(j + k * LPR, nck - 1);
                    if (STAGE_B)
                        bload[nv][k] = *(const uint4_t *)(b_stage + nv * BSTB + cc * 16);
                    sload[nv][k] = *(const uint16_t *)(sfb_stage + nv * SFBB + (cc >> 1) * 16 + (cc & 1) * 2);
                }
            }
        }
        // b' for this lane's chunks of the segment (registers, reused for every row)
#pragma unroll
        for (int nv = 0; nv < NV; ++nv) {
#pragma unroll
            for (int k = 0; k < kCpl; ++k)
                make_bprime(bload[nv][k], sload[nv][k], bp[nv][k]);
        }
        // rounds 0 .. DR-1 keep their block sums (straight-line code)
#pragma unroll
        for (int n = 0; n < DR; ++n)
            round(std::false_type{}, std::true_type{}, n, n % PR, n);

        __syncthreads();                                   // the staged scales are published

        // finish the deferred rounds: all at once, or (ILV) one per round of
        // the next DR rounds, so no burst of finishing work holds back refills
        auto finish = [&](int d) {
            float2_t sfk[kCpl];
            decode_sfa(sfa_of(d), sfk);
#pragma unroll
            for (int nv = 0; nv < NV; ++nv) {
                float acc = 0.0f;
#pragma unroll
                for (int k = 0; k < kCpl; ++k) {
                    const float nacc = __builtin_fmaf(bsum[d][k][nv].y, sfk[k].y,
                                                      __builtin_fmaf(bsum[d][k][nv].x, sfk[k].x, acc));
                    acc = live[k] ? nacc : acc;
                }
                store_row(grp + G * d, acc, nv);
            }
        };
        if (!ILV) {
#pragma unroll
            for (int d = 0; d < DR; ++d)
                finish(d);
        }
        // then the rest with the scales read one round ahead; at the loop
        // entry the youngest loads are A loads, as on the loop's back edge, so
        // its waits stay exact
        sf_next = sfa_of(DR);
        int32_t n0 = DR;
        if (ILV) {
#pragma unroll
            for (int it = 0; it < DR / PR; ++it) {
                if (n0 + PR < NR) {
#pragma unroll
                    for (int rr = 0; rr < PR; ++rr) {
                        round(std::true_type{}, std::true_type{}, n0 + rr, rr, 0);
                        finish(it * PR + rr);
                    }
                } else if (n0 < NR) {
#pragma unroll
                    for (int rr = 0; rr < PR; ++rr) {
                        round(std::true_type{}, std::false_type{}, n0 + rr, rr, 0);
                        finish(it * PR + rr);
                    }
                } else {
#pragma unroll
                    for (int rr = 0; rr < PR; ++rr)
                        finish(it * PR + rr);
                }
                n0 += PR;
            }
        }
        for (; n0 + PR < NR; n0 += PR) {
#pragma unroll
            for (int rr = 0; rr < PR; ++rr)
                round(std::true_type{}, std::true_type{}, n0 + rr, rr, 0);
        }
        // the last ring of rounds: every row is loaded, nothing to refill
        if (n0 < NR) {
#pragma unroll
            for (int rr = 0; rr < PR; ++rr)
                round(std::true_type{}, std::false_type{}, n0 + rr, rr, 0);
        }
    }
    __syncthreads();

    // ---- per-row totals: add the per-wave sums in a fixed order, round once
    if (!SPLIT) {
        for (int32_t q = tid; q < nq; q += kThreads) {
            const int32_t r = slot_row(first, nslots, q);
            if (r < M) {
#pragma unroll
                for (int nv = 0; nv < NV; ++nv) {
                    float v = part[(q * NV + nv) * WPG];
#pragma unroll
                    for (int w = 1; w < WPG; ++w)
                        v += part[(q * NV + nv) * WPG + w];
                    C[cbatch + nv * p.c_vec + r] = f16_bits(v * p.alpha);
                }
            }
        }
        return;
    }

    // ---- K-split: float32 partial per (row, slice); the last workgroup of the
    // row range (atomic ticket) adds the partials in slice order and resets the
    // ticket. Partials are written and read with agent-scope atomic stores and
    // loads, which are coherent across the XCDs without any cache maintenance,
    // so the handshake only needs the stores to have completed before the
    // ticket is taken. Agent-scope fences are avoided on purpose: on this chip
    // they write back and invalidate the whole L2 of the XCD, once per workgroup.
    for (int32_t q = tid; q < nq; q += kThreads) {
        const int32_t r = slot_row(first, nslots, q);
        if (r < M) {
            float v = part[q * WPG];
#pragma unroll
            for (int w = 1; w < WPG; ++w)
                v += part[q * WPG + w];
            __hip_atomic_store(&p.partials[(abatch + r) * p.S + s], v, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    __shared__ uint32_t is_last;
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);     // this wave's partial stores are done
    __syncthreads();
    if (tid == 0) {
        uint32_t *ctr = &p.counters[(int64_t)l * P + tile];
        const uint32_t prev = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool last = prev == (uint32_t)(p.S - 1);
        if (last)
            __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        is_last = last ? 1u : 0u;
    }
    __syncthreads();
    if (!is_last)
        return;
    for (int32_t q = tid; q < nq; q += kThreads) {
        const int32_t r = slot_row(first, nslots, q);
        if (r < M) {
            const float *pp = p.partials + (abatch + r) * p.S;
            float v = 0.0f;
            for (int k = 0; k < p.S; ++k)
                v += __hip_atomic_load(pp + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            C[cbatch + r] = f16_bits(v * p.alpha);
        }
    }
}

// Strides of the row kernels' operands. DENSE: derived from M and K (the
// layouts of the header), so that every address of the first loads depends
// only on preloaded kernel arguments; else the caller's strides from Params,
// a kernel-argument read before the first load.
template <int LAYOUT, bool DENSE>
struct RowStrides {
    int64_t a_row, a_batch, b_batch, sfa_row, sfa_batch, sfb_batch;
    __device__ RowStrides(int32_t M, int32_t K, const Params &p)
    {
        if (DENSE) {
            const int64_t nkb = K >> 4, ncb = (nkb + 3) >> 2;
            a_row = K >> 1;
            a_batch = (int64_t)M * (K >> 1);
            b_batch = K >> 1;
            sfa_row = nkb;
            sfa_batch = LAYOUT == NVFP4_SF_BLOCKED ? (int64_t)((M + 127) >> 7) * ncb * 512 : (int64_t)M * nkb;
            sfb_batch = LAYOUT == NVFP4_SF_BLOCKED ? ncb * 512 : nkb;
        } else {
            a_row = p.a_row;
            a_batch = p.a_batch;
            b_batch = p.b_batch;
            sfa_row = p.sfa_row;
            sfa_batch = p.sfa_batch;
            sfb_batch = p.sfb_batch;
        }
    }
};

// One round of loads for CPL chunks of row r (chunk i of the lane: cc[i]),
// then the scaled partial sum of the lane; used by both row kernels.
template <int LAYOUT, int CPL>
__device__ __attribute__((always_inline)) inline float row_partial(
    const uint8_t *a_r, const uint8_t *b_l, const uint8_t *sfa_l, const uint8_t *sfb_l, int64_t sfa_row, int32_t r,
    const int32_t (&cc)[CPL], const bool (&live)[CPL], int32_t nkb, int32_t ncb)
{
    uint4_t bq[CPL], aq[CPL];
    uint32_t sb[CPL], sa[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        bq[i] = *(const uint4_t *)(b_l + (int64_t)cc[i] * 16);
        sb[i] = *(const uint16_t *)(sfb_l + sf_pair_offset<LAYOUT>(0, cc[i], nkb, ncb));
        sa[i] = LAYOUT == NVFP4_SF_PLAIN ? *(const uint16_t *)(sfa_l + (int64_t)r * sfa_row + 2 * cc[i])
                                         : *(const uint16_t *)(sfa_l + sf_pair_offset<LAYOUT>(r, cc[i], nkb, ncb));
    }
#pragma unroll
    for (int i = 0; i < CPL; ++i)
        aq[i] = __builtin_nontemporal_load((const uint4_t *)(a_r + (int64_t)cc[i] * 16));
    // every load above is issued before any use (the scheduler would otherwise
    // trade registers for a second and third round trip)
    __builtin_amdgcn_sched_barrier(0);
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        uint4_t bp[4];
        make_bprime(bq[i], sb[i], bp);
        const float lo = dot_block(aq[i].x, aq[i].y, bp[0], bp[1]);
        const float hi = dot_block(aq[i].z, aq[i].w, bp[2], bp[3]);
        const float2_t sf = __builtin_amdgcn_cvt_pk_f32_fp8(sa[i], false);
        const float nacc = __builtin_fmaf(hi, sf.y, __builtin_fmaf(lo, sf.x, acc));
        acc = live[i] ? nacc : acc;
    }
    return acc;
}

// Row kernel for small problems: one wave per row, every load of the row
// issued at once. The main kernel's start-up (kernel-argument read, b's
// inputs, then the staged scales, each behind a barrier) takes about three
// memory round trips before the first result; a workgroup of a few rows pays
// it whole. Here a workgroup of 4 waves owns one slot (the 4 rows that share
// the blocked scale lines) and each wave one row. Lane j takes the chunks
// j, j+64, ... (CPL of them, K <= 64*CPL*32, short K only): it loads their B chunks, SFB
// pairs, SFA pairs and A chunks together, waits once, forms b', the exact
// block sums and the scaled row sum as the main kernel does, and the wave's
// lanes are summed with DPP. No LDS, no barrier, one memory round trip.
// The leading arguments (pointers, grid size, M, K, alpha, C) fill the
// kernel-argument SGPRs that the build preloads: the first loads and the
// final store need no kernel-argument read (with dense strides).
template <int LAYOUT, int CPL, bool DENSE>
__global__ __launch_bounds__(kRowThreads) void nvfp4_gemv_row_kernel(
    const uint8_t *__restrict__ A, const uint8_t *__restrict__ B, const uint8_t *__restrict__ SFA,
    const uint8_t *__restrict__ SFB, uint32_t n_wg, int32_t M, int32_t K, float alpha,
    uint16_t *__restrict__ C, Params p)
{
    const uint32_t lid = xcd_remap(blockIdx.x, n_wg);
    const int32_t ns = 32 * (M >> 7) + min(M & 127, 32);                 // slots per batch
    const int32_t slot = (int32_t)(lid % (uint32_t)ns), l = (int32_t)(lid / (uint32_t)ns);
    const int32_t wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int32_t lane = (int32_t)threadIdx.x & 63;
    const int32_t r = ((slot >> 5) << 7) + (wave << 5) + (slot & 31);   // sub-row `wave` of the slot
    if (r >= M)                                                         // wave-uniform; no barrier follows
        return;
    const int32_t nchunks = K >> 5, nkb = K >> 4, ncb = (nkb + 3) >> 2;
    const RowStrides<LAYOUT, DENSE> sd(M, K, p);
    const int64_t c_batch = DENSE ? (int64_t)M : p.c_batch;
    int32_t cc[CPL];
    bool live[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int32_t c = lane + 64 * i;
        live[i] = c < nchunks;
        cc[i] = min(c, nchunks - 1);                                    // clamped: every load is real
    }
    const float acc = row_partial<LAYOUT, CPL>(A + (int64_t)l * sd.a_batch + (int64_t)r * sd.a_row,
                                               B + (int64_t)l * sd.b_batch, SFA + (int64_t)l * sd.sfa_batch,
                                               SFB + (int64_t)l * sd.sfb_batch, sd.sfa_row, r, cc, live, nkb, ncb);
    const float v = group_sum<64>(acc);
    if (lane == 63)
        C[(int64_t)l * c_batch + r] = f16_bits(v * alpha);
}

// Wide-row kernel: the row kernel for longer rows. A workgroup of 4 waves
// owns one row; lane j of the workgroup (wave*64 + lane) takes the chunks
// j, j+256, ... (CPL of them, K <= 256*CPL*32), loads them with their scales
// and B in one round, forms the scaled partial sum, and the four waves' sums
// (DPP in each wave) are added in wave order through LDS. (Taking chunk
// pairs with one 4-byte scale load per pair measured the same.) Arguments as
// for the row kernel.
template <int LAYOUT, int CPL, bool DENSE>
__global__ __launch_bounds__(kRowThreads) void nvfp4_gemv_wide_row_kernel(
    const uint8_t *__restrict__ A, const uint8_t *__restrict__ B, const uint8_t *__restrict__ SFA,
    const uint8_t *__restrict__ SFB, uint32_t n_wg, int32_t M, int32_t K, float alpha,
    uint16_t *__restrict__ C, Params p)
{
    __shared__ float wsum[kRowThreads / 64];
    const uint32_t lid = xcd_remap(blockIdx.x, n_wg);
    const int32_t r = (int32_t)(lid % (uint32_t)M), l = (int32_t)(lid / (uint32_t)M);
    const int32_t wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int32_t lane = (int32_t)threadIdx.x & 63, j = (int32_t)threadIdx.x;
    const int32_t nchunks = K >> 5, nkb = K >> 4, ncb = (nkb + 3) >> 2;
    const RowStrides<LAYOUT, DENSE> sd(M, K, p);
    const int64_t c_batch = DENSE ? (int64_t)M : p.c_batch;
    int32_t cc[CPL];
    bool live[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int32_t c = j + kRowThreads * i;
        live[i] = c < nchunks;
        cc[i] = min(c, nchunks - 1);                                    // clamped: every load is real
    }
    const float acc = row_partial<LAYOUT, CPL>(A + (int64_t)l * sd.a_batch + (int64_t)r * sd.a_row,
                                               B + (int64_t)l * sd.b_batch, SFA + (int64_t)l * sd.sfa_batch,
                                               SFB + (int64_t)l * sd.sfb_batch, sd.sfa_row, r, cc, live, nkb, ncb);
    const float v = group_sum<64>(acc);
    if (lane == 63)
        wsum[wave] = v;
    __syncthreads();
    if (j == 0) {
        float t = 0.0f;
#pragma unroll
        for (int w = 0; w < kRowThreads / 64; ++w)
            t += wsum[w];
        C[(int64_t)l * c_batch + r] = f16_bits(t * alpha);
    }
}

// Multi-row kernel for short rows and many rows (K <= 4096): a workgroup of
// 4 waves owns the 32 rows of a 128-row block whose blocked scales fill one
// 128-byte line of every tile (rows 8h + p + 32w, p < 8: wave w takes 8 of
// them). Lane j takes the chunks j, j+64 (CPL of them) of each of its wave's
// rows, so b' of those chunks is formed once and used for 8 rows. Every load
// is issued at once, one memory round trip: the blocked SFA lines by
// direct-to-LDS copies (a line per tile, whole 1 KiB copies, ncb/8 of them),
// B and the SFB pairs, then the 8 rows' A chunks (plain scales: each row's
// pairs, one coalesced 128-byte run per row). Then the 8 rows' sums, each
// reduced over its wave with DPP. Several workgroups share a CU, so each one's
// round trip hides behind the others'. Arguments as for the row kernels.
template <int LAYOUT, int CPL, bool DENSE>
__global__ __launch_bounds__(kRowThreads) void nvfp4_gemv_rows_kernel(
    const uint8_t *__restrict__ A, const uint8_t *__restrict__ B, const uint8_t *__restrict__ SFA,
    const uint8_t *__restrict__ SFB, uint32_t n_wg, int32_t M, int32_t K, float alpha,
    uint16_t *__restrict__ C, Params p)
{
    constexpr int R = kRowsPerWave;
    extern __shared__ __attribute__((aligned(16))) uint8_t sfa_lines[];    // blocked: tile t's line at t * 128
    const uint32_t P = (uint32_t)((M + 127) >> 7) * 4;                  // workgroups per batch
    const uint32_t lid = xcd_remap(blockIdx.x, n_wg);
    const int32_t l = (int32_t)(lid / P);
    const uint32_t t = lid % P;
    const int32_t rb = (int32_t)(t >> 2), h = (int32_t)(t & 3);
    const int32_t wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int32_t lane = (int32_t)threadIdx.x & 63;
    const int32_t nchunks = K >> 5, nkb = K >> 4, ncb = (nkb + 3) >> 2;
    const RowStrides<LAYOUT, DENSE> sd(M, K, p);
    const int64_t c_batch = DENSE ? (int64_t)M : p.c_batch;
    const int32_t r0 = rb * 128 + 8 * h + 32 * wave;                   // row of p = 0
    const uint8_t *a_l = A + (int64_t)l * sd.a_batch;
    const uint8_t *b_l = B + (int64_t)l * sd.b_batch;
    const uint8_t *sfa_l = SFA + (int64_t)l * sd.sfa_batch;
    const uint8_t *sfb_l = SFB + (int64_t)l * sd.sfb_batch;

    int32_t cc[CPL];
    bool live[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int32_t c = lane + 64 * i;
        live[i] = c < nchunks;
        cc[i] = min(c, nchunks - 1);                                    // clamped: every load is real
    }
    // blocked: this wave's share of the line copies (copy i: tiles 8i .. 8i+7,
    // lane -> tile 8i + lane/8, 16-byte piece lane%8; past the last tile clamped)
    int32_t n_copies = 0;
    if (LAYOUT == NVFP4_SF_BLOCKED) {
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);                        // nothing in flight yet
        const int32_t nsc = (ncb + 7) >> 3;
        for (int32_t i = wave; i < nsc; i += kRowThreads / 64) {
            const int32_t tile = min(8 * i + (lane >> 3), ncb - 1);
            copy16_to_lds(sfa_l + ((int64_t)rb * ncb + tile) * 512 + h * 128 + (lane & 7) * 16,
                          sfa_lines + i * kDmaBytes);
            ++n_copies;
        }
    }
    uint4_t bq[CPL], aq[R][CPL];
    uint32_t sb[CPL], sa[R][CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        bq[i] = *(const uint4_t *)(b_l + (int64_t)cc[i] * 16);
        sb[i] = *(const uint16_t *)(sfb_l + sf_pair_offset<LAYOUT>(0, cc[i], nkb, ncb));
    }
    if (LAYOUT == NVFP4_SF_PLAIN) {
#pragma unroll
        for (int q = 0; q < R; ++q) {
            const int32_t r = min(r0 + q, M - 1);
#pragma unroll
            for (int i = 0; i < CPL; ++i)
                sa[q][i] = *(const uint16_t *)(sfa_l + (int64_t)r * sd.sfa_row + 2 * cc[i]);
        }
    }
#pragma unroll
    for (int q = 0; q < R; ++q) {
        const uint8_t *a_r = a_l + (int64_t)min(r0 + q, M - 1) * sd.a_row;
#pragma unroll
        for (int i = 0; i < CPL; ++i)
            aq[q][i] = __builtin_nontemporal_load((const uint4_t *)(a_r + (int64_t)cc[i] * 16));
    }
    __builtin_amdgcn_sched_barrier(0);                                  // one round of loads
    if (LAYOUT == NVFP4_SF_BLOCKED) {
        // the copies were issued before every other load of this wave, and
        // loads complete in order: wait until only the later ones are left
        wait_vmcnt(CPL * (2 + R));
        __syncthreads();                                                // every wave's lines are staged
#pragma unroll
        for (int q = 0; q < R; ++q)
#pragma unroll
            for (int i = 0; i < CPL; ++i)
                sa[q][i] = *(const uint16_t *)(sfa_lines + (cc[i] >> 1) * 128 + q * 16 + wave * 4 + (cc[i] & 1) * 2);
    }
    (void)n_copies;
    uint4_t bp[CPL][4];
#pragma unroll
    for (int i = 0; i < CPL; ++i)
        make_bprime(bq[i], sb[i], bp[i]);
#pragma unroll
    for (int q = 0; q < R; ++q) {
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const float lo = dot_block(aq[q][i].x, aq[q][i].y, bp[i][0], bp[i][1]);
            const float hi = dot_block(aq[q][i].z, aq[q][i].w, bp[i][2], bp[i][3]);
            const float2_t sf = __builtin_amdgcn_cvt_pk_f32_fp8(sa[q][i], false);
            const float nacc = __builtin_fmaf(hi, sf.y, __builtin_fmaf(lo, sf.x, acc));
            acc = live[i] ? nacc : acc;
        }
        const float v = group_sum<64>(acc);
        const int32_t r = r0 + q;
        if (lane == 63 && r < M)
            C[(int64_t)l * c_batch + r] = f16_bits(v * alpha);
    }
}

// ------------------------------------------------------------------ host side

struct Plan {
    int lpr;
    int S;
    int kc_split;         // chunks per K-slice
    int P;                // workgroups per (batch, slice)
    int spw;              // slots per workgroup (at most)
    int ns;               // slots per batch
    int stage_bytes;      // LDS bytes of staged scales
    int wide_plain;
    int bfirst;           // b's inputs before the first ring of A (few row rounds per workgroup)
    int ilv;              // deferred rounds finished one per following round
    int nv;               // right-hand vectors (1 for the GEMV)
    int row_cpl;          // > 0: the row kernel with this many chunks per lane
    int wide_cpl;         // > 0: the wide-row kernel with this many chunks per lane
    int rows_cpl;         // > 0: the multi-row kernel with this many chunks per lane
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

// Where the multi-row kernel runs (short K, rows not taken by the row
// kernel): when its grid is one workgroup for nearly every CU. With several
// workgroups per CU the CUs holding one more workgroup set the time, and the
// main kernel streams better: 7168x2048x4 8.0 -> 8.4 us, 7168x4096x3 10.4 ->
// 11.5, 1000x4096x3 4.42 -> 4.65, 7168x64x3 3.87 -> 4.74; with one per CU,
// 7168x64x1 3.55 -> 3.14 and 7168x4096x1 5.34 -> 5.25 (A/B, two passes).
inline bool rows_kernel_applies(int64_t M, int64_t K, int64_t L)
{
    (void)K;
    const int64_t grid = L * ((M + 127) / 128) * 4;
    return grid >= kRowsMinGrid && grid <= kTargetWGs;
}

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int pow2_ceil(int64_t v)
{
    int p = 1;
    while (p < v)
        p <<= 1;
    return p;
}

// Lanes per row for a K-slice of nc chunks: kCpl chunks per lane, the whole
// workgroup at most (longer slices are walked in segments of kCpl*256 chunks).
int choose_lpr(int64_t nc)
{
    return std::min<int>(kMaxLpr, pow2_ceil(cdiv(nc, kCpl)));
}

// LDS bytes of staged scales for spw slots: at most 2*lpr 16-byte items per
// slot and segment (2 bytes per row and chunk), in whole direct-to-LDS loads.
int stage_bytes(int lpr, int64_t spw)
{
    return (int)align_up((size_t)(32 * lpr * spw), kDmaBytes);
}

nvfp4_status_t check_shape(int64_t M, int64_t K, int64_t L)
{
    if (M < 1 || K < 32 || L < 1 || K % 32 != 0 || K > kMaxK)
        return NVFP4_ERR_INVALID_SHAPE;
    // int32 indices in the kernel; byte sizes well inside int64
    if (M > INT32_MAX / 2 || K > INT32_MAX / 2 || L > INT32_MAX / 2 || M * L > INT32_MAX / 2)
        return NVFP4_ERR_INVALID_SHAPE;
    if (L * M > (INT64_C(1) << 62) / K)
        return NVFP4_ERR_INVALID_SHAPE;
    return NVFP4_OK;
}

Plan make_plan(int64_t M, int64_t K, int64_t L, int nv = 1)
{
    Plan pl{};
    pl.nv = nv;
    const int64_t nchunks = K / 32;
    // slots holding at least one row: full 128-row blocks have 32, the last one min(32, M % 128)
    pl.ns = (int)(32 * (M / 128) + std::min<int64_t>(32, M % 128));
    const int64_t total_slots = L * pl.ns;

    int64_t S = 1;
    if (total_slots < kTargetWGs) {
        // Too few rows to fill the machine: K may be split, keeping >= 256
        // chunks per slice so that one slot (4 rows) still occupies every
        // lane. A split saves streaming time per workgroup but costs the
        // float32 partials, the ticket and the ordered sum (about 1.8 us,
        // measured): take the S with the least bytes per workgroup (one slot:
        // 4 rows of A and their scales) plus kSplitCostBytes when S > 1.
        const int64_t s_max = std::max<int64_t>(1, std::min<int64_t>(kTargetWGs / total_slots, nchunks / 256));
        int64_t best = INT64_MAX;
        for (int64_t cand = 1; cand <= s_max; ++cand) {
            const int64_t slice = cdiv(nchunks, cand) * 16;            // bytes of A per row and slice
            const int64_t cost = 4 * (slice + slice / 8) + (cand > 1 ? kSplitCostBytes : 0);
            if (cost < best) {
                best = cost;
                S = cand;
            }
        }
    }
    // chunks per slice: a multiple of 8, so that every slice starts on a
    // 4-block group (the blocked scales are staged, and their pairs indexed,
    // by groups of two chunks counted from the slice's first chunk) and plain
    // scale rows stay in 16-byte units
    const int64_t kc = S == 1 ? nchunks : cdiv(cdiv(nchunks, S), 8) * 8;
    S = cdiv(nchunks, kc);
    pl.S = (int)S;
    pl.kc_split = (int)kc;
    pl.lpr = choose_lpr(kc);

    // Slots per workgroup: tiles never straddle a batch, so a batch has
    // P = ceil(ns / spw) workgroups. Among grids of at most k * kTargetWGs
    // workgroups (k = 1, 2, ...), take the one whose busiest CU costs least,
    // then the smaller grid: its ceil(grid / 256) workgroups of spw slots
    // each cost a start-up of kWgStartSlots slots (b', the staged scales and
    // the first round of loads all wait on memory latency; workgroups that
    // share a CU do not overlap it) plus their slots. E.g. 258 workgroups
    // would leave two CUs with twice the work, and three 1-slot workgroups per
    // CU cost more than one 4-slot workgroup.
    // a workgroup's LDS: staged SFA, staged B, staged blocked SFB, per-wave row sums
    const int wpg = pl.lpr > 64 ? pl.lpr / 64 : 1;
    auto lds_of = [&](int64_t spw_) {
        return (int64_t)stage_bytes(pl.lpr, spw_) + nv * (kStageB ? align_up((size_t)(64 * pl.lpr), kDmaBytes) : 0) +
               nv * align_up((size_t)(32 * pl.lpr), kDmaBytes) + 4 * spw_ * wpg * nv * (int64_t)sizeof(float);
    };
    // The scales of a workgroup's rows are staged before its rounds can be
    // finished, so large stages delay every workgroup's start: keep them to
    // kSfaLdsBudget (measured: 88-row workgroups staging 88 KiB ran 37.8 us on
    // 7168x16384x3 against 35.5 us for three 28-row workgroups per CU).
    int64_t spw_max = 1;
    while (spw_max < pl.ns && lds_of(spw_max + 1) <= kLdsLimit &&
           stage_bytes(pl.lpr, spw_max + 1) <= kSfaLdsBudget)
        ++spw_max;
    int64_t spw = 1;
    if (total_slots >= kTargetWGs) {
        int64_t best_cost = INT64_MAX, best_grid = INT64_MAX;
        for (int64_t k = 1; k <= 8; ++k) {
            const int64_t per_batch = std::max<int64_t>(1, k * kTargetWGs / L);
            const int64_t cand = cdiv(pl.ns, per_batch);
            if (cand > spw_max)
                continue;
            const int64_t grid = L * S * cdiv(pl.ns, cand);
            const int64_t cost = cdiv(grid, kTargetWGs) * (kWgStartSlots + cand);
            if (cost < best_cost || (cost == best_cost && grid < best_grid)) {
                best_cost = cost;
                best_grid = grid;
                spw = cand;
            }
        }
        if (best_cost == INT64_MAX)
            spw = spw_max;
    }
    pl.spw = (int)spw;
    pl.P = (int)cdiv(pl.ns, spw);
    pl.n_wg = (int64_t)pl.P * L * S;
    if (nv == 1 && S == 1 && nchunks <= 64 * kRowMaxCpl &&
        (total_slots <= kRowMaxSlots || (nchunks <= 8 && total_slots <= kRowMaxSlotsShortK))) {
        // few rows and short K: one wave per row and one memory round trip
        // (row kernel). Measured against the main kernel: 1000x4096x1 3.79 ->
        // 3.13 us, 127x4096x3 3.98 -> 3.04, 128x256x1 3.59 -> 2.11, 1000x64x3
        // 3.55 -> 2.58. With K = 16384 its blocked scale-pair loads (one 2-byte
        // pair per lane, 32 lines per wave-wide load) made it slower (896x16384x1
        // 4.86 -> 5.96 us), and so did 750 workgroups of 1000x4096x3 (4.43 -> 4.94).
        pl.row_cpl = pow2_ceil(cdiv(nchunks, 64));
        pl.spw = 1;
        pl.P = pl.ns;
        pl.n_wg = L * pl.ns;
        pl.lpr = 64;
        pl.stage_bytes = 0;
        pl.lds_bytes = 0;
        pl.bfirst = pl.ilv = 0;
        return pl;
    }
    if (nv == 1 && S == 1 && nchunks <= 64 * kRowsMaxCpl && rows_kernel_applies(M, K, L)) {
        // many rows, short K: the multi-row kernel (32 rows per workgroup,
        // several workgroups per CU, one memory round trip each)
        pl.rows_cpl = pow2_ceil(cdiv(nchunks, 64));
        pl.spw = 8;
        pl.P = (int)(cdiv(M, 128) * 4);
        pl.n_wg = (int64_t)L * pl.P;
        pl.lpr = 64;
        pl.stage_bytes = 0;
        pl.lds_bytes = (int)(cdiv(cdiv(K / 16, 4), 8) * kDmaBytes);
        pl.bfirst = pl.ilv = 0;
        return pl;
    }
    if (nv == 1 && S == 1 && nchunks > 64 * kRowMaxCpl && nchunks <= kRowThreads * kWideMaxCpl &&
        (int64_t)L * M <= kWideMaxRows) {
        // few rows, longer K: one row per workgroup of 4 waves, one round of
        // loads (wide-row kernel). Measured against the main kernel:
        // 127x16384x1 4.26 -> 3.12-3.33 us, 127x16384x3 4.67 -> 4.34-4.41;
        // with 896 or 1000 rows it was slower (4.9 -> 6.7 us), hence the bound.
        pl.wide_cpl = pow2_ceil(cdiv(nchunks, kRowThreads));
        pl.spw = 1;
        pl.P = M;
        pl.n_wg = (int64_t)L * M;
        pl.lpr = kRowThreads;
        pl.stage_bytes = 0;
        pl.lds_bytes = 0;
        pl.bfirst = pl.ilv = 0;
        return pl;
    }
    pl.stage_bytes = stage_bytes(pl.lpr, spw);
    pl.lds_bytes = (int)lds_of(spw);
    pl.wide_plain = (nchunks % 8 == 0 && kc % 8 == 0) ? 1 : 0;
    // row rounds of a full workgroup: 4*spw rows, kThreads/lpr rows per round
    pl.bfirst = cdiv(4 * spw * pl.lpr, kThreads) <= kBFirstMaxRounds ? 1 : 0;
    pl.ilv = pl.lpr <= 64 && !pl.bfirst ? 1 : 0;
    if (S > 1) {
        pl.ws_partials = align_up((size_t)(L * M * S) * sizeof(float), kWsAlign);
        pl.ws_total = kCounterBytes + pl.ws_partials;
    }
    return pl;
}

thread_local int g_last_hip_error = 0;

template <int LAYOUT, int LPR, bool SPLIT, bool BFIRST, bool ILV, int NV>
hipError_t launch_kernel(const Plan &pl, const void *a, const void *b, const void *sfa, const void *sfb,
                         void *c, const Params &p, hipStream_t st)
{
    const dim3 grid((uint32_t)pl.n_wg), block(kBlock);
    hipLaunchKernelGGL((nvfp4_gemv_kernel<LAYOUT, LPR, SPLIT, BFIRST, ILV, NV>), grid, block, pl.lds_bytes, st,
                       (const uint8_t *)a, (uint32_t)pl.n_wg, p.M, p.K, p.L, p.spw, p.ns, p.kc_split,
                       p.a_row, p.a_extent, p.P, p.stage_bytes, (const uint8_t *)b, (const uint8_t *)sfa,
                       (const uint8_t *)sfb, (uint16_t *)c, p);
    return hipGetLastError();
}

template <int LAYOUT, int LPR, bool SPLIT, int NV>
hipError_t launch_split(const Plan &pl, const void *a, const void *b, const void *sfa, const void *sfb,
                        void *c, const Params &p, hipStream_t st)
{
    if constexpr (LPR <= 64) {                             // the plan sets ilv only there, never with bfirst
        if (pl.ilv)
            return launch_kernel<LAYOUT, LPR, SPLIT, false, true, NV>(pl, a, b, sfa, sfb, c, p, st);
    }
    return pl.bfirst ? launch_kernel<LAYOUT, LPR, SPLIT, true, false, NV>(pl, a, b, sfa, sfb, c, p, st)
                     : launch_kernel<LAYOUT, LPR, SPLIT, false, false, NV>(pl, a, b, sfa, sfb, c, p, st);
}

template <int LAYOUT, int LPR, int NV>
hipError_t launch_lpr(const Plan &pl, const void *a, const void *b, const void *sfa, const void *sfb,
                      void *c, const Params &p, hipStream_t st)
{
    if constexpr (NV == 1) {                               // several vectors never split K
        if (pl.S > 1)
            return launch_split<LAYOUT, LPR, true, NV>(pl, a, b, sfa, sfb, c, p, st);
    }
    return launch_split<LAYOUT, LPR, false, NV>(pl, a, b, sfa, sfb, c, p, st);
}

template <int LAYOUT, int NV>
hipError_t launch_layout(const Plan &pl, const void *a, const void *b, const void *sfa, const void *sfb,
                         void *c, const Params &p, hipStream_t st)
{
    switch (pl.lpr) {
    case 256: return launch_lpr<LAYOUT, 256, NV>(pl, a, b, sfa, sfb, c, p, st);
    case 128: return launch_lpr<LAYOUT, 128, NV>(pl, a, b, sfa, sfb, c, p, st);
    case 64: return launch_lpr<LAYOUT, 64, NV>(pl, a, b, sfa, sfb, c, p, st);
    case 32: return launch_lpr<LAYOUT, 32, NV>(pl, a, b, sfa, sfb, c, p, st);
    case 16: return launch_lpr<LAYOUT, 16, NV>(pl, a, b, sfa, sfb, c, p, st);
    case 8: return launch_lpr<LAYOUT, 8, NV>(pl, a, b, sfa, sfb, c, p, st);
    case 4: return launch_lpr<LAYOUT, 4, NV>(pl, a, b, sfa, sfb, c, p, st);
    case 2: return launch_lpr<LAYOUT, 2, NV>(pl, a, b, sfa, sfb, c, p, st);
    default: return launch_lpr<LAYOUT, 1, NV>(pl, a, b, sfa, sfb, c, p, st);
    }
}

// Dense strides: the layouts of the header (batch strides do not matter for one batch)
bool dense_row_strides(const Params &p, int sf_layout)
{
    const int64_t M = p.M, K = p.K, nkb = K / 16, ncb = (nkb + 3) / 4;
    const bool blocked = sf_layout == NVFP4_SF_BLOCKED;
    if (p.a_row != K / 2 || (!blocked && p.sfa_row != nkb))
        return false;
    if (p.L == 1)
        return true;
    return p.a_batch == M * (K / 2) && p.b_batch == K / 2 && p.c_batch == M &&
           p.sfa_batch == (blocked ? cdiv(M, 128) * ncb * 512 : M * nkb) &&
           p.sfb_batch == (blocked ? ncb * 512 : nkb);
}

template <int LAYOUT, bool DENSE>
hipError_t launch_row_kernels(const Plan &pl, const void *a, const void *b, const void *sfa, const void *sfb,
                              void *c, const Params &p, hipStream_t st)
{
    const dim3 grid((uint32_t)pl.n_wg), block(kRowThreads);
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, grid, block, 0, st, (const uint8_t *)a, (const uint8_t *)b, (const uint8_t *)sfa,
                           (const uint8_t *)sfb, (uint32_t)pl.n_wg, p.M, p.K, p.alpha, (uint16_t *)c, p);
        return hipGetLastError();
    };
    if (pl.rows_cpl > 0) {
        auto go_lds = [&](auto kern) {
            hipLaunchKernelGGL(kern, grid, block, LAYOUT == NVFP4_SF_BLOCKED ? pl.lds_bytes : 0, st,
                               (const uint8_t *)a, (const uint8_t *)b, (const uint8_t *)sfa, (const uint8_t *)sfb,
                               (uint32_t)pl.n_wg, p.M, p.K, p.alpha, (uint16_t *)c, p);
            return hipGetLastError();
        };
        return pl.rows_cpl == 1 ? go_lds(nvfp4_gemv_rows_kernel<LAYOUT, 1, DENSE>)
                                : go_lds(nvfp4_gemv_rows_kernel<LAYOUT, 2, DENSE>);
    }
    if (pl.row_cpl > 0) {
        switch (pl.row_cpl) {
        case 1: return go(nvfp4_gemv_row_kernel<LAYOUT, 1, DENSE>);
        case 2: return go(nvfp4_gemv_row_kernel<LAYOUT, 2, DENSE>);
        case 4: return go(nvfp4_gemv_row_kernel<LAYOUT, 4, DENSE>);
        default: return go(nvfp4_gemv_row_kernel<LAYOUT, 8, DENSE>);
        }
    }
    switch (pl.wide_cpl) {
    case 1: return go(nvfp4_gemv_wide_row_kernel<LAYOUT, 1, DENSE>);
    case 2: return go(nvfp4_gemv_wide_row_kernel<LAYOUT, 2, DENSE>);
    default: return go(nvfp4_gemv_wide_row_kernel<LAYOUT, 4, DENSE>);
    }
}

template <int LAYOUT>
hipError_t launch_row(const Plan &pl, const void *a, const void *b, const void *sfa, const void *sfb, void *c,
                      const Params &p, hipStream_t st)
{
    return dense_row_strides(p, LAYOUT) ? launch_row_kernels<LAYOUT, true>(pl, a, b, sfa, sfb, c, p, st)
                                        : launch_row_kernels<LAYOUT, false>(pl, a, b, sfa, sfb, c, p, st);
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
    if (!aligned(a, 16) || !aligned(b, 16) || !aligned(sfa, 16) || !aligned(sfb, 4) || !aligned(c, 2))
        return NVFP4_ERR_MISALIGNED;
    return NVFP4_OK;
}

// Dense operand strides (the layouts of the header).
nvfp4_strides_t dense_strides(int64_t M, int64_t K, int64_t L, int sf_layout)
{
    nvfp4_strides_t s{};
    const int64_t nkb = K / 16, ncb = cdiv(nkb, 4);
    s.a_row = K / 2;
    s.a_batch = M * (K / 2);
    s.b_batch = K / 2;
    s.sfa_row = nkb;
    s.sfa_batch = sf_layout == NVFP4_SF_BLOCKED ? cdiv(M, 128) * ncb * 512 : M * nkb;
    s.sfb_batch = sf_layout == NVFP4_SF_BLOCKED ? ncb * 512 : nkb;
    s.c_batch = M;
    (void)L;
    return s;
}

// Strides the kernel can take (see nvfp4_gemv_strided in the header).
nvfp4_status_t check_strides(const nvfp4_strides_t &s, int64_t M, int64_t K, int64_t L, int sf_layout,
                             const Plan &pl)
{
    const int64_t big = INT64_C(1) << 40;
    auto in = [&](int64_t v, int64_t lo, int64_t mult) { return v >= lo && v < big && v % mult == 0; };
    const bool blocked = sf_layout == NVFP4_SF_BLOCKED;
    if (!in(s.a_row, K / 2, 16) || !in(s.a_batch, 0, 16) || !in(s.b_batch, 0, 16) ||
        !in(s.sfa_batch, 0, blocked ? 16 : 2) || !in(s.sfb_batch, 0, blocked ? 16 : 2) ||
        (!blocked && !in(s.sfa_row, K / 16, 2)) || !in(s.c_batch, L > 1 ? M : 0, 1))
        return NVFP4_ERR_INVALID_STRIDE;
    // a workgroup's A offsets are 32-bit: its rows lie in at most
    // ceil(spw/32) + 1 blocks of 128 rows
    const int64_t span = (cdiv(pl.spw, 32) + 1) * 128;
    if (span * s.a_row + K / 2 > INT64_C(0x7FFFFFFF))
        return NVFP4_ERR_INVALID_STRIDE;
    return NVFP4_OK;
}

nvfp4_status_t launch(const void *a, const void *b, const void *sfa, const void *sfb, void *c,
                      int64_t M, int64_t K, int64_t L, int sf_layout, float alpha, const Plan &pl,
                      const nvfp4_strides_t &sd, void *ws, hipStream_t st)
{
    Params p{};
    p.alpha = alpha;
    p.M = (int32_t)M;
    p.K = (int32_t)K;
    p.L = (int32_t)L;
    p.S = pl.S;
    p.kc_split = pl.kc_split;
    p.P = pl.P;
    p.spw = pl.spw;
    p.ns = pl.ns;
    p.stage_bytes = pl.stage_bytes;
    // plain scales are staged 16 bytes at a time only from 16-byte aligned rows
    p.wide_plain = pl.wide_plain && sd.sfa_row % 16 == 0 && sd.sfa_batch % 16 == 0;
    p.a_row = (int32_t)sd.a_row;
    p.a_batch = sd.a_batch;
    p.a_extent = (L - 1) * sd.a_batch + (M - 1) * sd.a_row + K / 2;
    p.b_batch = sd.b_batch;
    p.sfa_row = sd.sfa_row;
    p.sfa_batch = sd.sfa_batch;
    p.sfb_batch = sd.sfb_batch;
    p.c_batch = sd.c_batch;
    if (pl.S > 1) {
        p.counters = (uint32_t *)ws;
        p.partials = (float *)((char *)ws + kCounterBytes);
    }
    hipError_t e;
    if (pl.row_cpl > 0 || pl.wide_cpl > 0 || pl.rows_cpl > 0) {
        e = sf_layout == NVFP4_SF_PLAIN ? launch_row<NVFP4_SF_PLAIN>(pl, a, b, sfa, sfb, c, p, st)
                                        : launch_row<NVFP4_SF_BLOCKED>(pl, a, b, sfa, sfb, c, p, st);
    } else if (pl.nv == 2) {
        // two vectors, dense: B [L][2][K/2], SFB per vector a row (plain) or
        // the next 16-byte line of each tile (blocked), C [L][2][M]
        p.b_vec = K / 2;
        p.sfb_vec = sf_layout == NVFP4_SF_PLAIN ? K / 16 : 16;
        p.c_vec = M;
        e = sf_layout == NVFP4_SF_PLAIN ? launch_layout<NVFP4_SF_PLAIN, 2>(pl, a, b, sfa, sfb, c, p, st)
                                        : launch_layout<NVFP4_SF_BLOCKED, 2>(pl, a, b, sfa, sfb, c, p, st);
    } else {
        e = sf_layout == NVFP4_SF_PLAIN ? launch_layout<NVFP4_SF_PLAIN, 1>(pl, a, b, sfa, sfb, c, p, st)
                                        : launch_layout<NVFP4_SF_BLOCKED, 1>(pl, a, b, sfa, sfb, c, p, st);
    }
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

// ------------------------------------------------ allocation-free split-K scratch
// nvfp4_gemv_noalloc takes its split-K workspace (tickets, then float32
// partials) from this file-scope device array instead of hipMalloc: one copy
// per GPU the library runs on, held until the process ends. In host code the
// name `scratch` is only a stand-in for the device symbol; host code uses the
// address hipGetSymbolAddress returns for the current device, kept per device.
constexpr size_t kScratchBytes = 64 * 1024;
static_assert(kScratchBytes > kCounterBytes, "the ticket region fits the scratch array");
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// zeroes n 32-bit words (the ticket region) once per device
__global__ void zero_words_kernel(uint32_t *p, int n)
{
    for (int i = (int)threadIdx.x; i < n; i += (int)blockDim.x)
        p[i] = 0u;
}

std::mutex g_scratch_mutex;
std::vector<void *> g_scratch;    // per device: the scratch array's device address (nullptr: not set up)

// The scratch array of the current device. Set-up (first call on a device):
// its address, and one clear of the ticket region on `st` (a small kernel, not
// a memset, so that it may be captured). Afterwards the tickets stay zero: the
// last workgroup of every row range resets its ticket, and every partial is
// written before it is read.
nvfp4_status_t scratch_for_device(hipStream_t st, void **out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        g_last_hip_error = (int)e;
        return NVFP4_ERR_HIP;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if ((int)g_scratch.size() <= dev)
        g_scratch.resize(dev + 1, nullptr);
    if (!g_scratch[dev]) {
        void *ptr = nullptr;
        if ((e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch))) != hipSuccess || !ptr) {
            g_last_hip_error = (int)e;
            return NVFP4_ERR_HIP;
        }
        hipLaunchKernelGGL(zero_words_kernel, dim3(1), dim3(256), 0, st, (uint32_t *)ptr,
                           (int)(kCounterBytes / sizeof(uint32_t)));
        if ((e = hipGetLastError()) != hipSuccess) {
            g_last_hip_error = (int)e;
            return NVFP4_ERR_HIP;
        }
        g_scratch[dev] = ptr;
    }
    *out = g_scratch[dev];
    return NVFP4_OK;
}

} // namespace

// Two right-hand vectors through the GEMV kernel (A streamed and decoded once),
// for the skinny GEMM with N = 2; dense operands laid out as nvfp4_gemm_small_n
// takes them. Shapes that would need a K-split return NVFP4_ERR_INVALID_SHAPE
// with nothing launched (the caller then uses its own kernel).
nvfp4_status_t nvfp4_gemv_two_vectors(const void *a, const void *b, const void *sfa, const void *sfb, void *c,
                                      int64_t M, int64_t K, int64_t L, int sf_layout, float alpha,
                                      void *stream)
{
    nvfp4_status_t st = validate(a, b, sfa, sfb, c, M, K, L, sf_layout);
    if (st != NVFP4_OK)
        return st;
    if (!std::isfinite(alpha))
        return NVFP4_ERR_INVALID_SCALE;
    const Plan pl = make_plan(M, K, L, 2);
    if (pl.S > 1 || L * 2 * M > INT32_MAX / 2)
        return NVFP4_ERR_INVALID_SHAPE;
    nvfp4_strides_t sd = dense_strides(M, K, L, sf_layout);
    sd.b_batch = K;                                        // two packed vectors per batch
    if (sf_layout == NVFP4_SF_PLAIN)
        sd.sfb_batch = 2 * (K / 16);                       // blocked: both rows sit in one 128-row block
    sd.c_batch = 2 * M;
    return launch(a, b, sfa, sfb, c, M, K, L, sf_layout, alpha, pl, sd, nullptr, (hipStream_t)stream);
}

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
    return launch(a, b, sfa, sfb, c, M, K, L, sf_layout, 1.0f, pl, dense_strides(M, K, L, sf_layout), ws,
                  (hipStream_t)stream);
}

nvfp4_status_t nvfp4_gemv_noalloc(const void *a, const void *b, const void *sfa, const void *sfb, void *c,
                                  int64_t M, int64_t K, int64_t L, int sf_layout, void *stream)
{
    nvfp4_status_t st = validate(a, b, sfa, sfb, c, M, K, L, sf_layout);
    if (st != NVFP4_OK)
        return st;
    const Plan pl = make_plan(M, K, L);
    void *ws = nullptr;
    if (pl.ws_total > 0) {
        if (pl.ws_total > kScratchBytes)
            return NVFP4_ERR_WORKSPACE;                    // beyond the fixed scratch array
        if ((st = scratch_for_device((hipStream_t)stream, &ws)) != NVFP4_OK)
            return st;
    }
    return launch(a, b, sfa, sfb, c, M, K, L, sf_layout, 1.0f, pl, dense_strides(M, K, L, sf_layout), ws,
                  (hipStream_t)stream);
}

size_t nvfp4_gemv_noalloc_scratch_bytes(void) { return kScratchBytes; }

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
    return launch(a, b, sfa, sfb, c, M, K, L, sf_layout, 1.0f, pl, dense_strides(M, K, L, sf_layout),
                  workspace, (hipStream_t)stream);
}

nvfp4_status_t nvfp4_gemv_scaled(const void *a, const void *b, const void *sfa, const void *sfb,
                                 void *c, int64_t M, int64_t K, int64_t L, int sf_layout,
                                 float alpha, void *workspace, size_t workspace_bytes,
                                 void *stream)
{
    nvfp4_status_t st = validate(a, b, sfa, sfb, c, M, K, L, sf_layout);
    if (st != NVFP4_OK)
        return st;
    const nvfp4_strides_t sd = dense_strides(M, K, L, sf_layout);
    return nvfp4_gemv_strided(a, b, sfa, sfb, c, M, K, L, sf_layout, &sd, alpha, workspace,
                              workspace_bytes, stream);
}

nvfp4_status_t nvfp4_gemv_strided(const void *a, const void *b, const void *sfa, const void *sfb,
                                  void *c, int64_t M, int64_t K, int64_t L, int sf_layout,
                                  const nvfp4_strides_t *strides, float alpha, void *workspace,
                                  size_t workspace_bytes, void *stream)
{
    nvfp4_status_t st = validate(a, b, sfa, sfb, c, M, K, L, sf_layout);
    if (st != NVFP4_OK)
        return st;
    if (!strides)
        return NVFP4_ERR_NULL_POINTER;
    if (!std::isfinite(alpha))
        return NVFP4_ERR_INVALID_SCALE;
    const Plan pl = make_plan(M, K, L);
    if ((st = check_strides(*strides, M, K, L, sf_layout, pl)) != NVFP4_OK)
        return st;
    void *ws = workspace;
    if (pl.ws_total > 0) {
        if (!workspace) {
            if (workspace_bytes != 0)
                return NVFP4_ERR_WORKSPACE;
            if ((st = device_workspace(pl.ws_total, &ws)) != NVFP4_OK)
                return st;
        } else if (workspace_bytes < pl.ws_total || !aligned(workspace, kWsAlign)) {
            return NVFP4_ERR_WORKSPACE;
        }
    }
    return launch(a, b, sfa, sfb, c, M, K, L, sf_layout, alpha, pl, *strides, ws, (hipStream_t)stream);
}

void nvfp4_gemv_dense_strides(int64_t M, int64_t K, int64_t L, int sf_layout, nvfp4_strides_t *strides)
{
    if (strides)
        *strides = dense_strides(M, K, L, sf_layout);
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
    plan->rows_per_wg = pl.wide_cpl > 0 ? 1 : 4 * pl.spw;
    plan->k_splits = pl.S;
    plan->k_per_split = pl.kc_split * 32;
    plan->workgroups = pl.n_wg;
    plan->threads_per_wg = (pl.row_cpl > 0 || pl.wide_cpl > 0 || pl.rows_cpl > 0) ? kRowThreads : kBlock;
    plan->lds_bytes = pl.lds_bytes;
    return NVFP4_OK;
}

nvfp4_status_t nvfp4_gemv_two_vectors_plan(int64_t M, int64_t K, int64_t L, nvfp4_plan_t *plan)
{
    if (!plan)
        return NVFP4_ERR_NULL_POINTER;
    nvfp4_status_t st = check_shape(M, K, L);
    if (st != NVFP4_OK)
        return st;
    const Plan pl = make_plan(M, K, L, 2);
    if (pl.S > 1 || L * 2 * M > INT32_MAX / 2)
        return NVFP4_ERR_INVALID_SHAPE;
    plan->lanes_per_row = pl.lpr;
    plan->rows_per_wg = 4 * pl.spw;
    plan->k_splits = pl.S;
    plan->k_per_split = pl.kc_split * 32;
    plan->workgroups = pl.n_wg;
    plan->threads_per_wg = kBlock;
    plan->lds_bytes = pl.lds_bytes;
    return NVFP4_OK;
}

const char *nvfp4_status_string(int status)
{
    switch (status) {
    case NVFP4_OK: return "success";
    case NVFP4_ERR_NULL_POINTER: return "a required pointer is NULL";
    case NVFP4_ERR_INVALID_SHAPE: return "invalid shape (need M, K, L >= 1, K % 32 == 0, sizes in range)";
    case NVFP4_ERR_MISALIGNED: return "misaligned pointer (a, b, sfa: 16 B; sfb: 4 B; c: 2 B)";
    case NVFP4_ERR_INVALID_LAYOUT: return "invalid scale layout";
    case NVFP4_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case NVFP4_ERR_HIP: return "HIP runtime error";
    case NVFP4_ERR_INVALID_SCALE: return "global scale alpha is not finite";
    case NVFP4_ERR_INVALID_STRIDE: return "operand stride out of range or misaligned";
    default: return "unknown status";
    }
}

int nvfp4_last_hip_error(void) { return g_last_hip_error; }

} // extern "C"

void nvfp4_record_hip_error(int error) { g_last_hip_error = error; }
