// NVFP4 block-scaled skinny GEMM for a few right-hand vectors (N = 1..8) on
// MI355X (gfx950): a dot-product kernel for N <= 2 and a matrix-core kernel
// from N = 3.
//
// c[l][n][m] = fp16( alpha * sum_k e2m1(A[l][m][k]) e4m3(SFA[l][m][k/16])
//                                 * e2m1(B[l][n][k]) e4m3(SFB[l][n][k/16]) )
// the general case of the product kernelbot NVFP4 GEMV submission 103289 hands
// to `torch._scaled_mm` (a @ b^T with block scales, float16 out); the GEMV is
// its N = 1 column. A is streamed once for all N vectors, so each chunk of A
// is decoded once and dotted with N vectors of b'.
//
// Dot-product kernel (N <= 2, where the GEMV kernel is not used). A workgroup
// (4 waves, 256 lanes) owns a contiguous range of R
// rows of one batch. Lane j owns chunk c0 + j of every K-segment of 256
// chunks (8192 k) and keeps b'_n = e2m1(B_n) * e4m3(SFB_n) of that chunk for
// all N vectors in registers (16 VGPRs each, exact float16). It walks the
// rows with a ring of kSnRing rows of A and SFA loads in flight, decodes the
// row's chunk once (v_cvt_scalef32_pk_f16_fp4), forms the two exact 16-element
// block sums against each b'_n (v_dot2_f32_f16), applies the SFA pair, and
// sums the wave's lanes with DPP; per-wave sums go to LDS and are added in a
// fixed order at the end, then rounded once to float16.
//
// From N = 3 the product runs on the matrix cores instead: a' = e2m1(A) *
// e4m3(SFA) and b' are both exact in float16 (an E2M1 value has two
// significant bits, an E4M3 one four; |a'| <= 6 * 448 and the smallest
// nonzero one is 2^-10, a float16 normal), so the block scales are applied
// before the contraction and sum_k a' b' is a plain float16 matrix product with
// float32 accumulation. One v_mfma_f32_16x16x32_f16 takes 16 rows of A by 16
// vector slots (N used, the others zero) over 32 k; its cost does not depend
// on N, where the dot-product kernel's grows with it. Three matrix-core
// kernels share that layout: with plain scales the unstaged one (each step
// loads its scale pairs and B from global memory); with blocked scales a
// staged one (B and the scales in LDS, only A read from global memory in the
// loop), streamed by a staging wave for grids of up to one workgroup per CU,
// staged all at once up front for larger grids.
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
// Workgroups to aim for: one per CU (N = 2 on the headline A: 27.8 us with
// one, 30.9 with two).
constexpr int64_t kSnTargetWGs = 256;

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

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

// Unstaged matrix-core kernel. A wave owns kMfRT tiles of 16 rows and every
// kMfWaves-th group of kMfGroup K-steps (one step = 4 chunks, 128 k), so the
// kMfWaves waves of a workgroup read neighbouring pieces of the same rows at
// the same time; their partial tiles are added in LDS in a fixed order. In a step, lane group g (lanes 16g .. 16g+15) takes chunk g:
// lane i of the group holds 16 bytes of row i of each tile (the MFMA's A
// operand, k split into four runs of 8) and the same chunk of vector i (its B
// operand; zero for i >= N). The 16x16 result has lane L holding rows
// 4 (L / 16) + j, j < 4, of vector slot L % 16.
constexpr int kMfMinN = 3;                    // N from which the matrix-core kernel runs
constexpr int kMfRT = 2;                      // 16-row tiles per wave
constexpr int kMfWaves = 4;                   // waves per workgroup, splitting K
constexpr int kMfThreads = 64 * kMfWaves;
constexpr int kMfRing = 4;                    // K-steps of loads in flight per lane
constexpr int kMfGroup = 1;                   // consecutive K-steps a wave takes in turn (a power of 2)

struct MfParams {
    int32_t M, K, L, N;
    int32_t P;                                // workgroups per batch
    int64_t sfa_batch, sfb_batch;             // bytes per batch of SFA / SFB
    float alpha;
};

template <int LAYOUT>
__global__ __launch_bounds__(kMfThreads) void nvfp4_gemm_small_n_mfma_kernel(
    const uint8_t *__restrict__ A, const uint8_t *__restrict__ B, const uint8_t *__restrict__ SFA,
    const uint8_t *__restrict__ SFB, uint16_t *__restrict__ C, MfParams p)
{
    __shared__ float4_t mf_part[kMfWaves][kMfRT][64];
    const uint32_t lid = xcd_remap(blockIdx.x, gridDim.x);
    const int32_t tile = (int32_t)(lid % (uint32_t)p.P), l = (int32_t)(lid / (uint32_t)p.P);
    const int32_t M = p.M, K = p.K, N = p.N;
    const int32_t nchunks = K >> 5, nkb = K >> 4, ncb = (nkb + 3) >> 2;
    const int32_t nfull = nchunks >> 2;                               // steps with all 4 chunks inside K
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);        // wave-uniform: scalar loop bounds
    const int grp = lane >> 4, i16 = lane & 15;
    const int32_t r0 = tile * (16 * kMfRT);
    // the wave's local steps u = 0 .. nu-1 are the K-steps
    // (u / kMfGroup) * kMfWaves * kMfGroup + wave * kMfGroup + u % kMfGroup
    constexpr int32_t kSpan = kMfWaves * kMfGroup;
    const int32_t ncyc = nfull / kSpan;
    const int32_t nu = ncyc * kMfGroup + min(max(nfull - ncyc * kSpan - wave * kMfGroup, 0), kMfGroup);
    const int32_t s_begin = 0, s_end = nu;
    const int64_t row_bytes = K >> 1;
    // step s of chunk column grp: A and B move by 64 bytes, a scale pair by
    // 8 bytes (plain) or two 512-byte tiles (blocked; the pair's place in the
    // tile depends only on the chunk's parity, which is grp's)
    constexpr int64_t kSfStep = LAYOUT == NVFP4_SF_PLAIN ? 8 : 1024;

    int32_t rows[kMfRT];                      // this lane's row of each tile (clamped: every load is real)
    const uint8_t *a_ptr[kMfRT], *sa_ptr[kMfRT];
    const uint8_t *sfa_l = SFA + (int64_t)l * p.sfa_batch;
#pragma unroll
    for (int t = 0; t < kMfRT; ++t) {
        rows[t] = min(r0 + 16 * t + i16, M - 1);
        a_ptr[t] = A + ((int64_t)l * M + rows[t]) * row_bytes + grp * 16;
        sa_ptr[t] = sfa_l + sn_pair_offset<LAYOUT>(rows[t], grp, nkb, ncb);
    }
    const int32_t n = min(i16, N - 1);
    const bool n_live = i16 < N;
    const uint8_t *b_row = B + ((int64_t)l * N + n) * row_bytes;
    const uint8_t *sfb_l = SFB + (int64_t)l * p.sfb_batch;
    const uint8_t *b_ptr = b_row + grp * 16;
    const uint8_t *sb_ptr = sfb_l + sn_pair_offset<LAYOUT>(n, grp, nkb, ncb);

    float4_t acc[kMfRT];
#pragma unroll
    for (int t = 0; t < kMfRT; ++t)
        acc[t] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

    // one step: a' of each tile and b' from the codes and scale pairs (a
    // vector slot past N gets a zero scale pair, so b' = 0 exactly), then
    // four MFMAs per tile over the chunk's four runs of 8 k
    auto mma_step = [&](const uint4_t (&araw)[kMfRT], const uint32_t (&sa)[kMfRT], uint4_t braw, uint32_t sb) {
        uint4_t bp[4];
        make_bprime(braw, sb, bp);
#pragma unroll
        for (int t = 0; t < kMfRT; ++t) {
            uint4_t ap[4];
            make_bprime(araw[t], sa[t], ap);                           // a' = e2m1(A) e4m3(SFA), exact
#pragma unroll
            for (int q = 0; q < 4; ++q)
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, ap[q]),
                                                                __builtin_bit_cast(half8_t, bp[q]), acc[t], 0, 0,
                                                                0);
        }
    };

    if (s_begin < s_end) {
        uint4_t abuf[kMfRing][kMfRT], bbuf[kMfRing];
        uint32_t sabuf[kMfRing][kMfRT], sbbuf[kMfRing];
        // loads of step s (s_begin <= s < s_end) into a ring slot. A is read
        // with the default cache policy: a step takes 64 of a row's 128-byte
        // line and the next step the other 64, which then hits L2 (with
        // non-temporal loads about 5% of the lines were fetched twice)
        auto load_step = [&](int32_t u, int slot) {
            const int32_t s = (u / kMfGroup) * kSpan + wave * kMfGroup + u % kMfGroup;
            const int64_t ao = (int64_t)s * 64, so = (int64_t)s * kSfStep;
#pragma unroll
            for (int t = 0; t < kMfRT; ++t) {
                abuf[slot][t] = *(const uint4_t *)(a_ptr[t] + ao);
                sabuf[slot][t] = *(const uint16_t *)(sa_ptr[t] + so);
            }
            bbuf[slot] = *(const uint4_t *)(b_ptr + ao);
            sbbuf[slot] = *(const uint16_t *)(sb_ptr + so);
        };
#pragma unroll
        for (int d = 0; d < kMfRing; ++d) {
            if (s_begin + d < s_end)                                   // in slot order, as in the loop
                load_step(s_begin + d, d);
            __builtin_amdgcn_sched_barrier(0);
        }
        // whole rings whose refills all fall before s_end, unconditional (a
        // branch per slot here made the compiler drain the loads at every
        // back-edge); then the last ring, refilled only up to s_end; then the
        // steps still in the ring. No load reads past the wave's last step.
        int32_t s0 = s_begin;
        for (; s0 + 2 * kMfRing <= s_end; s0 += kMfRing) {
#pragma unroll
            for (int d = 0; d < kMfRing; ++d) {
                // consume the slot, then refill it: its registers are reused
                // in place (refilling before the decode kept two copies of
                // the ring live and the compiler drained the loads every ring)
                mma_step(abuf[d], sabuf[d], bbuf[d], n_live ? sbbuf[d] : 0u);
                __builtin_amdgcn_sched_barrier(0);                     // keep the refill here, not
                load_step(s0 + d + kMfRing, d);                        // sunk to the end of the ring
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int d = 0; d < kMfRing; ++d) {
            if (s0 + d < s_end) {
                mma_step(abuf[d], sabuf[d], bbuf[d], n_live ? sbbuf[d] : 0u);
                __builtin_amdgcn_sched_barrier(0);
                if (s0 + d + kMfRing < s_end)
                    load_step(s0 + d + kMfRing, d);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        s0 += kMfRing;
#pragma unroll
        for (int d = 0; d < kMfRing; ++d)
            if (s0 + d < s_end)
                mma_step(abuf[d], sabuf[d], bbuf[d], n_live ? sbbuf[d] : 0u);
    }

    // the last step of a K that is not a multiple of 128: chunks past K (lane
    // groups past the end) load a real chunk and get zero scale pairs, so they
    // add exact zeros; taken by the last wave
    if ((nchunks & 3) != 0 && wave == kMfWaves - 1) {
        const int32_t c = min(4 * nfull + grp, nchunks - 1);
        const bool live = 4 * nfull + grp < nchunks;
        uint4_t araw[kMfRT];
        uint32_t sa[kMfRT];
#pragma unroll
        for (int t = 0; t < kMfRT; ++t) {
            araw[t] = __builtin_nontemporal_load(
                (const uint4_t *)(A + ((int64_t)l * M + rows[t]) * row_bytes + (int64_t)c * 16));
            const uint32_t v = *(const uint16_t *)(sfa_l + sn_pair_offset<LAYOUT>(rows[t], c, nkb, ncb));
            sa[t] = live ? v : 0u;
        }
        const uint4_t braw = *(const uint4_t *)(b_row + (int64_t)c * 16);
        const uint32_t v = *(const uint16_t *)(sfb_l + sn_pair_offset<LAYOUT>(n, c, nkb, ncb));
        mma_step(araw, sa, braw, (live && n_live) ? v : 0u);
    }

#pragma unroll
    for (int t = 0; t < kMfRT; ++t)
        mf_part[wave][t][lane] = acc[t];
    __syncthreads();
    for (int e = tid; e < kMfRT * 64 * 4; e += kMfThreads) {
        const int t = e >> 8, ln = (e >> 2) & 63, j = e & 3;
        const int32_t col = ln & 15, row = r0 + 16 * t + 4 * (ln >> 4) + j;
        if (col < N && row < M) {
            float v = 0.0f;
#pragma unroll
            for (int w = 0; w < kMfWaves; ++w)
                v += ((const float *)&mf_part[w][t][ln])[j];
            C[((int64_t)l * N + col) * M + row] = f16_bits(v * p.alpha);
        }
    }
}

// Streamed staged matrix-core kernel (blocked scales, N >= 3). Same MFMA
// layout as the kernel above, but the computing waves read only A from
// global memory: per step loads of the scale pairs and of B (a few bytes per
// lane, touching several lines each) took about a third of the streaming
// time there. A fifth wave stages B, the SFB dwords and the workgroup's SFA
// lines into LDS with direct-to-LDS copies, in blocks of kMsBlkSteps K-steps,
// two blocks ahead of the computing waves, in three LDS slots; a barrier per
// block hands a slot over. The computing waves' loads and waits never see the
// copies, so their rings of A stay full across the blocks (copies issued by
// the computing waves themselves, which the compiler cannot count, made its
// waits for the ring drain it at every block).
//
// Rows. A blocked scale tile is 128 rows x 4 blocks; its 16-byte piece p holds
// the 4 blocks of rows p, p+32, p+64, p+96. Workgroup h (0..3) of a 128-row
// block takes the pieces 8h .. 8h+7, i.e. the 32 rows 8h + p' + 32j (p' < 8,
// j < 4), so its SFA is one whole 128-byte line per tile and no line is
// shared. MFMA row m (0..15) of tile t is row 8h + (m & 7) + 32 (2 (m >> 3) + t):
// one 8-byte LDS read then gives a lane the 4 blocks of its row in both tiles.
//
// K-steps. Computing wave cw (0..3) takes the K-steps s = 4u + cw, u = 0, 1, ...
// (local step u). Block k is the K-steps 32k .. 32k+31 (local steps 8k .. 8k+7
// of every computing wave). A slot holds, per K-step sb of the block: B as
// [sb][NP vectors][4 chunks of 16 bytes], the SFA lines as [sb][2 groups][128
// bytes], the SFB dwords as [sb][NP vectors][2 groups][4 bytes].
constexpr int kMsWgPerBlock = 4;              // workgroups per 128-row block
constexpr int kMsWaves = kMfWaves + 1;        // wave 0 stages, waves 1..4 compute
constexpr int kMsThreads = 64 * kMsWaves;
constexpr int kMsBlkSteps = 32;               // K-steps per staged block (8 local steps of each computing wave)
constexpr int kMsLocal = kMsBlkSteps / kMfWaves;
constexpr int kMsSlots = 3;                   // slots in LDS: blocks k (computed), k+1, k+2 (landing)

template <int NP>
struct MsSlot {
    static constexpr int kB = kMsBlkSteps * 64 * NP;       // B bytes
    static constexpr int kSfa = kMsBlkSteps * 256;         // SFA bytes
    static constexpr int kSfb = kMsBlkSteps * 8 * NP;      // SFB bytes
    static constexpr int kBytes = kB + kSfa + kSfb;
    static constexpr int kCopiesB = kB / 1024;             // 16-byte copies, 64 lanes
    static constexpr int kCopiesSfa = kSfa / 1024;
    static constexpr int kCopiesSfb = kSfb / 256;          // 4-byte copies
    static constexpr int kCopies = kCopiesB + kCopiesSfa + kCopiesSfb;
    static_assert(kCopies <= 63, "one block of copies fits the wait counter");
};

// 16 or 4 bytes per lane from global memory straight into LDS at lds_dst +
// lane*16 (lane*4): global_load_lds_dwordx4 / _dword, LDS address from M0.
// Inline assembly, so the compiler does not track the copies: the staging
// wave waits for them itself. Nothing else in this file uses M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __attribute__((always_inline)) inline void ms_copy16(const void *src, const uint8_t *lds_dst)
{
    const uint32_t addr = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_dst);
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "s"(addr)
                 : "memory", "m0");
}
__device__ __attribute__((always_inline)) inline void ms_copy4(const void *src, const uint8_t *lds_dst)
{
    const uint32_t addr = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_dst);
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" : : "v"(src), "s"(addr)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt vmcnt(K0), other counters unconstrained
template <int K0>
__device__ __attribute__((always_inline)) inline void ms_wait_vmcnt()
{
    static_assert(K0 >= 0 && K0 < 64, "vmcnt holds 0..63");
    __builtin_amdgcn_s_waitcnt((0x0F70 & ~0xC00F) | (K0 & 15) | ((K0 >> 4) << 14));
}

// s_waitcnt vmcnt(k) for a wave-uniform k in 0..63
template <int K0 = 0>
__device__ __attribute__((always_inline)) inline void ms_wait_vmcnt_rt(int k)
{
    if constexpr (K0 < 63) {
        if (k == K0) {
            ms_wait_vmcnt<K0>();
            return;
        }
        ms_wait_vmcnt_rt<K0 + 1>(k);
    } else {
        ms_wait_vmcnt<63>();
    }
}

template <int NP>
__global__ __launch_bounds__(kMsThreads) void nvfp4_gemm_small_n_mfma_staged_kernel(
    const uint8_t *__restrict__ A, const uint8_t *__restrict__ B, const uint8_t *__restrict__ SFA,
    const uint8_t *__restrict__ SFB, uint32_t nL, int32_t M, int32_t K, int32_t N, uint16_t *__restrict__ C,
    MfParams p)
{
    using S = MsSlot<NP>;
    extern __shared__ __attribute__((aligned(16))) uint8_t ms_lds[];     // kMsSlots * S::kBytes
    __shared__ float4_t ms_part[kMfWaves][kMfRT][64];
    // everything the first loads and copies depend on comes from the leading
    // (preloaded) kernel arguments: the grid and the dense batch strides are
    // derived from them, so no kernel-argument read precedes the first load
    const uint32_t P = (uint32_t)((M + 127) >> 7) * kMsWgPerBlock;   // workgroups per batch
    const uint32_t lid = xcd_remap(blockIdx.x, nL * P);
    const int32_t wgb = (int32_t)(lid % P), l = (int32_t)(lid / P);
    const int32_t blk = wgb / kMsWgPerBlock, h = wgb % kMsWgPerBlock;
    const int32_t nchunks = K >> 5, ncb = ((K >> 4) + 3) >> 2;
    const int32_t nfull = nchunks >> 2;                                // whole K-steps
    const int32_t nblk = (nfull + kMsBlkSteps - 1) / kMsBlkSteps;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t row_bytes = K >> 1;
    const int32_t rbase = blk * 128 + 8 * h;                           // row of p' = 0, j = 0

    const uint8_t *b_l = B + (int64_t)l * N * row_bytes;
    const uint8_t *sfa_l = SFA + (int64_t)l * ((M + 127) >> 7) * ncb * 512;   // blocked, dense
    const uint8_t *sfb_l = SFB + (int64_t)l * ncb * 512;                      // N <= 128: one block of rows

    if (wave == 0) {
        // staging wave: block k's copies into slot k % 3, two blocks ahead of
        // the computing waves; a barrier per block hands a slot over. Copies
        // whose K-steps all lie past the last one are left out; stage returns
        // how many it issued, for the waits.
        __builtin_amdgcn_s_setprio(3);
        auto stage = [&](int32_t k) {
            uint8_t *slot = ms_lds + (k % kMsSlots) * S::kBytes;
            const int32_t s0 = k * kMsBlkSteps;
            int32_t issued = 0;
#pragma unroll
            for (int i = 0; i < S::kCopiesB; ++i) {
                if (s0 + (i * 64) / (4 * NP) >= nfull)
                    break;
                const int32_t e = 64 * i + lane;                       // 16-byte unit of the slot's B
                const int32_t s = min(s0 + e / (4 * NP), nfull - 1);   // past the end: clamped, never read
                const int32_t n = min((e >> 2) % NP, N - 1), g = e & 3;
                ms_copy16(b_l + (int64_t)n * row_bytes + (int64_t)(4 * s + g) * 16, slot + i * 1024);
                ++issued;
            }
#pragma unroll
            for (int i = 0; i < S::kCopiesSfa; ++i) {
                if (s0 + 4 * i >= nfull)
                    break;
                const int32_t e = 64 * i + lane;                       // 16-byte piece of the slot's SFA
                const int32_t s = min(s0 + (e >> 4), nfull - 1);
                const int32_t q = 2 * s + ((e >> 3) & 1);
                ms_copy16(sfa_l + ((int64_t)blk * ncb + q) * 512 + (8 * h + (e & 7)) * 16, slot + S::kB + i * 1024);
                ++issued;
            }
#pragma unroll
            for (int i = 0; i < S::kCopiesSfb; ++i) {
                if (s0 + (i * 64) / (2 * NP) >= nfull)
                    break;
                const int32_t e = 64 * i + lane;                       // dword of the slot's SFB
                const int32_t s = min(s0 + e / (2 * NP), nfull - 1);
                const int32_t n = min((e >> 1) % NP, N - 1), q = 2 * s + (e & 1);
                ms_copy4(sfb_l + (int64_t)q * 512 + n * 16, slot + S::kB + S::kSfa + i * 256);
                ++issued;
            }
            return issued;
        };
        __builtin_amdgcn_s_waitcnt(0x0F70);                            // nothing in flight: vmcnt(0)
        int32_t ahead = 0;                                             // copies of the block after k in flight
        if (nblk > 0)
            stage(0);
        if (nblk > 1)
            ahead = stage(1);
        for (int32_t k = 0; k < nblk; ++k) {
            ms_wait_vmcnt_rt(ahead);                                   // block k has landed
            __syncthreads();                                           // hand slot k % 3 over
            ahead = k + 2 < nblk ? stage(k + 2) : 0;                   // into the slot block k-1 used
        }
        __syncthreads();                                               // matches the epilogue's barrier
        return;
    }

    // computing waves
    const int cw = wave - 1;
    const int grp = lane >> 4, i16 = lane & 15;
    const int32_t nu = nfull / kMfWaves + (cw < nfull % kMfWaves ? 1 : 0);
    const uint8_t *a_row[kMfRT], *a_ptr[kMfRT];
#pragma unroll
    for (int t = 0; t < kMfRT; ++t) {
        const int32_t r = min(rbase + (i16 & 7) + 32 * (2 * (i16 >> 3) + t), M - 1);
        a_row[t] = A + ((int64_t)l * M + r) * row_bytes;
        a_ptr[t] = a_row[t] + grp * 16 + (int64_t)cw * 64;
    }
    uint4_t abuf[kMfRing][kMfRT];
    auto load_step = [&](int32_t u, int slot) {
        const int64_t ao = (int64_t)u * (64 * kMfWaves);
#pragma unroll
        for (int t = 0; t < kMfRT; ++t)
            abuf[slot][t] = *(const uint4_t *)(a_ptr[t] + ao);
    };
    // the first ring, loaded without conditions (a slot past the wave's last
    // step loads its last step again, or the row's first 16 bytes when the
    // wave has no step; never used): conditional loads here made the compiler
    // wait for the whole ring at every step of the loop
#pragma unroll
    for (int d = 0; d < kMfRing; ++d) {
#pragma unroll
        for (int t = 0; t < kMfRT; ++t)
            abuf[d][t] = *(const uint4_t *)(nu > 0 ? a_ptr[t] + (int64_t)min(d, nu - 1) * (64 * kMfWaves) : a_row[t]);
        __builtin_amdgcn_sched_barrier(0);
    }
    // alpha, a kernel-argument read, is taken here behind the first ring (its
    // wait overlaps the loads in flight), not in the epilogue, where its
    // latency would add to the kernel's end
    float alpha = p.alpha;
    asm volatile("" : "+s"(alpha));
    __builtin_amdgcn_sched_barrier(0);

    float4_t acc[kMfRT];
#pragma unroll
    for (int t = 0; t < kMfRT; ++t)
        acc[t] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

    const int32_t n = min(i16, N - 1);
    const bool n_live = i16 < N;
    // this lane's LDS offsets in a slot for local step u: K-step sb = 4 (u % 8) + cw of the block
    const int32_t ob = (cw * NP + n) * 64 + grp * 16;
    const int32_t osfb = S::kB + S::kSfa + (cw * NP + n) * 8 + 2 * grp;
    const int32_t osfa = S::kB + cw * 256 + (grp >> 1) * 128 + (i16 & 7) * 16 + 8 * (i16 >> 3);
    const int sa_shift = 16 * (grp & 1);

    struct Staged {
        uint4_t b;
        uint32_t sb;
        uint2_t sa2;
    };
    auto read_staged = [&](int32_t u) {
        const uint8_t *slot = ms_lds + ((u / kMsLocal) % kMsSlots) * S::kBytes;
        const int32_t d = u % kMsLocal;
        Staged o;
        o.b = *(const uint4_t *)(slot + ob + d * (4 * 64 * NP));
        o.sb = *(const uint16_t *)(slot + osfb + d * (4 * 8 * NP));   // a slot past N is zeroed at use
        o.sa2 = *(const uint2_t *)(slot + osfa + d * (4 * 256));
        return o;
    };
    auto mma_step = [&](const uint4_t (&araw)[kMfRT], const Staged &st) {
        uint4_t bp[4];
        make_bprime(st.b, n_live ? st.sb : 0u, bp);
#pragma unroll
        for (int t = 0; t < kMfRT; ++t) {
            const uint32_t sa = ((t == 0 ? st.sa2.x : st.sa2.y) >> sa_shift) & 0xFFFFu;
            uint4_t ap[4];
            make_bprime(araw[t], sa, ap);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, ap[q]),
                                                                __builtin_bit_cast(half8_t, bp[q]), acc[t], 0, 0,
                                                                0);
        }
    };

    // Block k starts with a barrier (the staging wave has landed block k) at
    // local step 8k; each step reads its staged operands from the block's
    // slot (reading them one step ahead measured slower: more registers, and
    // no gain with the ring of A in flight). The rings (4 steps) whose refills all fall
    // before nu run as a loop without conditions; then the last ring, refilled
    // only up to nu, and the steps still in the ring. (A loop body of two
    // rings, or conditional loads before the loop, made the compiler wait for
    // the whole ring at every step.) Every computing wave takes part in all
    // nblk block barriers, also past its own last step.
    int32_t kb = 0;                                                    // block barriers passed
    auto enter_ring = [&](int32_t r) {
        if ((r & 1) == 0) {
            __syncthreads();
            ++kb;
        }
    };
    const int32_t nr = max(0, (nu - kMfRing) / kMfRing);              // rings with every refill inside nu
    for (int32_t r = 0; r < nr; ++r) {
        enter_ring(r);
#pragma unroll
        for (int d = 0; d < kMfRing; ++d) {
            const int32_t u = kMfRing * r + d;
            mma_step(abuf[d], read_staged(u));
            __builtin_amdgcn_sched_barrier(0);
            load_step(u + kMfRing, d);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {                                   // the last ring, then the drain
        const int32_t r = nr + rr;
        if (kMfRing * r < nu) {
            enter_ring(r);
#pragma unroll
            for (int d = 0; d < kMfRing; ++d) {
                const int32_t u = kMfRing * r + d;
                if (u < nu) {
                    mma_step(abuf[d], read_staged(u));
                    __builtin_amdgcn_sched_barrier(0);
                    if (rr == 0 && u + kMfRing < nu)
                        load_step(u + kMfRing, d);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
    }
    for (; kb < nblk; ++kb)
        __syncthreads();

    // the ragged last step (K not a multiple of 128), taken by the last
    // computing wave from global memory: chunks past K read chunk nchunks-1
    // and get zero scale pairs
    if ((nchunks & 3) != 0 && cw == kMfWaves - 1) {
        const int32_t c = min(4 * nfull + grp, nchunks - 1);
        const bool live = 4 * nfull + grp < nchunks;
        uint4_t araw[kMfRT];
        uint32_t sa[kMfRT];
#pragma unroll
        for (int t = 0; t < kMfRT; ++t) {
            const int32_t r = min(rbase + (i16 & 7) + 32 * (2 * (i16 >> 3) + t), M - 1);
            araw[t] = *(const uint4_t *)(A + ((int64_t)l * M + r) * row_bytes + (int64_t)c * 16);
            const uint32_t v = *(const uint16_t *)(sfa_l + sn_pair_offset<NVFP4_SF_BLOCKED>(r, c, K >> 4, ncb));
            sa[t] = live ? v : 0u;
        }
        const uint4_t braw = *(const uint4_t *)(b_l + (int64_t)n * row_bytes + (int64_t)c * 16);
        const uint32_t v = *(const uint16_t *)(sfb_l + sn_pair_offset<NVFP4_SF_BLOCKED>(n, c, K >> 4, ncb));
        uint4_t bp[4];
        make_bprime(braw, (live && n_live) ? v : 0u, bp);
#pragma unroll
        for (int t = 0; t < kMfRT; ++t) {
            uint4_t ap[4];
            make_bprime(araw[t], sa[t], ap);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, ap[q]),
                                                                __builtin_bit_cast(half8_t, bp[q]), acc[t], 0, 0,
                                                                0);
        }
    }

#pragma unroll
    for (int t = 0; t < kMfRT; ++t)
        ms_part[cw][t][lane] = acc[t];
    __syncthreads();
    for (int e = tid - 64; e < kMfRT * 64 * 4; e += kMsThreads - 64) {
        const int t = e >> 8, ln = (e >> 2) & 63, j = e & 3;
        const int m = 4 * (ln >> 4) + j;                               // MFMA row of the result element
        const int32_t col = ln & 15, row = rbase + (m & 7) + 32 * (2 * (m >> 3) + t);
        if (col < N && row < M) {
            float v = 0.0f;
#pragma unroll
            for (int w = 0; w < kMfWaves; ++w)
                v += ((const float *)&ms_part[w][t][ln])[j];
            C[((int64_t)l * N + col) * M + row] = f16_bits(v * alpha);
        }
    }
}

// Up-front staged matrix-core kernel (blocked scales, N >= 3, where all of
// B, the SFB dwords and the workgroup's SFA lines fit in LDS). The same rows,
// MFMA layout and K-steps as the streamed kernel above, but 4 waves and no
// staging wave: a prologue stages the whole K range at once, the first ring
// of A issued first, and one barrier publishes it. Where several workgroups
// share a CU (grids of more than 256 workgroups) the others hide that one
// round trip, and this kernel needs fewer registers and no block barriers
// (4096x7168x8, N = 4: 29.8 against 33.5 us; N = 8: 31.1 against 38.5).
constexpr int kMuDmaBytes = 64 * 16;          // LDS bytes one wave-wide direct-to-LDS copy fills
constexpr int kMuMaxNcb = 256;                // 4-block groups (K / 64) at most
constexpr int kMuMaxDmaPerWave = 40;          // direct-to-LDS copies per wave (the wait counter holds 63)
constexpr int64_t kMuLdsLimit = 150 * 1024;   // dynamic LDS; the static partial tiles take 8 KiB more

struct MuLayout {
    int32_t b_vec;                            // LDS bytes per staged vector of B (16 more than its copies fill)
    int32_t sfb_vec;                          // LDS bytes per vector of staged SFB dwords
    int32_t b_bytes, sfa_bytes, sfb_bytes;    // LDS regions, in this order
    int32_t n_dma_b, n_dma_sfa;               // wave-wide copies per vector of B, and of SFA
    int32_t n_dma_sfb;                        // wave-wide 4-byte copies per vector of SFB
};

// LDS layout: vector n of B at n * b_vec (chunk c at +16 c; b_vec = 16 mod 128,
// so the vectors' chunks fall in different banks), the SFA line of 4-block
// group q at sfa + q * 128, the SFB dword (n, q) at sfb + n * sfb_vec + 4 q
// (sfb_vec / 4 = 2 mod 32; a vector's region holds its copies whole).
__host__ __device__ inline MuLayout mu_layout(int32_t K, int32_t N)
{
    const int32_t nchunks = K >> 5, ncb = ((K >> 4) + 3) >> 2;
    MuLayout o;
    o.n_dma_b = (nchunks + 63) / 64;
    o.n_dma_sfa = (ncb * 8 + 63) / 64;
    o.n_dma_sfb = (ncb + 63) / 64;
    o.b_vec = o.n_dma_b * kMuDmaBytes + 16;
    o.sfb_vec = o.n_dma_sfb * 256 + 8;
    o.b_bytes = (N * o.b_vec + 127) / 128 * 128;
    o.sfa_bytes = o.n_dma_sfa * kMuDmaBytes;
    o.sfb_bytes = N * o.sfb_vec;
    return o;
}

__global__ __launch_bounds__(kMfThreads) void nvfp4_gemm_small_n_mfma_upfront_kernel(
    const uint8_t *__restrict__ A, const uint8_t *__restrict__ B, const uint8_t *__restrict__ SFA,
    const uint8_t *__restrict__ SFB, uint32_t nL, int32_t M, int32_t K, int32_t N, uint16_t *__restrict__ C,
    MfParams p)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t mu_lds[];
    __shared__ float4_t mu_part[kMfWaves][kMfRT][64];
    // everything the first loads and copies depend on comes from the leading
    // (preloaded) kernel arguments: the grid and the dense batch strides are
    // derived from them, so no kernel-argument read precedes the first load
    const uint32_t P = (uint32_t)((M + 127) >> 7) * kMsWgPerBlock;   // workgroups per batch
    const uint32_t lid = xcd_remap(blockIdx.x, nL * P);
    const int32_t wgb = (int32_t)(lid % P), l = (int32_t)(lid / P);
    const int32_t blk = wgb / kMsWgPerBlock, h = wgb % kMsWgPerBlock;
    const int32_t nchunks = K >> 5, ncb = ((K >> 4) + 3) >> 2;
    const int32_t nfull = nchunks >> 2;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = lane >> 4, i16 = lane & 15;
    const int64_t row_bytes = K >> 1;
    const MuLayout lay = mu_layout(K, N);
    uint8_t *const sB = mu_lds;
    uint8_t *const sSFA = mu_lds + lay.b_bytes;
    uint8_t *const sSFB = sSFA + lay.sfa_bytes;
    const int32_t rbase = blk * 128 + 8 * h;                          // row of p' = 0, j = 0

    const uint8_t *b_l = B + (int64_t)l * N * row_bytes;
    const uint8_t *sfa_l = SFA + (int64_t)l * ((M + 127) >> 7) * ncb * 512;   // blocked, dense
    const uint8_t *sfb_l = SFB + (int64_t)l * ncb * 512;                      // N <= 128: one block of rows

    // the wave's local steps u = 0 .. nu-1 are the K-steps u * kMfWaves + wave
    const int32_t nu = nfull / kMfWaves + (wave < nfull % kMfWaves ? 1 : 0);
    const uint8_t *a_ptr[kMfRT];
#pragma unroll
    for (int t = 0; t < kMfRT; ++t) {
        const int32_t r = min(rbase + (i16 & 7) + 32 * (2 * (i16 >> 3) + t), M - 1);
        a_ptr[t] = A + ((int64_t)l * M + r) * row_bytes + grp * 16 + (int64_t)wave * 64;
    }

    // prologue, in issue order: the first ring of A, the copies of B and of
    // the SFA lines, the SFB dwords into registers
    uint4_t abuf[kMfRing][kMfRT];
    auto load_step = [&](int32_t u, int slot) {
        const int64_t ao = (int64_t)u * (64 * kMfWaves);
#pragma unroll
        for (int t = 0; t < kMfRT; ++t)
            abuf[slot][t] = *(const uint4_t *)(a_ptr[t] + ao);
    };
#pragma unroll
    for (int d = 0; d < kMfRing; ++d) {
        if (d < nu)
            load_step(d, d);
        __builtin_amdgcn_sched_barrier(0);
    }
    for (int32_t nv = 0; nv < N; ++nv)
        for (int32_t i = wave; i < lay.n_dma_b; i += kMfWaves)
            ms_copy16(b_l + (int64_t)nv * row_bytes + (int64_t)min(i * 64 + lane, nchunks - 1) * 16,
                      sB + nv * lay.b_vec + i * kMuDmaBytes);
    for (int32_t i = wave; i < lay.n_dma_sfa; i += kMfWaves) {
        const int32_t it = min(i * 64 + lane, ncb * 8 - 1);           // past the end: clamped, never read
        ms_copy16(sfa_l + ((int64_t)blk * ncb + (it >> 3)) * 512 + (8 * h + (it & 7)) * 16, sSFA + i * kMuDmaBytes);
    }
    // SFB of vector nv, 4-block group q: the dword of rows nv < 8 in the
    // first tile row, copied with the others (no register round trip)
    for (int32_t nv = 0; nv < N; ++nv)
        for (int32_t i = wave; i < lay.n_dma_sfb; i += kMfWaves)
            ms_copy4(sfb_l + (int64_t)min(i * 64 + lane, ncb - 1) * 512 + nv * 16,   // past the end: clamped
                     sSFB + nv * lay.sfb_vec + i * 256);
    // alpha, a kernel-argument read, is taken here behind the first loads and
    // copies (its wait overlaps them), not in the epilogue, where its latency
    // would add to the kernel's end
    __builtin_amdgcn_sched_barrier(0);
    float alpha = p.alpha;
    asm volatile("" : "+s"(alpha));
    __builtin_amdgcn_sched_barrier(0);
    ms_wait_vmcnt<0>();                                               // this wave's copies have landed
    __syncthreads();                                                  // B, SFB and SFA are staged

    float4_t acc[kMfRT];
#pragma unroll
    for (int t = 0; t < kMfRT; ++t)
        acc[t] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

    const int32_t n = min(i16, N - 1);
    const bool n_live = i16 < N;
    // LDS addresses of step s = 0 for this lane; a step moves them by
    // 64 (B), 8 (SFB) and 256 (SFA) bytes
    const uint8_t *lb = sB + n * lay.b_vec + grp * 16;
    const uint8_t *lsb = sSFB + n * lay.sfb_vec + 2 * grp;
    const uint8_t *lsa = sSFA + (grp >> 1) * 128 + (i16 & 7) * 16 + 8 * (i16 >> 3);
    const int sa_shift = 16 * (grp & 1);

    // the staged operands of the wave's local step u (clamped to its last
    // step, so that a read ahead past the end stays on real data)
    struct Staged {
        uint4_t b;
        uint32_t sb;
        uint2_t sa2;
    };
    auto read_staged = [&](int32_t u) {
        const int32_t s = min(u, nu - 1) * kMfWaves + wave;
        Staged o;
        o.b = *(const uint4_t *)(lb + s * 64);
        o.sb = *(const uint16_t *)(lsb + s * 8);                      // a slot past N is zeroed at use
        o.sa2 = *(const uint2_t *)(lsa + s * 256);
        return o;
    };
    // one step from the ring slot's A and the staged operands
    auto mma_step = [&](const uint4_t (&araw)[kMfRT], const Staged &st) {
        uint4_t bp[4];
        make_bprime(st.b, n_live ? st.sb : 0u, bp);
#pragma unroll
        for (int t = 0; t < kMfRT; ++t) {
            const uint32_t sa = ((t == 0 ? st.sa2.x : st.sa2.y) >> sa_shift) & 0xFFFFu;
            uint4_t ap[4];
            make_bprime(araw[t], sa, ap);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, ap[q]),
                                                                __builtin_bit_cast(half8_t, bp[q]), acc[t], 0, 0,
                                                                0);
        }
    };

    if (nu > 0) {
        // as in the kernel above: whole rings with unconditional refills, the
        // last ring refilled only up to nu, then the steps still in the ring.
        // The staged operands are read one step ahead, so that their LDS
        // latency hides behind the current step's work.
        Staged cur = read_staged(0);
        int32_t u0 = 0;
        for (; u0 + 2 * kMfRing <= nu; u0 += kMfRing) {
#pragma unroll
            for (int d = 0; d < kMfRing; ++d) {
                const Staged nxt = read_staged(u0 + d + 1);
                __builtin_amdgcn_sched_barrier(0);                     // issue the reads ahead of the step
                mma_step(abuf[d], cur);
                cur = nxt;
                __builtin_amdgcn_sched_barrier(0);
                load_step(u0 + d + kMfRing, d);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int d = 0; d < kMfRing; ++d) {
            if (u0 + d < nu) {
                const Staged nxt = read_staged(u0 + d + 1);
                __builtin_amdgcn_sched_barrier(0);                     // issue the reads ahead of the step
                mma_step(abuf[d], cur);
                cur = nxt;
                __builtin_amdgcn_sched_barrier(0);
                if (u0 + d + kMfRing < nu)
                    load_step(u0 + d + kMfRing, d);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        u0 += kMfRing;
#pragma unroll
        for (int d = 0; d < kMfRing; ++d)
            if (u0 + d < nu) {
                const Staged nxt = read_staged(u0 + d + 1);
                __builtin_amdgcn_sched_barrier(0);                     // issue the reads ahead of the step
                mma_step(abuf[d], cur);
                cur = nxt;
            }
    }

    // the ragged last step (K not a multiple of 128), taken by the last wave:
    // chunks past K read chunk nchunks-1 and get zero scale pairs
    if ((nchunks & 3) != 0 && wave == kMfWaves - 1) {
        const int32_t c = min(4 * nfull + grp, nchunks - 1);
        const bool live = 4 * nfull + grp < nchunks;
        uint4_t araw[kMfRT];
#pragma unroll
        for (int t = 0; t < kMfRT; ++t)
            araw[t] = *(const uint4_t *)(a_ptr[t] - grp * 16 - (int64_t)wave * 64 + (int64_t)c * 16);
        // staged operands of chunk c: the lane's step-0 addresses are for
        // chunk grp, so move them to chunk c by hand
        const uint4_t braw = *(const uint4_t *)(sB + n * lay.b_vec + c * 16);
        const uint32_t sb = (live && n_live) ? (uint32_t) * (const uint16_t *)(sSFB + n * lay.sfb_vec + 2 * c) : 0u;
        const uint2_t sa2 = *(const uint2_t *)(sSFA + (c >> 1) * 128 + (i16 & 7) * 16 + 8 * (i16 >> 3));
        const int sh = 16 * (c & 1);
        uint4_t bp[4];
        make_bprime(braw, sb, bp);
#pragma unroll
        for (int t = 0; t < kMfRT; ++t) {
            const uint32_t sa = live ? ((t == 0 ? sa2.x : sa2.y) >> sh) & 0xFFFFu : 0u;
            uint4_t ap[4];
            make_bprime(araw[t], sa, ap);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, ap[q]),
                                                                __builtin_bit_cast(half8_t, bp[q]), acc[t], 0, 0,
                                                                0);
        }
    }

#pragma unroll
    for (int t = 0; t < kMfRT; ++t)
        mu_part[wave][t][lane] = acc[t];
    __syncthreads();
    for (int e = tid; e < kMfRT * 64 * 4; e += kMfThreads) {
        const int t = e >> 8, ln = (e >> 2) & 63, j = e & 3;
        const int m = 4 * (ln >> 4) + j;                               // MFMA row of the result element
        const int32_t col = ln & 15, row = rbase + (m & 7) + 32 * (2 * (m >> 3) + t);
        if (col < N && row < M) {
            float v = 0.0f;
#pragma unroll
            for (int w = 0; w < kMfWaves; ++w)
                v += ((const float *)&mu_part[w][t][ln])[j];
            C[((int64_t)l * N + col) * M + row] = f16_bits(v * alpha);
        }
    }
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

        // the lane sums of a whole ring come after its dot products, as
        // independent DPP chains (N = 2: 27.8 -> 25.5 us on the headline A)
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
    // N >= kMfMinN runs the matrix-core kernel
    static_assert(kMfMinN == 3, "the dot-product kernel is instantiated for N = 1, 2");
    return N == 1 ? sn_launch<LAYOUT, 1>(grid, lds, a, b, sfa, sfb, c, p, st)
                  : sn_launch<LAYOUT, 2>(grid, lds, a, b, sfa, sfb, c, p, st);
}

template <int LAYOUT>
hipError_t mf_launch(int64_t grid, const void *a, const void *b, const void *sfa, const void *sfb, void *c,
                     const MfParams &p, hipStream_t st)
{
    hipLaunchKernelGGL((nvfp4_gemm_small_n_mfma_kernel<LAYOUT>), dim3((uint32_t)grid), dim3(kMfThreads), 0, st,
                       (const uint8_t *)a, (const uint8_t *)b, (const uint8_t *)sfa, (const uint8_t *)sfb,
                       (uint16_t *)c, p);
    return hipGetLastError();
}

// Whether a matrix-core kernel runs: from N = 3 always; N = 2 with blocked
// scales where the staged kernels get at least kMfMinGrid2 workgroups and K is
// at least kMfMinK2. The MFMA's cost does not depend on N: for N = 2 it ran
// 15.6 us on the headline A and 28.8 on the batched A, against 19.0 and 38.3
// through the two-vector GEMV kernel; with short rows (7168x2048x4: 12.2
// against 9.8) or few workgroups the GEMV's plan uses the chip better.
constexpr int64_t kMfMinGrid2 = 128;
constexpr int64_t kMfMinK2 = 4096;
bool mf_runs(int64_t M, int64_t N, int64_t K, int64_t L, int sf_layout)
{
    if (N >= kMfMinN)
        return true;
    return N == 2 && sf_layout == NVFP4_SF_BLOCKED && K >= kMfMinK2 &&
           L * ((M + 127) / 128) * kMsWgPerBlock >= kMfMinGrid2;
}

// The streamed kernel's dynamic LDS bytes (three slots), or -1 where it does
// not run: plain scales, no matrix-core kernel, or more workgroups than a
// grid holds.
int64_t ms_lds_bytes(int64_t M, int64_t N, int64_t K, int64_t L, int sf_layout)
{
    if (sf_layout != NVFP4_SF_BLOCKED || !mf_runs(M, N, K, L, sf_layout) || N > kSnMaxN ||
        L * ((M + 127) / 128) * kMsWgPerBlock > INT32_MAX)
        return -1;
    return (int64_t)kMsSlots * (N <= 4 ? MsSlot<4>::kBytes : MsSlot<8>::kBytes);
}

hipError_t ms_launch(int64_t grid, int64_t lds, const void *a, const void *b, const void *sfa, const void *sfb,
                     void *c, const MfParams &p, hipStream_t st)
{
    if (p.N <= 4)
        hipLaunchKernelGGL(nvfp4_gemm_small_n_mfma_staged_kernel<4>, dim3((uint32_t)grid), dim3(kMsThreads),
                           (uint32_t)lds, st, (const uint8_t *)a, (const uint8_t *)b, (const uint8_t *)sfa,
                           (const uint8_t *)sfb, (uint32_t)p.L, p.M, p.K, p.N, (uint16_t *)c, p);
    else
        hipLaunchKernelGGL(nvfp4_gemm_small_n_mfma_staged_kernel<8>, dim3((uint32_t)grid), dim3(kMsThreads),
                           (uint32_t)lds, st, (const uint8_t *)a, (const uint8_t *)b, (const uint8_t *)sfa,
                           (const uint8_t *)sfb, (uint32_t)p.L, p.M, p.K, p.N, (uint16_t *)c, p);
    return hipGetLastError();
}

// The up-front kernel's LDS bytes for (M, N, K, L), or -1 where it does not
// apply: N >= 2, LDS within the limit, each wave's copies within what the
// wait counter holds next to the ring, at most 256 4-block groups (K <= 16384).
int64_t mu_lds_bytes(int64_t M, int64_t N, int64_t K, int64_t L)
{
    if (N < 2 || N > kSnMaxN)
        return -1;
    const MuLayout o = mu_layout((int32_t)K, (int32_t)N);
    const int64_t bytes = (int64_t)o.b_bytes + o.sfa_bytes + o.sfb_bytes;
    const int64_t ncb = (K / 16 + 3) / 4;
    if (bytes > kMuLdsLimit ||
        N * ((o.n_dma_b + kMfWaves - 1) / kMfWaves) + (o.n_dma_sfa + kMfWaves - 1) / kMfWaves +
                N * ((o.n_dma_sfb + kMfWaves - 1) / kMfWaves) > kMuMaxDmaPerWave ||
        ncb > kMuMaxNcb || L * ((M + 127) / 128) * kMsWgPerBlock > INT32_MAX)
        return -1;
    return bytes;
}

hipError_t mu_launch(int64_t grid, int64_t lds, const void *a, const void *b, const void *sfa, const void *sfb,
                     void *c, const MfParams &p, hipStream_t st)
{
    hipLaunchKernelGGL(nvfp4_gemm_small_n_mfma_upfront_kernel, dim3((uint32_t)grid), dim3(kMfThreads),
                       (uint32_t)lds, st, (const uint8_t *)a, (const uint8_t *)b, (const uint8_t *)sfa,
                       (const uint8_t *)sfb, (uint32_t)p.L, p.M, p.K, p.N, (uint16_t *)c, p);
    return hipGetLastError();
}

// Which matrix-core kernel runs (N >= 3), and its dynamic LDS bytes. Blocked
// scales: with more than 256 workgroups (several per CU) the up-front staged
// kernel where all of K fits in LDS, else the streamed one. Plain scales: the
// unstaged kernel.
enum class MfKind { Unstaged, Upfront, Streamed };
MfKind mf_select(int64_t M, int64_t N, int64_t K, int64_t L, int sf_layout, int64_t *lds)
{
    const int64_t streamed = ms_lds_bytes(M, N, K, L, sf_layout);
    if (streamed < 0) {
        *lds = 0;
        return MfKind::Unstaged;
    }
    const int64_t grid = L * ((M + 127) / 128) * kMsWgPerBlock;
    const int64_t upfront = mu_lds_bytes(M, N, K, L);
    if (grid > 256 && upfront >= 0) {
        *lds = upfront;
        return MfKind::Upfront;
    }
    *lds = streamed;
    return MfKind::Streamed;
}

bool sn_aligned(const void *q, uintptr_t a) { return ((uintptr_t)q & (a - 1)) == 0; }

} // namespace

extern "C" {

nvfp4_status_t nvfp4_gemm_small_n_plan(int64_t M, int64_t N, int64_t K, int64_t L, int sf_layout,
                                       int32_t *rows_per_wg, int64_t *workgroups, int32_t *lds_bytes)
{
    if (M < 1 || N < 1 || N > kSnMaxN || L < 1 || K < 32 || K % 32 != 0 || K > (INT64_C(1) << 22) ||
        M > INT32_MAX / 2 || L > INT32_MAX / 2 || L * M > (INT64_C(1) << 62) / K)
        return NVFP4_ERR_INVALID_SHAPE;
    if (sf_layout != NVFP4_SF_PLAIN && sf_layout != NVFP4_SF_BLOCKED)
        return NVFP4_ERR_INVALID_LAYOUT;
    int64_t mf_lds = 0;
    if (mf_runs(M, N, K, L, sf_layout) && mf_select(M, N, K, L, sf_layout, &mf_lds) != MfKind::Unstaged) {
        // a staged matrix-core kernel: 4 workgroups of 32 rows per 128-row block
        if (rows_per_wg)
            *rows_per_wg = (int32_t)std::min<int64_t>(32, M);
        if (workgroups)
            *workgroups = L * ((M + 127) / 128) * kMsWgPerBlock;
        if (lds_bytes)
            *lds_bytes = (int32_t)mf_lds;
        return NVFP4_OK;
    }
    if (N >= kMfMinN) {
        // the matrix-core kernel: one workgroup per kMfRT tiles of 16 rows, static LDS only
        const int64_t rows = 16 * kMfRT, P = (M + rows - 1) / rows;
        if (L * P > INT32_MAX)
            return NVFP4_ERR_INVALID_SHAPE;
        if (rows_per_wg)
            *rows_per_wg = (int32_t)std::min<int64_t>(rows, M);
        if (workgroups)
            *workgroups = L * P;
        if (lds_bytes)
            *lds_bytes = 0;
        return NVFP4_OK;
    }
    // about the target number of workgroups, each a contiguous row range of one batch,
    // with the per-wave row sums inside the LDS budget
    const int64_t rmax = kSnPartBudget / (N * kSnWaves * (int64_t)sizeof(float));
    const int64_t target = kSnTargetWGs;
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
    nvfp4_status_t st = nvfp4_gemm_small_n_plan(M, N, K, L, sf_layout, &R, &grid, &lds);
    if (st != NVFP4_OK)
        return st;
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
    // Two vectors: the GEMV kernel with b' of both in registers, where it
    // needs no K-split and no matrix-core kernel runs.
    if (N == 2 && !mf_runs(M, N, K, L, sf_layout) && nvfp4_gemv_workspace_bytes(M, K, L) == 0) {
        const nvfp4_status_t st2 = nvfp4_gemv_two_vectors(a, b, sfa, sfb, c, M, K, L, sf_layout, alpha, stream);
        if (st2 != NVFP4_ERR_INVALID_SHAPE)
            return st2;
    }
    const int64_t nkb = K / 16, ncb = (nkb + 3) / 4;
    const int64_t sfa_batch = sf_layout == NVFP4_SF_PLAIN ? M * nkb : ((M + 127) / 128) * ncb * 512;
    const int64_t sfb_batch = sf_layout == NVFP4_SF_PLAIN ? N * nkb : ((N + 127) / 128) * ncb * 512;
    hipError_t e;
    if (mf_runs(M, N, K, L, sf_layout)) {
        MfParams q{};
        q.M = (int32_t)M;
        q.K = (int32_t)K;
        q.L = (int32_t)L;
        q.N = (int32_t)N;
        q.P = (int32_t)(grid / L);
        q.sfa_batch = sfa_batch;
        q.sfb_batch = sfb_batch;
        q.alpha = alpha;
        int64_t mf_lds = 0;
        switch (mf_select(M, N, K, L, sf_layout, &mf_lds)) {
        case MfKind::Streamed:
            e = ms_launch(grid, mf_lds, a, b, sfa, sfb, c, q, (hipStream_t)stream);
            break;
        case MfKind::Upfront:
            e = mu_launch(grid, mf_lds, a, b, sfa, sfb, c, q, (hipStream_t)stream);
            break;
        default:                                                       // plain scales
            e = sf_layout == NVFP4_SF_PLAIN
                    ? mf_launch<NVFP4_SF_PLAIN>(grid, a, b, sfa, sfb, c, q, (hipStream_t)stream)
                    : mf_launch<NVFP4_SF_BLOCKED>(grid, a, b, sfa, sfb, c, q, (hipStream_t)stream);
            break;
        }
    } else {
        SnParams p{};
        p.M = (int32_t)M;
        p.K = (int32_t)K;
        p.L = (int32_t)L;
        p.R = R;
        p.P = (int32_t)(grid / L);
        p.alpha = alpha;
        p.sfa_batch = sfa_batch;
        p.sfb_batch = sfb_batch;
        e = sf_layout == NVFP4_SF_PLAIN
                ? sn_dispatch<NVFP4_SF_PLAIN>(N, grid, lds, a, b, sfa, sfb, c, p, (hipStream_t)stream)
                : sn_dispatch<NVFP4_SF_BLOCKED>(N, grid, lds, a, b, sfa, sfb, c, p, (hipStream_t)stream);
    }
    if (e != hipSuccess) {
        nvfp4_record_hip_error((int)e);
        return NVFP4_ERR_HIP;
    }
    return NVFP4_OK;
}

} // extern "C"
