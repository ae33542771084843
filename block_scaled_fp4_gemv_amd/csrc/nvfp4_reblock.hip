// Plain -> 128x4 blocked reblocking of NVFP4 scale factors on MI355X (gfx950).
//
// The blocked ("permuted") layout is the one kernelbot NVFP4 GEMV submission
// 69953 builds with `to_blocked_batch` and submission 69575 with
// `blocked_transform_kernel`: a rows x cols matrix of E4M3 codes (cols = K/16)
// is cut into 128x4 tiles, tile (rb, cb) is stored as 512 contiguous bytes at
// (rb * ceil(cols/4) + cb) * 512, and inside a tile scale (r, c) sits at
// (r % 32) * 16 + (r / 32) * 4 + c. So each 16-byte line of a tile holds the
// 4 scales of rows r, r+32, r+64, r+96. Padding (rows >= rows, columns >=
// cols) is written as zero bytes.
//
// Work split. A workgroup of 256 threads owns one batch, one 128-row block
// and TILES consecutive tiles of it (16 or 32). Workgroup ids are remapped so that
// each XCD takes a contiguous range: with 16 tiles, the two workgroups that
// read the halves of a row's 128-byte lines then share one L2 and each line is fetched once
// (with ids dealt round-robin over the XCDs, every line was fetched twice). It reads the 128 rows x 4*TILES
// plain bytes row by row (consecutive threads take consecutive 16-byte units,
// or words, of a row, so the reads are contiguous 64- or 128-byte runs of each row;
// 16-byte loads where the rows allow them: 1.45x faster than words),
// parks them in LDS, and writes the tiles as contiguous 16-byte lines
// (consecutive threads write consecutive lines).
// The kernel is a byte shuffle: it is bound by HBM, with read bytes = the
// plain scales and write bytes = the blocked scales (padding included).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "nvfp4_gemv.h"
#include "nvfp4_internal.h"

namespace {

typedef uint32_t uint4_t __attribute__((ext_vector_type(4)));

constexpr int kRbThreads = 256;
// Tiles per workgroup (TILES, one 4-byte word per tile and row, 4*TILES scale
// columns): 32 where that still gives the chip a full grid with little
// padding (the headline SFA: 4.8 -> 4.1 us, whole 128-byte lines per row and
// twice the loads in flight per thread), else 16 (fewer tiles per block row:
// 32 left half the CUs idle on 7168x2048x4, 2.57 -> 2.82 us).
constexpr int kTilesSmall = 16, kTilesLarge = 32;
constexpr int64_t kLargeMinGrid = 256;          // workgroups the 32-tile grid must reach

struct ReblockParams {                          // the host's launch plan
    int32_t rows, cols;                         // plain matrix per batch (cols = K/16)
    int32_t nrb, ncb;                           // 128-row blocks, 4-column groups
    int32_t wg_per_rb;                          // workgroups per row block
};

// Read modes: bytes (any alignment), 4-byte words (row starts 4-byte
// aligned), 16-byte units (row starts 16-byte aligned, cols % 16 == 0).
enum { kReadBytes = 0, kReadWords = 1, kReadVec16 = 2 };

// 4 plain bytes of row r, columns 4*cb .. 4*cb+3 (zero past the matrix),
// little-endian in a word. WORDS: the row starts are 4-byte aligned.
template <bool WORDS>
__device__ inline uint32_t load_word(const uint8_t *__restrict__ in, int32_t rows, int32_t cols, int32_t r, int32_t cb)
{
    if (r >= rows || 4 * cb >= cols)
        return 0u;
    const uint8_t *src = in + (int64_t)r * cols + 4 * cb;
    if (WORDS && 4 * cb + 4 <= cols)
        return *(const uint32_t *)src;
    uint32_t w = 0;
    const int32_t n = min(4, cols - 4 * cb);
    for (int32_t i = 0; i < n; ++i)
        w |= (uint32_t)src[i] << (8 * i);
    return w;
}

// The arguments are the kernel's only inputs, all of them scalars the build
// preloads into SGPRs (the leading kernel arguments): the first loads wait for
// no kernel-argument read. Per batch: rows x cols plain bytes in, nrb x ncb
// tiles of 512 bytes out.
template <int MODE, int TILES>
__global__ __launch_bounds__(kRbThreads) void nvfp4_reblock_kernel(const uint8_t *__restrict__ plain,
                                                                  uint8_t *__restrict__ blocked, uint32_t n_wg,
                                                                  int32_t rows, int32_t cols, int32_t nrb,
                                                                  int32_t ncb, int32_t wg_per_rb)
{
    constexpr int kWordsPerRow = TILES;                    // one 4-byte word per tile and row
    constexpr int kLdsPitch = kWordsPerRow + 1;            // words; odd pitch avoids bank conflicts
    __shared__ uint32_t tile_words[128 * kLdsPitch];
    const int32_t t = threadIdx.x;
    // contiguous ids per XCD (hardware id i runs on XCD i % 8), so that the
    // workgroups sharing a row's 128-byte lines share an L2
    const uint32_t n = n_wg, x = blockIdx.x % 8, j = blockIdx.x / 8;
    const uint32_t lid = x * (n / 8) + min(x, n % 8) + j;
    const int32_t wg = lid % (uint32_t)wg_per_rb;
    const uint32_t rbl = lid / (uint32_t)wg_per_rb;        // batch * nrb + row block
    const int32_t l = (int32_t)(rbl / (uint32_t)nrb), rb = (int32_t)(rbl % (uint32_t)nrb);
    const int32_t cb0 = wg * TILES;
    const uint8_t *in = plain + (int64_t)l * rows * cols;
    uint8_t *out = blocked + (int64_t)l * nrb * ncb * 512;

    // read: 128 rows x kWordsPerRow words, in units of UW words (one load each)
    constexpr int UW = MODE == kReadVec16 ? 4 : 1;
    constexpr int UPR = kWordsPerRow / UW;                 // units per row
    constexpr int NU = 128 * UPR / kRbThreads;             // units per thread
    if constexpr (MODE == kReadVec16) {
        // every load first, then the LDS writes: one memory round trip (with
        // the writes between them the compiler waited for each load in turn).
        // cols % 16 == 0: a unit is wholly inside the row or wholly past it;
        // units past the matrix load a real unit (clamped) and write zeros.
        uint4_t v[NU];
        bool in_mat[NU];
#pragma unroll
        for (int i = 0; i < NU; ++i) {
            const int32_t e = t + i * kRbThreads;
            const int32_t row = e / UPR, u = e % UPR;
            const int32_t r = rb * 128 + row, cb = cb0 + u * UW;
            in_mat[i] = r < rows && 4 * cb < cols;
            v[i] = *(const uint4_t *)(in + (int64_t)min(r, rows - 1) * cols + 4 * min(cb, cols / 4 - 4));
        }
#pragma unroll
        for (int i = 0; i < NU; ++i) {
            const int32_t e = t + i * kRbThreads;
            const int32_t row = e / UPR, u = e % UPR;
            const uint4_t w = in_mat[i] ? v[i] : (uint4_t){0u, 0u, 0u, 0u};
            uint32_t *dst = &tile_words[row * kLdsPitch + u * 4];
            dst[0] = w.x;
            dst[1] = w.y;
            dst[2] = w.z;
            dst[3] = w.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < NU; ++i) {
            const int32_t e = t + i * kRbThreads;
            const int32_t row = e / UPR, u = e % UPR;
            tile_words[row * kLdsPitch + u] = load_word<MODE == kReadWords>(in, rows, cols, rb * 128 + row, cb0 + u * UW);
        }
    }
    __syncthreads();
    // write: TILES tiles of 32 lines; line (tile, r32) = rows r32 + 32*i4
#pragma unroll
    for (int i = 0; i < TILES * 32 / kRbThreads; ++i) {
        const int32_t e = t + i * kRbThreads;
        const int32_t tl = e / 32, r32 = e % 32;
        if (cb0 + tl < ncb) {
            uint4_t v;
            v.x = tile_words[(r32 + 0) * kLdsPitch + tl];
            v.y = tile_words[(r32 + 32) * kLdsPitch + tl];
            v.z = tile_words[(r32 + 64) * kLdsPitch + tl];
            v.w = tile_words[(r32 + 96) * kLdsPitch + tl];
            // written once and not read back here: non-temporal (measured
            // 4-13% faster than plain stores; non-temporal loads were slower)
            __builtin_nontemporal_store(v, (uint4_t *)(out + ((int64_t)rb * ncb + cb0 + tl) * 512 + r32 * 16));
        }
    }
}

} // namespace

extern "C" {

size_t nvfp4_blocked_scales_bytes(int64_t rows, int64_t K, int64_t L)
{
    if (rows < 1 || K < 32 || K % 32 != 0 || L < 1 || rows > INT32_MAX / 2 || K / 16 > INT32_MAX / 2)
        return 0;
    const int64_t nrb = (rows + 127) / 128, ncb = (K / 16 + 3) / 4;
    if (L > (INT64_C(1) << 62) / (nrb * ncb * 512))
        return 0;
    return (size_t)(L * nrb * ncb * 512);
}

nvfp4_status_t nvfp4_scales_to_blocked(const void *plain, void *blocked, int64_t rows, int64_t K,
                                       int64_t L, void *stream)
{
    if (!plain || !blocked)
        return NVFP4_ERR_NULL_POINTER;
    if (nvfp4_blocked_scales_bytes(rows, K, L) == 0)
        return NVFP4_ERR_INVALID_SHAPE;
    if (((uintptr_t)blocked & 15) != 0)
        return NVFP4_ERR_MISALIGNED;
    ReblockParams p{};
    p.rows = (int32_t)rows;
    p.cols = (int32_t)(K / 16);
    p.nrb = (int32_t)((rows + 127) / 128);
    p.ncb = (p.cols + 3) / 4;
    // 32 tiles where that grid fills the chip and pads the last group of a
    // block row by at most an eighth
    const int32_t large = (p.ncb + kTilesLarge - 1) / kTilesLarge;
    const bool big = L * p.nrb * large >= kLargeMinGrid && (int64_t)large * kTilesLarge - p.ncb <= p.ncb / 8;
    const int tiles = big ? kTilesLarge : kTilesSmall;
    p.wg_per_rb = (p.ncb + tiles - 1) / tiles;
    const int64_t grid = L * p.nrb * p.wg_per_rb;
    if (grid > INT32_MAX)
        return NVFP4_ERR_INVALID_SHAPE;
    const bool vec16 = p.cols % 16 == 0 && ((uintptr_t)plain & 15) == 0;
    const bool words = p.cols % 4 == 0 && ((uintptr_t)plain & 3) == 0;
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3((uint32_t)grid), dim3(kRbThreads), 0, (hipStream_t)stream,
                           (const uint8_t *)plain, (uint8_t *)blocked, (uint32_t)grid, p.rows, p.cols, p.nrb, p.ncb,
                           p.wg_per_rb);
    };
    if (vec16)
        big ? go(nvfp4_reblock_kernel<kReadVec16, kTilesLarge>) : go(nvfp4_reblock_kernel<kReadVec16, kTilesSmall>);
    else if (words)
        big ? go(nvfp4_reblock_kernel<kReadWords, kTilesLarge>) : go(nvfp4_reblock_kernel<kReadWords, kTilesSmall>);
    else
        big ? go(nvfp4_reblock_kernel<kReadBytes, kTilesLarge>) : go(nvfp4_reblock_kernel<kReadBytes, kTilesSmall>);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        nvfp4_record_hip_error((int)e);
        return NVFP4_ERR_HIP;
    }
    return NVFP4_OK;
}

} // extern "C"
