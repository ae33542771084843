/*
 * nvfp4_gemv.h -- C ABI of the MI355X (gfx950) NVFP4 block-scaled batched GEMV.
 *
 * Operation (kernelbot NVFP4 GEMV, submission 103289, `cute_kernel`: each k
 * contributes a * sfa * b * sfb, the contributions of one output row are
 * accumulated in float32 and the sum is cast to float16):
 *
 *   c[l][m] = fp16( sum_{k<K} e2m1(A[l][m][k]) * e4m3(SFA[l][m][k/16])
 *                            * e2m1(B[l][k])    * e4m3(SFB[l][k/16]) )
 *
 * for m < M, l < L (N = 1). Element format: E2M1 (Float4E2M1FN), packed two per
 * byte along k, the even k in the low nibble. Scale format: E4M3 (Float8E4M3FN),
 * one scale per 16 consecutive k. Accumulation is float32; the cast to float16
 * rounds to nearest even and overflows to +-inf. Summation order inside a row
 * is the library's own (all products are exact; partial sums round in float32),
 * and it does not depend on the scale layout.
 *
 * Memory order of every operand is batch-outermost and dense (the CuTe layouts
 * of submission 103289 `cute_jit_kernel`: A stride (K, 1, M*K), C stride
 * (1, 1, M)):
 *
 *   a    uint8  [L][M][K/2]     packed E2M1 codes of A
 *   b    uint8  [L][K/2]        packed E2M1 codes of the vector B
 *   c    fp16   [L][M]          output (IEEE binary16 bits), written
 *   sfa, sfb in one of two layouts, chosen by sf_layout for both:
 *     NVFP4_SF_PLAIN:   sfa uint8 [L][M][K/16], sfb uint8 [L][K/16]
 *     NVFP4_SF_BLOCKED: the 128x4 blocked ("permuted") layout of submission
 *       69953 `to_blocked_batch` (equivalently submission 69575
 *       `blocked_transform_kernel`, and the 6-D tensor of submission 103289
 *       `permuted_to_blocked`), per batch, batches back to back:
 *         scale (r, kb) of a rows x (K/16) matrix is at byte
 *           ((r/128)*ceil(K/64) + kb/4)*512 + (r%32)*16 + ((r%128)/32)*4 + kb%4
 *         sfa: rows = M, ceil(M/128)*ceil(K/64)*512 bytes per batch
 *         sfb: rows = 1, ceil(K/64)*512 bytes per batch (B padded to 128 rows)
 *       Padding bytes (rows >= M, columns >= K/16) are never read.
 *
 * Conventions shared by all entry points:
 *   - a, b, sfa, sfb, c and workspace are DEVICE pointers owned by the caller;
 *     the library keeps no reference to them after the call returns.
 *   - Calls only enqueue work on `stream` (a hipStream_t; NULL = the null
 *     stream) and never synchronise. Faults inside the kernel surface later on
 *     the stream.
 *   - Every argument is validated before any HIP call; on failure nothing is
 *     launched and a nonzero nvfp4_status_t is returned.
 *   - Requirements: M, K, L >= 1; K % 32 == 0; L*M*K/2 < 2^62; a, b and sfa
 *     16-byte aligned; sfb 4-byte aligned; c 2-byte aligned.
 */
#ifndef NVFP4_GEMV_H
#define NVFP4_GEMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    NVFP4_SF_PLAIN = 0,
    NVFP4_SF_BLOCKED = 1
} nvfp4_sf_layout_t;

typedef enum {
    NVFP4_OK = 0,
    NVFP4_ERR_NULL_POINTER = 1,     /* a required pointer is NULL                 */
    NVFP4_ERR_INVALID_SHAPE = 2,    /* M, K or L out of range, or K % 32 != 0      */
    NVFP4_ERR_MISALIGNED = 3,       /* a pointer misses its required alignment     */
    NVFP4_ERR_INVALID_LAYOUT = 4,   /* sf_layout is not an nvfp4_sf_layout_t       */
    NVFP4_ERR_WORKSPACE = 5,        /* workspace missing, misaligned or too small  */
    NVFP4_ERR_HIP = 6,              /* a HIP call failed; see nvfp4_last_hip_error */
    NVFP4_ERR_INVALID_SCALE = 7,    /* the global scale alpha is NaN or infinite   */
    NVFP4_ERR_INVALID_STRIDE = 8    /* an operand stride is out of range or misaligned */
} nvfp4_status_t;

/*
 * Batched GEMV as defined above. If the problem is split along K (small M*L),
 * float32 partial sums go to a workspace that the library allocates on first
 * need, per device, grows on demand (with a device synchronisation) and keeps
 * until the process ends. Calls that overlap in time on one device therefore
 * must not use this entry point concurrently from two streams; use
 * nvfp4_gemv_ex with separate workspaces instead. Under HIP graph capture:
 * make the first call of the largest split shape eagerly, before capturing
 * (allocation is not capturable), and note that a captured graph keeps the
 * workspace address, which a later call needing a larger workspace frees;
 * nvfp4_gemv_ex with a caller-owned workspace, or nvfp4_gemv_noalloc, has
 * neither concern.
 */
nvfp4_status_t nvfp4_gemv(const void *a, const void *b, const void *sfa, const void *sfb,
                          void *c, int64_t M, int64_t K, int64_t L, int sf_layout,
                          void *stream);

/*
 * As nvfp4_gemv, for callers that cannot allocate: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation. It calls no
 * hipMalloc, hipFree or allocating routine. The split-K workspace comes from a
 * fixed scratch array of nvfp4_gemv_noalloc_scratch_bytes() bytes that the
 * library holds in device memory, one copy per GPU it runs on, until the
 * process ends. The first call on a device looks up that copy's address and
 * enqueues one small kernel on `stream` that zeroes its ticket region; every
 * completed call leaves the tickets zero again. All calls on one GPU share its
 * copy, so calls that overlap in time on one GPU (two streams, or two host
 * threads) race and must not be made. A shape whose workspace
 * (nvfp4_gemv_workspace_bytes) exceeds the array returns NVFP4_ERR_WORKSPACE
 * with nothing launched; the library's own plans split K only for small M*L,
 * whose workspace stays far below it.
 */
nvfp4_status_t nvfp4_gemv_noalloc(const void *a, const void *b, const void *sfa, const void *sfb,
                                  void *c, int64_t M, int64_t K, int64_t L, int sf_layout,
                                  void *stream);

/* Bytes of nvfp4_gemv_noalloc's fixed scratch array (the workspace limit). */
size_t nvfp4_gemv_noalloc_scratch_bytes(void);

/*
 * Workspace bytes nvfp4_gemv_ex needs for this shape (0 when the shape is not
 * split along K). The value depends only on M, K and L.
 */
size_t nvfp4_gemv_workspace_bytes(int64_t M, int64_t K, int64_t L);

/*
 * As nvfp4_gemv, with a caller-owned device workspace of at least
 * nvfp4_gemv_workspace_bytes(M, K, L) bytes, 256-byte aligned (may be NULL
 * when that size is 0). The workspace must be zero-filled before its first use;
 * every completed call leaves its counter region zero again, so it can be reused
 * for any later shape without clearing. Two calls may share a workspace only
 * if they are ordered on one stream.
 */
nvfp4_status_t nvfp4_gemv_ex(const void *a, const void *b, const void *sfa, const void *sfb,
                             void *c, int64_t M, int64_t K, int64_t L, int sf_layout,
                             void *workspace, size_t workspace_bytes, void *stream);

/*
 * Batched GEMV with NVFP4's second scaling level: one float32 scale per tensor
 * pair on top of the per-16-element E4M3 scales (the "dual scaling" that
 * kernelbot NVFP4 GEMV submission 69575 lists among its notes on the format;
 * none of the pages' kernels applies it, so its placement is this library's
 * reading: it multiplies the finished float32 row sum once, before the cast):
 *
 *   c[l][m] = fp16( alpha * sum_{k<K} e2m1(A) * e4m3(SFA) * e2m1(B) * e4m3(SFB) )
 *
 * A caller whose A and B carry global scales ga and gb passes alpha = ga * gb.
 * alpha must be finite (else NVFP4_ERR_INVALID_SCALE, nothing launched); with
 * alpha = 1 the result is bit-identical to nvfp4_gemv. The product alpha * sum
 * is rounded to float32 and then to float16 (two roundings, within the
 * library's float32-accumulation error). Layouts, alignment and the other
 * arguments are as for nvfp4_gemv.
 * Workspace: NULL with workspace_bytes = 0 uses the library-owned workspace as
 * nvfp4_gemv does; otherwise it is a caller-owned workspace with the
 * requirements of nvfp4_gemv_ex (NVFP4_ERR_WORKSPACE if too small or
 * misaligned when the shape needs one).
 */
nvfp4_status_t nvfp4_gemv_scaled(const void *a, const void *b, const void *sfa, const void *sfb,
                                 void *c, int64_t M, int64_t K, int64_t L, int sf_layout,
                                 float alpha, void *workspace, size_t workspace_bytes,
                                 void *stream);

/*
 * Operand strides, for callers whose tensors are not densely packed (the
 * pages' harness, kernelbot NVFP4 GEMV submission 103289, hands B over with
 * its N dimension padded to 128 rows, so B's batch stride is 128*K/2 bytes;
 * submission 69575 reads plain scales through arbitrary row and batch
 * strides). Inside a row everything stays contiguous. Byte strides except
 * c_batch, which counts float16 elements:
 *   a_row      between rows m, m+1 of A        >= K/2, multiple of 16
 *   a_batch    between batches of A            >= 0,   multiple of 16
 *   b_batch    between batches of B            >= 0,   multiple of 16
 *   sfa_row    between rows of SFA (plain layout only; ignored for blocked,
 *              whose tiles fix it)             >= K/16, even
 *   sfa_batch  between batches of SFA          >= 0, even (plain) / multiple of 16 (blocked)
 *   sfb_batch  between batches of SFB          >= 0, even (plain) / multiple of 16 (blocked)
 *   c_batch    between batches of C, elements  >= M when L > 1 (outputs must not overlap)
 * A batch stride of 0 broadcasts one input to every batch. All strides are
 * below 2^40, and the rows of A that one workgroup reads must lie within 2^31
 * bytes: (ceil(rows_per_wg/128) + 1) * 128 * a_row + K/2 < 2^31, with
 * rows_per_wg from nvfp4_gemv_plan (about a_row <= 2^21 for any shape).
 */
typedef struct {
    int64_t a_row, a_batch;
    int64_t b_batch;
    int64_t sfa_row, sfa_batch;
    int64_t sfb_batch;
    int64_t c_batch;
} nvfp4_strides_t;

/* The dense strides of the layouts above (what nvfp4_gemv assumes). */
void nvfp4_gemv_dense_strides(int64_t M, int64_t K, int64_t L, int sf_layout,
                              nvfp4_strides_t *strides);

/*
 * nvfp4_gemv_scaled with operand strides (`strides` must not be NULL):
 * pointers, alignment, alpha and workspace as for nvfp4_gemv_scaled;
 * NVFP4_ERR_INVALID_STRIDE, nothing launched, for strides outside the rules
 * above. Results are bit-identical to the dense call on the same values.
 */
nvfp4_status_t nvfp4_gemv_strided(const void *a, const void *b, const void *sfa, const void *sfb,
                                  void *c, int64_t M, int64_t K, int64_t L, int sf_layout,
                                  const nvfp4_strides_t *strides, float alpha, void *workspace,
                                  size_t workspace_bytes, void *stream);

/*
 * Launch plan chosen for a shape (for tests and reports). Returns NVFP4_OK and
 * fills the fields, or an error status for an invalid shape.
 *   lanes_per_row  lanes that share one output row (1..256)
 *   rows_per_wg    output rows per workgroup (at most; 4 per 16-byte scale slot)
 *   k_splits       number of K-slices (1 = no split)
 *   k_per_split    K-elements per slice
 *   workgroups     grid size; threads_per_wg threads each (the first 64 of
 *                  them stage the scales, the others compute)
 *   lds_bytes      dynamic LDS per workgroup
 */
typedef struct {
    int32_t lanes_per_row;
    int32_t rows_per_wg;
    int32_t k_splits;
    int32_t k_per_split;
    int64_t workgroups;
    int32_t threads_per_wg;
    int32_t lds_bytes;
} nvfp4_plan_t;

nvfp4_status_t nvfp4_gemv_plan(int64_t M, int64_t K, int64_t L, nvfp4_plan_t *plan);

/*
 * Launch plan of the GEMV kernel with two right-hand vectors, which
 * nvfp4_gemm_small_n runs for N = 2 where no matrix-core kernel applies and
 * the GEMV's plan needs no K-split (for tests and reports; fields as for
 * nvfp4_gemv_plan). NVFP4_ERR_INVALID_SHAPE where that kernel does not run.
 */
nvfp4_status_t nvfp4_gemv_two_vectors_plan(int64_t M, int64_t K, int64_t L, nvfp4_plan_t *plan);

/*
 * Block-scaled skinny GEMM with N = 1..8 right-hand vectors (the general
 * product kernelbot NVFP4 GEMV submission 103289 hands to torch._scaled_mm,
 * a @ b^T with block scales and a float16 result; the GEMV is N = 1):
 *
 *   c[l][n][m] = fp16( alpha * sum_{k<K} e2m1(A[l][m][k]) * e4m3(SFA[l][m][k/16])
 *                                      * e2m1(B[l][n][k]) * e4m3(SFB[l][n][k/16]) )
 *
 *   a    uint8 [L][M][K/2]      as for nvfp4_gemv
 *   b    uint8 [L][N][K/2]      N packed vectors per batch
 *   sfa  as for nvfp4_gemv (layout sf_layout)
 *   sfb  plain uint8 [L][N][K/16]; blocked: the 128x4 layout of the N x K/16
 *        matrix (rows padded to 128), ceil(K/64)*512 bytes per batch
 *   c    fp16 [L][N][M]          written (column n of batch l contiguous)
 * Requirements and alignment as for nvfp4_gemv, 1 <= N <= 8, alpha finite.
 * Accumulation is float32 per row and vector (summation order the library's
 * own); no K-split and no workspace: small M*L leaves the GPU partly idle.
 * N = 1 runs the GEMV kernel (nvfp4_gemv_scaled), and N = 2 the GEMV kernel
 * with two vectors, whenever the GEMV's plan needs no split-K workspace; else
 * a dot-product kernel. From N = 3 a matrix-core kernel runs (and for N = 2
 * with blocked scales, K >= 4096 and at least 128 of its workgroups): a' =
 * e2m1 * e4m3 and b' are exact in float16, so the product is a float16 MFMA
 * with float32 accumulation. Either way nothing is allocated.
 */
nvfp4_status_t nvfp4_gemm_small_n(const void *a, const void *b, const void *sfa, const void *sfb,
                                  void *c, int64_t M, int64_t N, int64_t K, int64_t L, int sf_layout,
                                  float alpha, void *stream);

/* Launch plan of nvfp4_gemm_small_n's own kernels for a shape and scale
 * layout: rows per workgroup, workgroups and dynamic LDS bytes (for N = 1 or
 * 2 where the GEMV's kernel runs instead, the plan of the dot-product kernel
 * that would run otherwise). The matrix-core kernels (N >= 3, and N = 2 on
 * large blocked shapes) give each workgroup 32 rows, 4 workgroups per 128-row
 * block. With blocked scales they stage B, the SFB dwords and the workgroup's
 * SFA lines in LDS: grids of more than 256 workgroups stage all of K at once
 * where that fits in 150 KiB (about (3N/4 + 2) * K bytes; 256 threads per
 * workgroup), other grids stream K through three slots of 32 K-steps (52 KiB
 * for N <= 4, 78 KiB up to N = 8; 320 threads per workgroup). Plain scales:
 * no LDS. Any output pointer may be NULL. Returns NVFP4_ERR_INVALID_SHAPE for
 * shapes it does not take, NVFP4_ERR_INVALID_LAYOUT for an unknown layout. */
nvfp4_status_t nvfp4_gemm_small_n_plan(int64_t M, int64_t N, int64_t K, int64_t L, int sf_layout,
                                       int32_t *rows_per_wg, int64_t *workgroups, int32_t *lds_bytes);

/*
 * Device-side reblocking of plain scale factors into the 128x4 blocked layout
 * (the transformation kernelbot NVFP4 GEMV submission 69953 performs with
 * `to_blocked_batch` and submission 69575 with `blocked_transform_kernel`,
 * here as one HIP kernel for all batches), so that callers holding plain
 * scales can produce what nvfp4_gemv reads with sf_layout = NVFP4_SF_BLOCKED.
 *
 *   plain    uint8 [L][rows][K/16] E4M3 codes (rows = M for SFA, 1 for SFB)
 *   blocked  uint8, nvfp4_blocked_scales_bytes(rows, K, L) bytes, written:
 *            per batch ceil(rows/128)*ceil(K/64)*512 bytes, scale (r, kb) at
 *            ((r/128)*ceil(K/64) + kb/4)*512 + (r%32)*16 + ((r%128)/32)*4 + kb%4;
 *            padding bytes (r >= rows or kb >= K/16) are written as 0.
 * Both are DEVICE pointers owned by the caller; blocked must be 16-byte
 * aligned (plain has no alignment requirement) and the two must not overlap.
 * Requirements: rows, L >= 1; K >= 32, K % 32 == 0. Errors are reported before
 * any HIP call (nothing launched); the call only enqueues work on `stream`.
 */
nvfp4_status_t nvfp4_scales_to_blocked(const void *plain, void *blocked, int64_t rows, int64_t K,
                                       int64_t L, void *stream);

/* Bytes of the blocked layout for (rows, K, L); 0 for an invalid shape. */
size_t nvfp4_blocked_scales_bytes(int64_t rows, int64_t K, int64_t L);

/* Static description of a status code (never NULL). */
const char *nvfp4_status_string(int status);

/* The hipError_t of the last failed HIP call in this thread (0 if none). */
int nvfp4_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_GEMV_H */
