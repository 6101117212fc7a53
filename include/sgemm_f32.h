/*
 * sgemm_f32 — FP32 GEMM for AMD Instinct MI355X (gfx950).
 *
 *     C  <-  alpha * A * op(B) + beta * C          row-major, FP32, op(B) in {B, B^T}
 *
 * The operation is the one defined on the pages this library follows:
 *   - "CUDA矩阵乘法性能优化实战：从朴素内核到寄存器分块与Nsight剖析", section 1.1:
 *     C(MxN) = A(MxK) x B(KxN), every C[i][j] a sum of K multiply-adds; section 2.1
 *     gives the row-major element addressing A[row*K+k], B[k*N+col], C[row*N+col].
 *   - Baidu Cloud article comparing the naive and 2-D block-tiled CUDA matmul,
 *     paragraph on the naive mapping: the general form D = alpha*A*B^T + beta*C, in
 *     which C[i][j] is row i of A dotted with row j of B.
 * The result D is written in place into C (one C buffer in the interface).
 *
 * Layout (row-major, leading dimensions in elements):
 *   A      M x K,  element (i,k) at A[i*lda + k],  lda >= max(1, K)
 *   B      transB == 0:  K x N,  op(B)(k,j) = B[k*ldb + j],  ldb >= max(1, N)
 *          transB == 1:  N x K,  op(B)(k,j) = B[j*ldb + k],  ldb >= max(1, K)
 *   C      M x N,  element (i,j) at C[i*ldc + j],  ldc >= max(1, N)
 *
 * Ownership: A, B and C are DEVICE pointers owned by the caller.  The library
 * never allocates, frees, copies or synchronises.  The plain calls use no memory
 * beyond their operands; the workspace calls below take a caller-owned
 * workspace, and sgemm_f32_splitk_noalloc a static array of the library.
 *
 * Asynchrony: a call validates its arguments on the host, enqueues its kernel on
 * `stream` (a hipStream_t; NULL means the null stream) and returns.  Faults inside
 * a kernel surface at the caller's next synchronisation.
 *
 * Quick returns and special values (BLAS conventions; the pages are silent):
 *   - M == 0 or N == 0: nothing is touched, SGEMM_OK.
 *   - alpha == 0 or K == 0: C <- beta*C and A, B are not read
 *     (beta == 1: nothing is touched; beta == 0: C <- 0 without reading C).
 *   - beta == 0: C is not read, so NaN/Inf already in C do not propagate.
 *
 * Accuracy: every element satisfies
 *     |D - D_exact| <= 4*K*2^-24 * sum_k |a(i,k)*b(k,j)| + 1e-6
 * against the exact result, for |alpha| <= 4 and moderate beta*C; the summation
 * order is unspecified and may differ between algorithms.
 *
 * Errors are returned before any HIP call where possible, so they are testable
 * without a GPU:
 *   SGEMM_ERR_INVALID_VALUE   negative or too large (> 2^31 - 1025) dimension, a
 *                             leading dimension below its minimum, transB not 0/1, a
 *                             NULL pointer, or one not on a 4-byte (float) boundary,
 *                             for an operand that would be read or written, an
 *                             unknown algorithm id, or a launch that would need
 *                             2^32 or more work-items;
 *   SGEMM_ERR_ALIAS           C's byte range overlaps A's or B's (the kernels rely on
 *                             the no-alias premise of __restrict__, section 5.3 of the
 *                             first page); A and B may overlap each other;
 *   SGEMM_ERR_NO_DEVICE       no HIP device is current;
 *   SGEMM_ERR_UNSUPPORTED_ARCH the current device is not gfx950 (the code objects
 *                             hold gfx950 code only; compare the "no kernel image"
 *                             case of section 6.2 of the first page);
 *   SGEMM_ERR_LAUNCH          the launch was rejected (hipGetLastError after it).
 *
 * Thread safety: calls are reentrant; the only shared host state is a
 * per-device architecture cache filled once and, for sgemm_f32_splitk_noalloc,
 * a mutex-guarded per-device table of its scratch address (that call's device
 * scratch itself is shared by all its calls on a GPU; see there).
 */
#ifndef SGEMM_F32_H
#define SGEMM_F32_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SGEMM_OK = 0,
    SGEMM_ERR_INVALID_VALUE = 1,
    SGEMM_ERR_ALIAS = 2,
    SGEMM_ERR_NO_DEVICE = 3,
    SGEMM_ERR_UNSUPPORTED_ARCH = 4,
    SGEMM_ERR_LAUNCH = 5,
    SGEMM_ERR_SCRATCH_LIMIT = 6   /* only from sgemm_f32_splitk_noalloc */
} sgemm_status;

/*
 * Algorithms.  Every stage stays available for comparison; all compute the same
 * operation under the same contract.
 *   NAIVE            one work-item per output element, operands read from global
 *                    memory (first page, section 2.1).
 *   LDS_TILED        16x16 output tile per workgroup, A and B tiles staged through
 *                    LDS with a +1 padded row (first page, sections 3.2-3.3; second
 *                    page, section 4.1), zero-filled outside the matrices.
 *   LDS_TILED_NOPAD  the same kernel without the padding column (second page,
 *                    section 3.1); kept to measure LDS bank conflicts against it.
 *   REGBLOCK         128x128 macro tile, 8x8 outputs per work-item held in
 *                    registers (first page, section 5.2), 128-bit global loads
 *                    (section 5.3) and double-buffered LDS staging (second page,
 *                    section 3.2).  Vector FP32 FMA (v_fmac_f32).
 *   MFMA             CDNA matrix-core path: v_mfma_f32_32x32x2_f32, FP32 inputs and
 *                    FP32 accumulation, multi-level tiling (second page, section 7.3).
 *   NAIVE_WG         one 64-lane wavefront per output element: lanes form partial
 *                    dot products over k (k = lane, lane + 64, ...) and a fixed
 *                    cross-lane butterfly adds them (Baidu Cloud article comparing
 *                    the naive and 2-D block-tiled CUDA matmul, paragraph on the
 *                    naive implementation: one block per output element with an
 *                    in-block reduction).
 *   MFMA_256, MFMA_128, MFMA_64, MFMA_32, MFMA_128X64
 *                    the MFMA path with its workgroup tile fixed: 256 x 256 (8
 *                    wavefronts), 128 x 128 (8 wavefronts as two k-slices of 4),
 *                    64 x 64 (4 wavefronts, up to 4 workgroups per CU), 32 x 32
 *                    (4 wavefronts, each a k-slice of a quarter of k; 2 per CU)
 *                    or 128 x 64 (8 wavefronts as two k-slices of 4).
 *   AUTO             MFMA with a tile chosen from the problem shape; where it picks
 *                    the 64 x 64 tile it runs it as 8 wavefronts (two k-slices of
 *                    4, kernel id 45), except: on grids of 257 to 512 such tiles
 *                    with K of at least 256 it takes the 128 x 64 tile (kernel id
 *                    47, as MFMA_128X64: one workgroup per CU) when that tile
 *                    gives at most 256 workgroups and pads at most 1/16 more
 *                    rows, else the 4-wavefront kernel (id 42, as MFMA_64), which
 *                    also runs those grids when K is below 256; and where the
 *                    64 x 64 grid has at most 144 tiles (too few to fill the 256
 *                    CUs) it takes the 32 x 32 tile (kernel id 46, as MFMA_32).
 */
typedef enum {
    SGEMM_ALGO_AUTO = 0,
    SGEMM_ALGO_NAIVE = 1,
    SGEMM_ALGO_LDS_TILED = 2,
    SGEMM_ALGO_REGBLOCK = 3,
    SGEMM_ALGO_MFMA = 4,
    SGEMM_ALGO_LDS_TILED_NOPAD = 5,
    SGEMM_ALGO_NAIVE_WG = 6,
    SGEMM_ALGO_MFMA_256 = 7,
    SGEMM_ALGO_MFMA_128 = 8,
    SGEMM_ALGO_MFMA_64 = 9,
    SGEMM_ALGO_MFMA_32 = 10,
    SGEMM_ALGO_MFMA_128X64 = 11
} sgemm_algo;

/*
 * Environment: SGEMM_F32_ALGO, read once per process, forces the algorithm of
 * the AUTO entry points (sgemm_f32, and sgemm_f32_algo / sgemm_f32_plan with
 * SGEMM_ALGO_AUTO): the lower-case name of an sgemm_algo value without its
 * prefix ("naive", "lds_tiled", "regblock", "mfma", "lds_tiled_nopad",
 * "naive_wg", "mfma_256", "mfma_128", "mfma_64", "mfma_32", "mfma_128x64";
 * "auto" or an
 * empty value: no override) or its number.  Any other value makes those calls
 * return SGEMM_ERR_INVALID_VALUE.  The workspace, k-split, stream-K and
 * mixed-precision calls are not affected.
 */

/*
 * C <- alpha*A*op(B) + beta*C with the AUTO algorithm.
 * Arguments as described above; `stream` is a hipStream_t (NULL: null stream).
 * Returns an sgemm_status.
 */
int sgemm_f32(int64_t M, int64_t N, int64_t K, float alpha,
              const float *A, int64_t lda, const float *B, int64_t ldb, int transB,
              float beta, float *C, int64_t ldc, void *stream);

/* The same operation with an explicit algorithm (an sgemm_algo value). */
int sgemm_f32_algo(int algo, int64_t M, int64_t N, int64_t K, float alpha,
                   const float *A, int64_t lda, const float *B, int64_t ldb, int transB,
                   float beta, float *C, int64_t ldc, void *stream);

/*
 * Host-only planning query, no HIP call: validates the arguments exactly as
 * sgemm_f32_algo would (pointers may be any non-NULL values; only their
 * numeric ranges are compared for aliasing) and reports what would run.
 *   *kernel_id   receives the launched kernel's id (0 when nothing would launch);
 *   *tiles_m, *tiles_n receive the workgroup grid (0 when nothing would launch);
 *   name/name_len receive a NUL-terminated kernel description (may be NULL/0).
 * Returns the sgemm_status the call would return before touching the device.
 */
int sgemm_f32_plan(int algo, int64_t M, int64_t N, int64_t K, float alpha,
                   const float *A, int64_t lda, const float *B, int64_t ldb, int transB,
                   float beta, const float *C, int64_t ldc,
                   int *kernel_id, int64_t *tiles_m, int64_t *tiles_n,
                   char *name, int name_len);

/*
 * Out-of-place FP32 matrix transpose (a second, memory-bound operation of the
 * library):
 *
 *     dst(j, i) = src(i, j)        0 <= i < rows, 0 <= j < cols
 *
 * The operation, its naive baseline and its shared-memory version with one
 * padding column per tile row are those of "现代 CUDA 工具箱实战：从朴素代码到硬件
 * 极限的优化之路", section 代码实现 (square N x N there; any rows x cols here).
 *
 * Layout (row-major, leading dimensions in elements):
 *   src    rows x cols,  element (i,j) at src[i*ld_src + j],  ld_src >= max(1, cols)
 *   dst    cols x rows,  element (j,i) at dst[j*ld_dst + i],  ld_dst >= max(1, rows)
 * Elements are moved bit for bit (NaN payloads, signed zeros and subnormals
 * included); dst elements outside the cols x rows window (row padding) are not
 * written.
 *
 * Ownership and asynchrony as for sgemm_f32: device pointers owned by the caller,
 * no allocation, no workspace, no synchronisation; the call enqueues one kernel
 * on `stream` and returns.
 *
 * Quick return: rows == 0 or cols == 0 touches nothing and returns SGEMM_OK.
 * Errors:
 *   SGEMM_ERR_INVALID_VALUE   negative or too large (> 2^31 - 1025) dimension, a
 *                             leading dimension below its minimum, a NULL pointer
 *                             with a non-zero extent, an unknown algorithm id, or
 *                             2^32 or more work units of the chosen kernel (never
 *                             reached within device memory);
 *   SGEMM_ERR_ALIAS           dst's byte range overlaps src's (the transpose is out
 *                             of place only);
 *   SGEMM_ERR_NO_DEVICE, SGEMM_ERR_UNSUPPORTED_ARCH, SGEMM_ERR_LAUNCH as above.
 *
 * Algorithms:
 *   NAIVE      one work-item per element: source rows read contiguously,
 *              destination written with a stride of ld_dst between lanes (the
 *              page's baseline);
 *   LDS        128 x 128 tiles staged through LDS with a row pitch of 129
 *              floats: contiguous reads and writes, conflict-free LDS access (the
 *              page's shared-memory + padding version); up to 2048 tiles a
 *              persistent grid overlaps each workgroup's next loads with its
 *              current stores, above that one tile per workgroup with
 *              non-temporal loads and stores; with fewer tiles than CUs, 64 x 64
 *              tiles (pitch 65) instead;
 *   LDS_NOPAD  the same kernels without the padding column (the page's "forgot
 *              the padding" case); kept to measure the bank conflicts;
 *   NARROW     one work-item per destination element: destination rows written
 *              contiguously, source read with a stride of ld_src;
 *   AUTO       NAIVE for fewer than 32 source rows, NARROW for fewer than 32
 *              source columns, LDS otherwise.
 */
typedef enum {
    SGEMM_TRANSPOSE_AUTO = 0,
    SGEMM_TRANSPOSE_NAIVE = 1,
    SGEMM_TRANSPOSE_LDS = 2,
    SGEMM_TRANSPOSE_LDS_NOPAD = 3,
    SGEMM_TRANSPOSE_NARROW = 4
} sgemm_transpose_algo;

/* dst <- src^T with the AUTO algorithm.  Returns an sgemm_status. */
int sgemm_f32_transpose(int64_t rows, int64_t cols, const float *src, int64_t ld_src,
                        float *dst, int64_t ld_dst, void *stream);

/* The same operation with an explicit algorithm (an sgemm_transpose_algo value). */
int sgemm_f32_transpose_algo(int algo, int64_t rows, int64_t cols, const float *src,
                             int64_t ld_src, float *dst, int64_t ld_dst, void *stream);

/*
 * Host-only planning query for the transpose, no HIP call: validates exactly as
 * sgemm_f32_transpose_algo would and reports the kernel id (0 when nothing
 * would launch), the number of workgroups launched (each loops over tiles; at
 * most 2^20) and a NUL-terminated kernel name (name may be NULL/0).  Returns the status the call would return before
 * touching the device.
 */
int sgemm_f32_transpose_plan(int algo, int64_t rows, int64_t cols, const float *src,
                             int64_t ld_src, const float *dst, int64_t ld_dst,
                             int *kernel_id, int64_t *blocks, char *name, int name_len);

/*
 * Mixed precision (a variant with its own accuracy contract, not a faster
 * sgemm_f32):
 *
 *     C  <-  alpha * r(A) * r(op(B)) + beta * C
 *
 * A, B and C are the same FP32 row-major matrices as for sgemm_f32 (same
 * layout, leading dimensions, ownership, asynchrony, quick returns, errors and
 * aliasing rules); r converts each operand element to IEEE binary16 (`fp16`)
 * or to bfloat16 (`bf16`), rounding to nearest with ties to even, as the tile
 * is staged into LDS, and the matrix cores (v_mfma_f32_32x32x16_f16 / _bf16)
 * multiply the converted values and sum the products in FP32.  This is the
 * half-precision variant of "GPU矩阵乘法优化：共享内存Tiling技术实战", section 7.1
 * (convert to half precision before the matrix cores), with bfloat16 as the
 * second format.  fp16 keeps 11 significant bits and overflows past 65504
 * (values that large become inf); bf16 keeps 8 significant bits with the FP32
 * exponent range.  C, alpha and beta stay FP32.
 *
 * Accuracy: against the exact result on the ROUNDED operands,
 *     |D - D~| <= 4*K*2^-24 * sum_k |r(a(i,k)) * r(b(k,j))| + 1e-6
 * (every product of two rounded operands is exact in FP32, so only the
 * summation rounds).  Against the exact FP32-operand product the difference
 * is larger by up to (2u + u^2) * sum_k |a*b|, u = 2^-11 (fp16) or 2^-8 (bf16)
 * -- the numerical-stability caveat of that section.
 */
typedef enum {
    SGEMM_PREC_FP16 = 1,
    SGEMM_PREC_BF16 = 2
} sgemm_precision;

/* The mixed-precision GEMM above; `precision` is an sgemm_precision value
 * (anything else: SGEMM_ERR_INVALID_VALUE).  Returns an sgemm_status. */
int sgemm_f32_lowp(int precision, int64_t M, int64_t N, int64_t K, float alpha,
                   const float *A, int64_t lda, const float *B, int64_t ldb, int transB,
                   float beta, float *C, int64_t ldc, void *stream);

/* Host-only planning query for sgemm_f32_lowp, the counterpart of sgemm_f32_plan.
 * The kernel takes 256 x 256 output tiles when there are at least 128 of them
 * (half the compute units), else 64 x 64 tiles; tiles_m / tiles_n count them. */
int sgemm_f32_lowp_plan(int precision, int64_t M, int64_t N, int64_t K, float alpha,
                        const float *A, int64_t lda, const float *B, int64_t ldb, int transB,
                        float beta, const float *C, int64_t ldc,
                        int *kernel_id, int64_t *tiles_m, int64_t *tiles_n,
                        char *name, int name_len);

/*
 * Mixed precision with a caller workspace: the same operation, rounding and
 * accuracy contract as sgemm_f32_lowp, in two passes.  A rounding pass writes
 * r(A) (M x K) and r(op(B)) (N x K, op(B) = B transposed on the way) into the
 * workspace as k-contiguous 16-bit rows, zero-padded to whole output tiles
 * and to a multiple of 32 in k; the GEMM then stages those 16-bit tiles
 * straight from memory into LDS (the one-pass kernel re-reads the FP32
 * operands and converts them inside its k-loop).  The FP32 sums run in the
 * same k order as the one-pass kernel's, so for a given tile size the two
 * calls give the same bits.
 *
 * Workspace: a DEVICE buffer owned by the caller, 16-byte aligned, at least
 * the bytes sgemm_f32_lowp_ws_plan reports (2 * K' * (M' + N') plus alignment,
 * M' and N' rounded up to the tile, K' to 32), not overlapping A, B or C
 * (SGEMM_ERR_ALIAS), ordered on one stream with its other uses; its contents
 * on return are undefined.  With a smaller or misaligned workspace (or NULL)
 * the call runs exactly as sgemm_f32_lowp.  Everything else (validation, quick returns,
 * asynchrony) is sgemm_f32_lowp's.
 */
int sgemm_f32_lowp_ws(int precision, int64_t M, int64_t N, int64_t K, float alpha,
                      const float *A, int64_t lda, const float *B, int64_t ldb, int transB,
                      float beta, float *C, int64_t ldc,
                      void *workspace, int64_t workspace_bytes, void *stream);

/* Host-only query for sgemm_f32_lowp_ws: the kernel id (64/65: fp16/bf16 with
 * 256 x 256 tiles, chosen when there are more than 128 of them; 66/67: 128 x
 * 128 tiles; otherwise the one-pass call's id: the two passes run for products
 * of at least 1e10 FLOPs, of at least 4e9 FLOPs with K >= min(M, N), or of 1e9
 * when M or N is not a multiple of 64 or K of 32, where they measured faster,
 * and K <= 64 * 65535 = 4,194,240; longer K
 * runs the one-pass call), the output tiles and the workspace bytes (0 when
 * the one-pass call runs).  Output pointers may be NULL. */
int sgemm_f32_lowp_ws_plan(int precision, int64_t M, int64_t N, int64_t K, int transB, int *kernel_id,
                           int64_t *tiles_m, int64_t *tiles_n, int64_t *workspace_bytes);

/* The two passes whatever the size (`tile`: 0 = the rule above, 256 or 128 =
 * that tile; anything else SGEMM_ERR_INVALID_VALUE), for callers that want
 * them and for testing them at every shape.  A workspace smaller than
 * sgemm_f32_lowp_2pass_plan reports or not 16-byte aligned, or K above
 * 4,194,240, is SGEMM_ERR_INVALID_VALUE. */
int sgemm_f32_lowp_2pass(int precision, int tile, int64_t M, int64_t N, int64_t K, float alpha,
                         const float *A, int64_t lda, const float *B, int64_t ldb, int transB,
                         float beta, float *C, int64_t ldc,
                         void *workspace, int64_t workspace_bytes, void *stream);

/* Host-only query for sgemm_f32_lowp_2pass, with the outputs of
 * sgemm_f32_lowp_ws_plan. */
int sgemm_f32_lowp_2pass_plan(int precision, int tile, int64_t M, int64_t N, int64_t K, int transB,
                              int *kernel_id, int64_t *tiles_m, int64_t *tiles_n,
                              int64_t *workspace_bytes);

/*
 * k-split with a caller workspace.  A product whose 64 x 64 output tiles are
 * too few to keep the 256 CUs busy (for example 512^3, or a small M x N with a
 * long K such as 256 x 256 x 8192) can split its k-range over several
 * workgroups per tile: split s multiplies k in [s*kc, min(K, (s+1)*kc)) (kc a
 * multiple of 32) into its own FP32 partial product in the workspace, and a
 * second kernel adds the partials in a fixed order and applies the epilogue
 *     C <- alpha * sum_s partial_s + beta*C      (C not read when beta == 0).
 * The result is the same operation under the same accuracy contract as
 * sgemm_f32 (each element is still a sum of its K products, "CUDA矩阵乘法性能优化
 * 实战：从朴素内核到寄存器分块与Nsight剖析" section 1.1; splitting a sum into partial
 * sums is the Tiling page's own device, "GPU矩阵乘法优化：共享内存Tiling技术实战"
 * section 4.2), reproducible from call to call, but its rounding differs from
 * the unsplit kernel's.
 *
 * Workspace: a DEVICE buffer owned by the caller, at least splits*M*N*4 bytes
 * (sgemm_f32_splitk_plan reports the size), starting on a 16-byte boundary
 * (every workspace of the library does; hipMalloc's are), not overlapping A,
 * B or C (SGEMM_ERR_ALIAS).  Its contents on entry are ignored and on return
 * undefined; it must stay allocated until the kernels enqueued on `stream`
 * have run.  Calls that share one workspace must be ordered on one stream.
 * The library itself still allocates nothing.
 */

/*
 * Host-only query, no HIP call: the split count a call with this shape would
 * use (`splits` = 0: what sgemm_f32_ws chooses -- no split while the 64 x 64
 * tile grid has at least 128 tiles; otherwise floor(512 / tiles) splits, two
 * workgroups per CU, when each gets at least 1024 of k, else the most splits
 * that keep one workgroup per CU with at least 128 of k each, at most 64; and
 * no split when that comes to 4 or fewer, where the plain call's 32 x 32 tile
 * already runs as many workgroups; otherwise the requested count, clipped to
 * the non-empty splits), the MFMA kernel id of the partial pass, and the
 * workspace bytes it needs.  *splits_used = 1 and *workspace_bytes = 0 when
 * the call runs unsplit (shapes that already fill the chip, K too short to
 * split, product-free cases).  Returns SGEMM_ERR_INVALID_VALUE for invalid
 * dimensions, transB or a split count outside 0..64.  Output pointers may be NULL.
 */
int sgemm_f32_splitk_plan(int64_t splits, int64_t M, int64_t N, int64_t K, int transB,
                          int64_t *splits_used, int *kernel_id, int64_t *workspace_bytes);

/*
 * sgemm_f32 with a workspace: runs the k-split or the stream-K schedule below
 * as sgemm_f32_ws_plan reports, when workspace_bytes is at least the size it
 * reports and the workspace is 16-byte aligned; otherwise (including
 * workspace == NULL) it runs exactly as sgemm_f32.
 */
int sgemm_f32_ws(int64_t M, int64_t N, int64_t K, float alpha,
                 const float *A, int64_t lda, const float *B, int64_t ldb, int transB,
                 float beta, float *C, int64_t ldc,
                 void *workspace, int64_t workspace_bytes, void *stream);

/*
 * The same with an explicit split count (1..64; 1 runs the plain MFMA path).
 * A workspace smaller than sgemm_f32_splitk_plan(splits, ...) reports, or not
 * 16-byte aligned, is SGEMM_ERR_INVALID_VALUE.
 */
int sgemm_f32_splitk(int64_t splits, int64_t M, int64_t N, int64_t K, float alpha,
                     const float *A, int64_t lda, const float *B, int64_t ldb, int transB,
                     float beta, float *C, int64_t ldc,
                     void *workspace, int64_t workspace_bytes, void *stream);

/*
 * The k-split for callers that cannot allocate (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): sgemm_f32_splitk
 * with the partial products in the library's own static device scratch
 * instead of a caller workspace.  The operation, the kernels, the result
 * bits and the argument checks are sgemm_f32_splitk's with one addition:
 * splits = 0 (which sgemm_f32_splitk rejects) takes the split count of the
 * AUTO rule of sgemm_f32_ws, and runs the plain call where that rule does not
 * split.  The call allocates and frees nothing and calls no allocating
 * library routine.
 *
 * Scratch: SGEMM_F32_SCRATCH_BYTES (16 MiB) of device memory, one array per
 * GPU the library runs on, held until the process ends; its address on a
 * device is looked up on the first call there.  A split whose partials need
 * more (sgemm_f32_splitk_plan reports the bytes; the AUTO rule never needs
 * more than 8 MiB) returns SGEMM_ERR_SCRATCH_LIMIT before touching the
 * device.  Every call on one GPU shares that GPU's array and leaves its
 * contents behind (each call writes all of the partials it reads): calls that
 * may overlap on one GPU -- on different streams, or from different threads
 * without ordering -- race on it, and must be serialised by the caller.
 */
#define SGEMM_F32_SCRATCH_BYTES (16 << 20)
int sgemm_f32_splitk_noalloc(int64_t splits, int64_t M, int64_t N, int64_t K, float alpha,
                             const float *A, int64_t lda, const float *B, int64_t ldb, int transB,
                             float beta, float *C, int64_t ldc, void *stream);

/*
 * Stream-K.  With T output tiles and 256 CUs, a plain launch runs ceil(T/256)
 * waves of tiles and leaves CUs idle in the last one (T = 324 tiles of
 * 256 x 256 keep only 68 CUs busy in their second wave).  The stream-K
 * schedule (Osama et al., "Stream-K: Work-centric Parallel Decomposition for
 * Dense Matrix-Matrix Multiplication on the GPU") keeps the whole waves as
 * they are and deals the k-iterations of the remaining tiles (all of them when
 * T < 256) out evenly over up to 256 workgroups, each a contiguous run that may
 * start and end inside a tile.  A workgroup that covers a whole tile writes it
 * to C; every other piece of a tile is a raw FP32 partial product in the
 * workspace, and a fix-up kernel adds a tile's pieces in k order and applies
 * C <- alpha * sum + beta*C (C not read when beta == 0).  The operation, its
 * accuracy contract and its determinism are those of the k-split above (a
 * sum of K products split into partial sums, in a fixed order).
 *
 * `tile`: 0 = the library's choice from its cost model, 256 = the 256 x 256
 * tile, 128 = the 128 x 128 tile (anything else: SGEMM_ERR_INVALID_VALUE).
 * Workspace: a DEVICE buffer owned by the caller, at least
 * 2 * workers * tile_rows * tile_cols * 4 bytes (sgemm_f32_streamk_plan
 * reports it; 0 when T is a multiple of 256 and the schedule is the plain
 * one), with the same rules as the k-split workspace (16-byte aligned, any
 * contents, not overlapping A, B or C, ordered on one stream).  Too small or
 * misaligned: SGEMM_ERR_INVALID_VALUE.
 * Quick returns, product-free cases and argument errors are sgemm_f32's.
 */
int sgemm_f32_streamk(int tile, int64_t M, int64_t N, int64_t K, float alpha,
                      const float *A, int64_t lda, const float *B, int64_t ldb, int transB,
                      float beta, float *C, int64_t ldc,
                      void *workspace, int64_t workspace_bytes, void *stream);

/*
 * Host-only query for sgemm_f32_streamk: the kernel id (43: 256 x 256
 * stream-K, 44: 128 x 128 stream-K; the plain call's id for quick returns and
 * product-free cases), the tiles run data-parallel, the tiles shared out, the
 * stream-K workgroups and the workspace bytes.  Output pointers may be NULL.
 */
int sgemm_f32_streamk_plan(int tile, int64_t M, int64_t N, int64_t K, int transB, int *kernel_id,
                           int64_t *dp_tiles, int64_t *sk_tiles, int64_t *workers,
                           int64_t *workspace_bytes);

/*
 * Host-only query of what sgemm_f32_ws does with a large enough workspace:
 * *method = 1 (k-split) when sgemm_f32_splitk_plan(0, ...) splits; otherwise
 * 2 (stream-K) when the library's cost model expects stream-K to be at least
 * 1% faster than the plain call; otherwise 0 (plain).  Also the kernel id and
 * the workspace bytes that method needs (0 for the plain call).  With a
 * smaller or misaligned workspace sgemm_f32_ws runs the plain call.
 */
int sgemm_f32_ws_plan(int64_t M, int64_t N, int64_t K, int transB, int *method, int *kernel_id,
                      int64_t *workspace_bytes);

/* Static, NUL-terminated text for a status code (unknown codes included). */
const char *sgemm_f32_status_string(int status);

/* Static, NUL-terminated library version string; debug builds of the library
 * (LDS poisoning, host sanitizers) say so in it. */
const char *sgemm_f32_version(void);

/*
 * The device check every call makes before it enqueues work (the "no kernel
 * image" case of "CUDA矩阵乘法性能优化实战：从朴素内核到寄存器分块与Nsight剖析",
 * section 6.2: code built for one architecture does not run on another).
 *
 * sgemm_f32_arch_status: host-only, no HIP call.  `arch` is an architecture
 * name as HIP reports it in hipDeviceProp_t::gcnArchName: a processor name,
 * optionally followed by ':'-separated target features.  Returns SGEMM_OK when
 * the processor is gfx950 (with any features), SGEMM_ERR_UNSUPPORTED_ARCH
 * otherwise (NULL and the empty string included).
 *
 * sgemm_f32_device_status: the current HIP device of the calling thread:
 * SGEMM_ERR_NO_DEVICE when there is none (no GPU, or none visible),
 * SGEMM_ERR_UNSUPPORTED_ARCH when its architecture fails the check above,
 * SGEMM_OK otherwise.  Enqueues nothing.
 */
int sgemm_f32_arch_status(const char *arch);
int sgemm_f32_device_status(void);

/*
 * Measurement aid, not part of the GEMM: the FP32 matrix-core rate the device
 * sustains and the shader clock it runs at.  The roofline of the GEMM is the
 * matrix cores' peak ("CUDA矩阵乘法性能优化实战：从朴素内核到寄存器分块与Nsight剖析",
 * section 1.2, places a kernel against the peak rate and the ridge point); the
 * published figure is a clock times a unit count, and the Baidu Cloud page on
 * naive versus 2-D tiled matrix multiplication (its migration advice on
 * performance evaluation) asks for measurement on the target hardware rather
 * than conclusions from theory alone.  It launches `workgroups` workgroups of
 * four wavefronts; each wavefront issues trips * 8 v_mfma_f32_32x32x2_f32 on
 * random operands in registers (4096 FLOP each; no memory traffic but the
 * final stores), so one call performs workgroups * 4 * trips * 8 * 4096 FLOP.
 * Wavefront 0 of workgroup w writes its elapsed shader cycles to clocks[2w] and
 * elapsed ticks of the constant 100 MHz counter to clocks[2w+1] (shader clock
 * in MHz = 100 * clocks[2w] / clocks[2w+1]); every work-item writes one float
 * of its sums to sink (keeps the work live; the values carry no meaning).
 *
 * sink: DEVICE buffer of workgroups * 256 floats; clocks: DEVICE buffer of
 * workgroups * 2 uint64; both owned by the caller, not overlapping
 * (SGEMM_ERR_ALIAS).  workgroups in 1..2^20, trips in 1..2^24, else
 * SGEMM_ERR_INVALID_VALUE (checked before any HIP call).  Enqueued on `stream`;
 * SGEMM_ERR_NO_DEVICE / SGEMM_ERR_UNSUPPORTED_ARCH / SGEMM_ERR_LAUNCH as
 * sgemm_f32.
 */
int sgemm_f32_mfma_probe(int64_t workgroups, int64_t trips, float *sink, unsigned long long *clocks,
                         void *stream);

/*
 * Measurement aid, not part of the GEMM: the same chain on the 16-bit matrix
 * cores behind the mixed-precision calls ("GPU矩阵乘法优化：共享内存Tiling技术实战",
 * section 7.1: half-precision operands on the matrix cores).  Each wavefront
 * issues trips * 8 v_mfma_f32_32x32x16_{f16,bf16} (32768 FLOP each; precision
 * SGEMM_PREC_FP16 or SGEMM_PREC_BF16) over four accumulators, on eight operand
 * pairs of random values in [-1, 1) rounded to 16 bits, or all zeros when
 * zero_operands = 1 (how much the operands toggle decides the power the matrix
 * cores draw, and with it the clock the part holds).  One call performs
 * workgroups * 4 * trips * 8 * 32768 FLOP.  sink, clocks, the limits, the
 * errors and the asynchrony are sgemm_f32_mfma_probe's; precision or
 * zero_operands out of range: SGEMM_ERR_INVALID_VALUE.
 */
int sgemm_f32_mfma_probe_lp(int precision, int zero_operands, int64_t workgroups, int64_t trips, float *sink,
                            unsigned long long *clocks, void *stream);

/*
 * Measurement aid, not part of the GEMM: the rate at which one CU stages
 * global memory into LDS with the direct loads the MFMA kernels use
 * (global_load_lds_dwordx4: 16 bytes per lane, 1 KB per wavefront instruction,
 * no registers), with nothing else running.  The tiled kernels' pages put a
 * kernel's time in its loads and their latency ("GPU矩阵乘法优化：共享内存Tiling
 * 技术实战", section 3.2, double buffering hides the load latency); this gives
 * that stream's own ceiling.  `workgroups` workgroups of `waves` wavefronts
 * (4 or 8); each workgroup claims 100 KB of LDS, so one runs per CU.
 * Workgroup w reads the region g = w % 8 + 8 * ((w / 8) / share) of
 * `region_bytes` bytes at src + g * region_bytes (workgroups are dealt to the
 * eight XCDs in turn, so `share` workgroups of one XCD read each region, as
 * the tiles of a GEMM share operand panels); its wavefront v issues `loads`
 * loads, the j-th taking the region's 1 KB chunk (j * waves + v) modulo
 * region_bytes / 1024, and keeps at most `depth` (1, 2, 4 or 8) in flight.  The
 * data land in LDS and are dropped.  Wavefront 0 writes the elapsed shader
 * cycles (all of the workgroup's loads landed) to clocks[2w] and the 100 MHz
 * ticks to clocks[2w+1]: one workgroup moves loads * waves * 1024 bytes.
 *
 * src: DEVICE buffer of src_bytes bytes, 16-byte aligned, owned by the caller
 * and only read; it must hold every region read,
 * (8 * (((workgroups - 1) / 8) / share) + 8) * region_bytes bytes.  clocks:
 * DEVICE buffer of workgroups * 2 uint64, not overlapping those regions
 * (SGEMM_ERR_ALIAS).  workgroups in 1..2^16, share in 1..2^16, loads in
 * 1..2^24, region_bytes a multiple of 1024 in 1024..2^31, else
 * SGEMM_ERR_INVALID_VALUE (checked before any HIP call).  Enqueued on
 * `stream`; SGEMM_ERR_NO_DEVICE / SGEMM_ERR_UNSUPPORTED_ARCH /
 * SGEMM_ERR_LAUNCH as sgemm_f32.
 */
int sgemm_f32_load_probe(int waves, int depth, int64_t workgroups, const void *src, int64_t src_bytes,
                         int64_t region_bytes, int64_t share, int64_t loads, unsigned long long *clocks,
                         void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SGEMM_F32_H */
