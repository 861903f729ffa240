/*
 * libgemm -- dense matrix multiply C = A.B for AMD Instinct MI355X (gfx950).
 *
 * The operation every page describes: A is M x K, B is K x N, C is M x N and
 *     C[i][j] = sum over k = 0 .. K-1 of A[i][k] * B[k][j]
 * ("GEMM", Part 4 of How to make your models fast, opening definition;
 *  "GEMM Optimization", section "The Problem").  C is overwritten.
 *
 * Layout.  Each operand is a logical matrix with its own leading dimension and order:
 * element (r, c) of a logical R x C operand X is X[r*ldx + c] when the order is
 * GEMM_ROW_MAJOR and X[r + c*ldx] when it is GEMM_COL_MAJOR.  Leading dimensions must
 * be at least:
 *     A: K (row-major) or M (column-major);  B: N (row-major) or K (column-major);
 *     C: N (row-major) or M (column-major);  and always at least 1.
 * The matrix-core example of "How a Matrix Multiply Runs on a GPU" (section "Level 3:
 * tensor cores") uses row-major A with column-major B (ld = K); any mix is accepted.
 *
 * Degenerate sizes.  M == 0 or N == 0: nothing is launched, GEMM_OK.  K == 0: C is set
 * to zero (the empty sum; zero is the additive identity, as the teaching module's
 * boundary discussion puts it in "A06 - Tiled Matrix Multiply (GEMM)", section "The
 * tiled kernel, and what each line is protecting").
 *
 * Ownership.  All matrix pointers are device pointers owned by the caller; A and B are
 * only read and must not overlap C.  C is only written, except by the fused-epilogue calls
 * with beta != 0, which read C's previous contents first, and by AUTO's two-halves mode for
 * few FP32 rows (SKINNY below), which zeroes C and then adds two partial sums into it with
 * device-scope atomic float adds (C must then be ordinary device memory, as from hipMalloc).  Pointers need only their element's
 * natural alignment (4 bytes for float, 2 for bf16/fp16, 1 for fp8); no kernel needs more.  The plain
 * calls allocate no device memory and keep no state beyond a per-device property cache; the
 * _ws calls use the caller's workspace, and gemm_bf16_f32acc_noalloc a static array of the
 * library's (both below).
 *
 * Streams and errors.  Work is enqueued on `stream` (0 = the null stream) of the
 * current device and the call returns without waiting for it.  Argument errors are
 * detected before anything is enqueued and leave C untouched:
 *     GEMM_ERR_INVALID_VALUE      negative size, leading dimension too small, unknown
 *                                 order or algorithm, null pointer for a non-empty
 *                                 operand, or a shape the chosen algorithm cannot run;
 *     GEMM_ERR_UNSUPPORTED_DEVICE the current device is not gfx950;
 *     GEMM_ERR_LAUNCH             the HIP runtime refused the launch (see
 *                                 gemm_last_hip_error);
 *     GEMM_ERR_SCRATCH_TOO_SMALL  gemm_bf16_f32acc_noalloc only: the problem's split-K partial
 *                                 sums would not fit in the library's static scratch.
 */
#ifndef LIBGEMM_GEMM_H
#define LIBGEMM_GEMM_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { GEMM_ROW_MAJOR = 0, GEMM_COL_MAJOR = 1 } gemm_order_t;

typedef enum {
    GEMM_OK = 0,
    GEMM_ERR_INVALID_VALUE = 1,
    GEMM_ERR_UNSUPPORTED_DEVICE = 2,
    GEMM_ERR_LAUNCH = 3,
    GEMM_ERR_SCRATCH_TOO_SMALL = 4
} gemm_status_t;

/*
 * Kernel choice.  GEMM_ALGO_AUTO lets the library pick from the shape, dtype and
 * alignment.  The others force one kernel; they exist so that each step of the pages'
 * ladder can be run, checked and measured on its own:
 *   NAIVE_UNCOALESCED  one thread per output, the thread's fast index walks rows of C
 *                      ("GEMM", Part 4, the first direct kernel);
 *   NAIVE              one thread per output, fast index along columns of C
 *                      ("How a Matrix Multiply Runs on a GPU", "Level 0");
 *   TILED              32 x 32 tiles staged in LDS, one output per thread ("Level 1");
 *   REGBLOCK           128 x 128 block tiles, 8 x 8 outputs per thread on the vector
 *                      ALUs, double-buffered LDS ("Level 2"; "GEMM Optimization", V2/V3);
 *   MFMA               the matrix-core kernels only (AUTO without the small-problem kernel),
 *                      tile and kernel picked by the same cost model as AUTO ("A06 - Tiled
 *                      Matrix Multiply (GEMM)", "Matrix cores: MFMA and Tensor Cores").  FP32:
 *                      the direct-copy kernel (v_mfma_f32_16x16x4_f32, MFMA_DMA below)
 *                      wherever it applies, else the register-staged kernel
 *                      (v_mfma_f32_32x32x2_f32, 128 x 128 or 64 x 64 tiles, any layout).  BF16 /
 *                      FP16: the direct-copy kernel (v_mfma_f32_32x32x16_bf16 / _f16) for
 *                      row-major A with column-major B, or with row-major B and N % 8 == 0,
 *                      and K >= 64, else the register-staged kernel (128 x 128, 64 x 64 or
 *                      256 x 128 tiles, any layout);
 *   MFMA_256x256, MFMA_256x128, MFMA_128x128, MFMA_64x64
 *                      a block tile forced.  256x256: the direct-copy kernel at 256 x 256 (its
 *                      requirements below; GEMM_ERR_INVALID_VALUE otherwise).  256x128 (16-bit
 *                      inputs only): the direct-copy kernel at 256 x 128 where it applies, else
 *                      the register-staged kernel.  128x128, 64x64: the register-staged kernel;
 *   SKINNY             the small-problem kernel ("How a Matrix Multiply Runs on a GPU",
 *                      "Shapes that run slowly, and why": few rows make the product bound
 *                      by reading B; few tiles leave the chip idle): 64 x 16 or 64 x 64 blocks
 *                      of C per workgroup, K split over its eight wavefronts, partial sums added
 *                      in a fixed order; needs row-major A, and for 16-bit inputs a column-major
 *                      B (with a column-major C the roles of M/N and A/B swap, C^T = B^T A^T),
 *                      else GEMM_ERR_INVALID_VALUE.  AUTO uses it when it applies and M <= 64
 *                      or 64 x 64 tiles would fill less than half of the CUs.  For FP32 with
 *                      row-major A and B, M <= 16, K >= 4096, N and ldb even, B 8-byte aligned
 *                      and 32-column blocks giving between half and all of the CUs a
 *                      workgroup per K half, AUTO takes it in a two-halves mode instead (a
 *                      split of K; "A06", "The next two rungs"): C is zeroed, then one
 *                      workgroup per 32-column block and K half adds its sum into C (8-byte
 *                      loads along each row of B; exactly two contributions per output, so
 *                      the result does not depend on their order and repeats bit for bit).
 *                      With M <= 16, K >= 512 and N > 16 x CUs (16-column blocks would take
 *                      more than one round), AUTO runs one round of 32-column blocks over the
 *                      whole of K instead, with plain stores: for a column-major B of any input
 *                      type, and for a row-major FP32 B with N and ldb even and B 8-byte
 *                      aligned;
 *   MFMA_DMA           the direct-copy kernels: operands copied global -> LDS as laid out in
 *                      memory by buffer loads straight into LDS, no register staging ("GEMM
 *                      Optimization", V3 staging), tile picked by the cost model.  FP32:
 *                      v_mfma_f32_16x16x4_f32, 256 x 256 tiles of eight wavefronts or 128 x 128
 *                      of four; needs K >= 32 and M, N at least the tile; tiles may overhang
 *                      the edge along a k-contiguous operand, other remainders run as strips on
 *                      the register-staged kernel in the same call.  16-bit inputs:
 *                      v_mfma_f32_32x32x16, 256 x 256 tiles of four wavefronts (128 x 128 each,
 *                      a ring of five half-stage LDS buffers) or 256 x 128 of eight (64 x 64
 *                      each, three stages); needs row-major A and K >= 64, with column-major B
 *                      any M and N (tiles overhang both edges; rows past M or N read as zero),
 *                      with row-major B (kept in LDS as laid out and read by gfx950's
 *                      transposing LDS read) any M and N % 8 == 0, and element offsets into B
 *                      below 2^30.
 *                      Conditions apply after the column-major-C swap; otherwise
 *                      GEMM_ERR_INVALID_VALUE.  AUTO picks these kernels wherever they apply and
 *                      the cost model prefers them (every workload of the benchmark suite).
 * The FP32 entry point accepts every algorithm but MFMA_256x128; the 16-bit entry points only
 * AUTO, the MFMA ones and SKINNY (others give GEMM_ERR_INVALID_VALUE).  The value 10 is unused
 * (it named a ping-pong kernel that was slower than the direct-copy kernel and was removed).
 */
typedef enum {
    GEMM_ALGO_AUTO = 0,
    GEMM_ALGO_NAIVE_UNCOALESCED = 1,
    GEMM_ALGO_NAIVE = 2,
    GEMM_ALGO_TILED = 3,
    GEMM_ALGO_REGBLOCK = 4,
    GEMM_ALGO_MFMA = 5,
    GEMM_ALGO_MFMA_256x256 = 6,
    GEMM_ALGO_MFMA_256x128 = 7,
    GEMM_ALGO_MFMA_128x128 = 8,
    GEMM_ALGO_MFMA_64x64 = 9,
    GEMM_ALGO_SKINNY = 11,
    GEMM_ALGO_MFMA_DMA = 12
} gemm_algo_t;

/* FP32 inputs, FP32 arithmetic, FP32 C.  Same as gemm_f32_algo(GEMM_ALGO_AUTO, ...). */
gemm_status_t gemm_f32(int64_t M, int64_t N, int64_t K,
                       const float *A, int64_t lda, gemm_order_t order_a,
                       const float *B, int64_t ldb, gemm_order_t order_b,
                       float *C, int64_t ldc, gemm_order_t order_c,
                       hipStream_t stream);

/* BF16 inputs (raw bit patterns, 2 bytes each), products and sums in FP32, FP32 C.
 * Same as gemm_bf16_f32acc_algo(GEMM_ALGO_AUTO, ...). */
gemm_status_t gemm_bf16_f32acc(int64_t M, int64_t N, int64_t K,
                               const uint16_t *A, int64_t lda, gemm_order_t order_a,
                               const uint16_t *B, int64_t ldb, gemm_order_t order_b,
                               float *C, int64_t ldc, gemm_order_t order_c,
                               hipStream_t stream);

/* FP16-input, FP32-accumulate GEMM: as gemm_bf16_f32acc, with A and B holding IEEE
 * binary16 bit patterns (1 sign, 5 exponent, 10 fraction bits), the other 16-bit input
 * type of the matrix cores ("A06 - Tiled Matrix Multiply (GEMM)", "Matrix cores: MFMA and
 * Tensor Cores"): the same kernels with the fp16 matrix instructions
 * (v_mfma_f32_32x32x16_f16, v_mfma_f32_16x16x32_f16); every product of two fp16 values is
 * exact in FP32, sums are FP32.  Layouts, kernel choice and errors as for BF16. */
gemm_status_t gemm_f16_f32acc(int64_t M, int64_t N, int64_t K,
                              const uint16_t *A, int64_t lda, gemm_order_t order_a,
                              const uint16_t *B, int64_t ldb, gemm_order_t order_b,
                              float *C, int64_t ldc, gemm_order_t order_c,
                              hipStream_t stream);

/* 8-bit floating-point inputs, FP32 products and sums, FP32 C.  The matrix cores take fp8 as
 * well as 16-bit inputs with FP32 accumulation ("A06 - Tiled Matrix Multiply (GEMM)", "Matrix
 * cores: MFMA and Tensor Cores", the table's inputs row), and quantized inference runs this same
 * GEMM on a narrower operand type (same page, section 7, "Real-World Use Cases").  A and B hold
 * one byte per element in one of the two OCP 8-bit formats, chosen per operand:
 *   GEMM_FP8_E4M3  sign, 4 exponent bits (bias 7), 3 fraction bits; subnormals; no infinities;
 *                  S.1111.111 is NaN; largest finite 448;
 *   GEMM_FP8_E5M2  sign, 5 exponent bits (bias 15), 2 fraction bits; subnormals; IEEE infinities
 *                  (S.11111.00) and NaNs (S.11111.xx, xx != 00); largest finite 57344.
 * C[i][j] = sum over k of decode(A[i][k]) * decode(B[k][j]); every product is exact in FP32,
 * sums are FP32 (v_mfma_scale_f32_32x32x64_f8f6f4 with unit block scales), so results agree with
 * an exact sum to FP32 rounding of partial sums, as for BF16.  A NaN or infinite input gives a
 * non-finite result in its row or column of C.
 * Layout: A row-major and B column-major (both contiguous along k, one byte apart; the
 * layout the 8-bit matrix instruction gathers its operands in); C either order; lda >= K and
 * ldb >= K, any alignment.  Any M, N, K (K == 0: C = 0).  The library has no other kernel for
 * these inputs and no split-K path for them.
 * Errors: GEMM_ERR_INVALID_VALUE as for gemm_bf16_f32acc, and for a format other than the two
 * below or A column-major or B row-major. */
typedef enum { GEMM_FP8_E4M3 = 0, GEMM_FP8_E5M2 = 1 } gemm_fp8_t;
gemm_status_t gemm_fp8_f32acc(int64_t M, int64_t N, int64_t K,
                              const uint8_t *A, int64_t lda, gemm_order_t order_a, gemm_fp8_t format_a,
                              const uint8_t *B, int64_t ldb, gemm_order_t order_b, gemm_fp8_t format_b,
                              float *C, int64_t ldc, gemm_order_t order_c,
                              hipStream_t stream);

/* As gemm_f32, with the kernel forced (see gemm_algo_t). */
gemm_status_t gemm_f32_algo(gemm_algo_t algo, int64_t M, int64_t N, int64_t K,
                            const float *A, int64_t lda, gemm_order_t order_a,
                            const float *B, int64_t ldb, gemm_order_t order_b,
                            float *C, int64_t ldc, gemm_order_t order_c,
                            hipStream_t stream);

/* As gemm_bf16_f32acc, with the kernel forced (AUTO or one of the MFMA values). */
gemm_status_t gemm_bf16_f32acc_algo(gemm_algo_t algo, int64_t M, int64_t N, int64_t K,
                                    const uint16_t *A, int64_t lda, gemm_order_t order_a,
                                    const uint16_t *B, int64_t ldb, gemm_order_t order_b,
                                    float *C, int64_t ldc, gemm_order_t order_c,
                                    hipStream_t stream);

/* As gemm_f16_f32acc, with the kernel forced (AUTO, one of the MFMA values or SKINNY). */
gemm_status_t gemm_f16_f32acc_algo(gemm_algo_t algo, int64_t M, int64_t N, int64_t K,
                                   const uint16_t *A, int64_t lda, gemm_order_t order_a,
                                   const uint16_t *B, int64_t ldb, gemm_order_t order_b,
                                   float *C, int64_t ldc, gemm_order_t order_c,
                                   hipStream_t stream);

/* Static, never-null description of a status code. */
const char *gemm_status_string(gemm_status_t status);

/* hipError_t of this thread's last GEMM_ERR_LAUNCH (0 if none yet). */
int gemm_last_hip_error(void);

/* Name of the kernel the last successful call on this thread enqueued (static string,
 * "none" before any call); for tests and the bench. */
const char *gemm_last_kernel(void);

/* Library version, e.g. "0.1.0". */
const char *gemm_version(void);

/* What gemm_f32 (dtype 0), gemm_bf16_f32acc (dtype 1), gemm_f16_f32acc (dtype 2) or
 * gemm_fp8_f32acc (dtype 3; either format: the choice does not depend on it) would run
 * for a problem of these extents and orders, with tight leading dimensions, on a device of `cus` compute units,
 * without touching a device or launching anything; for tests of the kernel choice.
 *   *kernel     static name, as gemm_last_kernel() would report it ("none" for M == 0 or
 *               N == 0, "zero_c" for K == 0);
 *   *core_rows, *core_cols   the part of C the named kernel's own launch covers, in the
 *               orientation the library computes in: C itself when order_c is row-major,
 *               C^T (N x M) when it is column-major.  The rest of C runs as edge strips,
 *               separate GEMMs on the same stream chosen the same way;
 *   *workspace_bytes   the workspace with which gemm_f32_ws / gemm_bf16_f32acc_ws split K
 *               across workgroups for this problem (0: they never do).
 * Errors: GEMM_ERR_INVALID_VALUE for a null output pointer, cus <= 0, a dtype other than
 * 0 .. 3, negative or too large extents (> INT_MAX), an invalid order, or for dtype 3 orders
 * gemm_fp8_f32acc refuses; outputs untouched then. */
gemm_status_t gemm_plan(int dtype, int64_t M, int64_t N, int64_t K, gemm_order_t order_a,
                        gemm_order_t order_b, gemm_order_t order_c, int cus, const char **kernel,
                        int64_t *core_rows, int64_t *core_cols, size_t *workspace_bytes);

/* ---- With a caller's workspace: split-K across workgroups ---------------------------------
 * "A06 - Tiled Matrix Multiply (GEMM)", "The next two rungs" (split-K: workers take parts of
 * K and a second step combines their partial sums): for problems whose output gives too few
 * workgroups to occupy the device, K is also divided among workgroups -- by the small-problem
 * kernel for few rows (or few columns after the column-major-C swap), and by the direct-copy
 * kernels on 256 x 256 tiles when those leave CUs idle (FP32 inputs with M and N multiples of
 * 256; 16-bit inputs in that kernel's layouts, row-major A with column-major B or with row-major
 * B and N % 8 == 0), where a time
 * model prices the split below the unsplit plan (one GPU's 4096 x 512 x 4096 column shard of a
 * 4096^3 product, for one).  The slices' partial products go to the workspace (the tile kernels
 * write the first slice straight to C) and a second kernel adds them in slice order, so results
 * are deterministic
 * (identical from call to call; they may differ in the last bits from the plain calls, which
 * sum in another order).  The library still allocates nothing.
 *
 * gemm_workspace_size: bytes of workspace with which the _ws calls split K for this problem
 * (dtype as for gemm_plan) on the current device (the same extents and orders as the call;
 * leading dimensions do not matter); 0 if they would not split, for invalid arguments, or
 * without a gfx950 device.
 *
 * gemm_f32_ws / gemm_bf16_f32acc_ws / gemm_f16_f32acc_ws: as the plain calls.  workspace: device
 * memory, 16-byte aligned, not overlapping A, B or C, of workspace_bytes bytes; it is used
 * only if workspace_bytes >= gemm_workspace_size(...) and the call would split; otherwise,
 * or with workspace == NULL, the call runs exactly as the plain one.  Its contents are
 * scratch: overwritten by the call and meaningless afterwards.  Calls that share one
 * workspace must not run concurrently (use one stream, or one workspace per stream).
 * Errors: as the plain calls, plus GEMM_ERR_INVALID_VALUE for a workspace that is not
 * 16-byte aligned. */
size_t gemm_workspace_size(int dtype, int64_t M, int64_t N, int64_t K, gemm_order_t order_a,
                           gemm_order_t order_b, gemm_order_t order_c);
gemm_status_t gemm_f32_ws(int64_t M, int64_t N, int64_t K,
                          const float *A, int64_t lda, gemm_order_t order_a,
                          const float *B, int64_t ldb, gemm_order_t order_b,
                          float *C, int64_t ldc, gemm_order_t order_c,
                          void *workspace, size_t workspace_bytes, hipStream_t stream);
gemm_status_t gemm_bf16_f32acc_ws(int64_t M, int64_t N, int64_t K,
                                  const uint16_t *A, int64_t lda, gemm_order_t order_a,
                                  const uint16_t *B, int64_t ldb, gemm_order_t order_b,
                                  float *C, int64_t ldc, gemm_order_t order_c,
                                  void *workspace, size_t workspace_bytes, hipStream_t stream);
gemm_status_t gemm_f16_f32acc_ws(int64_t M, int64_t N, int64_t K,
                                 const uint16_t *A, int64_t lda, gemm_order_t order_a,
                                 const uint16_t *B, int64_t ldb, gemm_order_t order_b,
                                 float *C, int64_t ldc, gemm_order_t order_c,
                                 void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Strided batched GEMM: C_z = A_z . B_z for z = 0 .. batch-1, every entry M x N x K with the
 * orders and leading dimensions of the plain calls.  Attention runs one such product per head:
 * the scores Q.K^T and the scores times V ("A06 - Tiled Matrix Multiply (GEMM)", sections
 * "2. First Principles" and "7. Real-World Use Cases").
 *
 * Entry z reads A + z*stride_a and B + z*stride_b and writes C + z*stride_c; strides count
 * elements (of the input type for A and B, floats for C).  stride_a or stride_b 0 uses one
 * operand for every entry.  Heads interleaved in one row, as in a [tokens, heads, head_dim]
 * tensor, are leading dimension heads*head_dim with stride head_dim.  Entries run on the kernels
 * the plain calls of the same type use (same arithmetic, same accuracy), the kernel and tile
 * chosen for the batch as a whole, all of them on `stream` in one launch per kernel (65535
 * entries at most per launch; more take several).
 * No workspace is used and nothing is allocated.
 *
 * Errors: as the plain calls, plus GEMM_ERR_INVALID_VALUE for batch < 0, a negative stride,
 * entry offsets beyond int64 bytes, or entries of C that may overlap: they must either follow
 * one another (stride_c at least one entry's span, (rows-1)*ldc + columns in C's own order) or
 * sit side by side within each row (stride_c >= the entry's row length, all batch entries
 * inside ldc).  batch == 0, M == 0 or N == 0: nothing happens. */
gemm_status_t gemm_f32_strided_batched(int64_t batch, int64_t M, int64_t N, int64_t K,
                                       const float *A, int64_t lda, int64_t stride_a, gemm_order_t order_a,
                                       const float *B, int64_t ldb, int64_t stride_b, gemm_order_t order_b,
                                       float *C, int64_t ldc, int64_t stride_c, gemm_order_t order_c,
                                       hipStream_t stream);
gemm_status_t gemm_bf16_f32acc_strided_batched(int64_t batch, int64_t M, int64_t N, int64_t K,
                                               const uint16_t *A, int64_t lda, int64_t stride_a,
                                               gemm_order_t order_a,
                                               const uint16_t *B, int64_t ldb, int64_t stride_b,
                                               gemm_order_t order_b,
                                               float *C, int64_t ldc, int64_t stride_c, gemm_order_t order_c,
                                               hipStream_t stream);
gemm_status_t gemm_f16_f32acc_strided_batched(int64_t batch, int64_t M, int64_t N, int64_t K,
                                              const uint16_t *A, int64_t lda, int64_t stride_a,
                                              gemm_order_t order_a,
                                              const uint16_t *B, int64_t ldb, int64_t stride_b,
                                              gemm_order_t order_b,
                                              float *C, int64_t ldc, int64_t stride_c, gemm_order_t order_c,
                                              hipStream_t stream);

/* Fused epilogue: C = act(alpha * A.B + beta * C + bias), computed on each output inside the GEMM
 * kernel, between its accumulators and its store, and stored as FP32 or bf16 ("How a Matrix Multiply Runs on a GPU", section
 * "Level 2", the epilogue of the block-tile loop, and section "Operational guidance and
 * trade-offs"; "A06 - Tiled Matrix Multiply (GEMM)", section "6. Challenges, Drawbacks &
 * Tradeoffs").
 *
 *   alpha, beta   scale of the product and of C's previous contents; beta == 0 does not read C
 *                 (it may hold anything, NaN included)
 *   bias          device pointer to N floats, bias[j] added to every element of column j;
 *                 NULL: none
 *   activation    GEMM_ACT_NONE; GEMM_ACT_RELU max(x, 0); GEMM_ACT_GELU x * Phi(x), Phi the
 *                 standard normal distribution function (the erf form), applied last
 *   out_type      GEMM_OUT_F32: C is float; GEMM_OUT_BF16: C holds bf16 bit patterns
 *                 (uint16_t), rounded to nearest even from the FP32 result, ldc in elements */
typedef enum { GEMM_ACT_NONE = 0, GEMM_ACT_RELU = 1, GEMM_ACT_GELU = 2 } gemm_activation_t;
typedef enum { GEMM_OUT_F32 = 0, GEMM_OUT_BF16 = 1 } gemm_out_t;
typedef struct {
    float alpha;
    float beta;
    const float *bias;
    gemm_activation_t activation;
    gemm_out_t out_type;
} gemm_epilogue_t;

/* gemm_bf16_f32acc_fused / gemm_f16_f32acc_fused: C = epilogue(A.B) for bf16 or fp16 inputs,
 * FP32 products and sums.  C is `void *` (float or uint16_t per out_type); the rest as the plain
 * calls.  The epilogue runs in the 16-bit direct-copy kernel: row-major A with column-major B (a
 * PyTorch Linear: x . W^T) or with row-major B and N % 8 == 0 (x . W), and K >= 64 (K == 0
 * gives act(beta * C + bias)).  A core launch plus at most two edge strips on the same stream, all on
 * that kernel; nothing is allocated.  An identity epilogue (alpha 1, beta 0, no bias or
 * activation, FP32 C) runs the plain kernel on the same plan.
 * gemm_f32_fused: the same for FP32 inputs on the FP32 direct-copy kernel: row-major A with
 * column-major B, K >= 32; an identity epilogue is gemm_f32.
 * Errors: as the plain calls, plus GEMM_ERR_INVALID_VALUE for a NULL epilogue, an unknown
 * activation or output type, a bias not 4-byte aligned, a C not aligned to its output element,
 * or operands the direct-copy kernels do not take (other orders, row-major B with N % 8 != 0
 * for 16-bit inputs, 0 < K < 64 for 16-bit inputs, 0 < K < 32 for FP32 ones). */
gemm_status_t gemm_bf16_f32acc_fused(int64_t M, int64_t N, int64_t K,
                                     const uint16_t *A, int64_t lda, gemm_order_t order_a,
                                     const uint16_t *B, int64_t ldb, gemm_order_t order_b,
                                     void *C, int64_t ldc, gemm_order_t order_c,
                                     const gemm_epilogue_t *epilogue, hipStream_t stream);
gemm_status_t gemm_f16_f32acc_fused(int64_t M, int64_t N, int64_t K,
                                    const uint16_t *A, int64_t lda, gemm_order_t order_a,
                                    const uint16_t *B, int64_t ldb, gemm_order_t order_b,
                                    void *C, int64_t ldc, gemm_order_t order_c,
                                    const gemm_epilogue_t *epilogue, hipStream_t stream);
gemm_status_t gemm_f32_fused(int64_t M, int64_t N, int64_t K,
                             const float *A, int64_t lda, gemm_order_t order_a,
                             const float *B, int64_t ldb, gemm_order_t order_b,
                             void *C, int64_t ldc, gemm_order_t order_c,
                             const gemm_epilogue_t *epilogue, hipStream_t stream);

/* ---- Without any allocation: split-K partial sums in a static scratch array ---------------
 * For callers that cannot allocate device memory or pass a workspace: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * gemm_bf16_f32acc_noalloc: as gemm_bf16_f32acc_ws (same kernels, same split-K choice, same
 * results bit for bit), with the workspace replaced by a fixed array of
 * GEMM_NOALLOC_SCRATCH_BYTES bytes in device memory that the library holds on every GPU it
 * runs on until the process ends.  The call allocates nothing (no hipMalloc, no library
 * allocation); its first call on a device looks the array's address up once.  A problem whose
 * partial sums would need more than GEMM_NOALLOC_SCRATCH_BYTES (gemm_workspace_size(1, ...))
 * is refused with GEMM_ERR_SCRATCH_TOO_SMALL before anything is enqueued.  Every call on one
 * GPU uses that GPU's one array, which keeps the last call's contents (every value a call reads
 * from it is written earlier in the same call): calls that may overlap on one GPU -- on two
 * streams, or from two threads -- race and must be serialised by the caller.
 * Errors: as gemm_bf16_f32acc, plus GEMM_ERR_SCRATCH_TOO_SMALL, and GEMM_ERR_LAUNCH if the
 * array's address cannot be obtained on the current device. */
#define GEMM_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
gemm_status_t gemm_bf16_f32acc_noalloc(int64_t M, int64_t N, int64_t K,
                                       const uint16_t *A, int64_t lda, gemm_order_t order_a,
                                       const uint16_t *B, int64_t ldb, gemm_order_t order_b,
                                       float *C, int64_t ldc, gemm_order_t order_c,
                                       hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBGEMM_GEMM_H */
