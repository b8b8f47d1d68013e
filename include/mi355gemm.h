/*
 * mi355gemm -- dense matrix multiply for AMD Instinct MI355X (gfx950).
 *
 * Public C ABI.  Plain pointers and sizes only.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All matrices are row-major.  Element (i, j) of X with leading dimension
 *    ldx sits at X[i*ldx + j].  Dimensions and leading dimensions are int;
 *    offsets are computed in 64 bits.
 *  - A, B and C are DEVICE pointers, allocated and owned by the caller.  The
 *    library never allocates, frees or keeps device memory, and keeps no
 *    pointer after a call returns; the one exception is the static scratch
 *    area of gemm_f16_nt_splitk_static, part of the library's code object
 *    (see there).  gemm_f32, gemm_f16_nt and gemm_f16_nt_ex
 *    need nothing beyond their operands.  The calls whose kernels need
 *    scratch memory take it from the caller as a `workspace` argument and
 *    say how much through a size query: gemm_f32_splitk / gemm_f16_nt_splitk
 *    (fp32 partial sums of the K ranges) and gemm_ex (transposed operand
 *    copies for smaller products in the other layouts, partial sums of the
 *    K-major matrix-vector kernel).
 *  - `stream` is a hipStream_t passed as void*; NULL means the default stream.
 *    Work is enqueued on it and the call returns without synchronising; a
 *    fault during execution surfaces at the caller's next synchronisation.
 *  - C must not overlap A or B (undefined otherwise).  A and B may alias.
 *  - Misaligned pointers or leading dimensions are never an error: they only
 *    select a slower kernel.
 *  - Calls are thread-safe: the library's only state is a per-device record,
 *    set once, that the device is a gfx950 (and, for
 *    gemm_f16_nt_splitk_static, the device address of its scratch area).
 *
 * Return value: GEMM_OK (0) or one of the negative GEMM_ERR_* codes below.
 * On an error no work is enqueued and C is untouched.
 */
#ifndef MI355GEMM_H
#define MI355GEMM_H

#ifdef __cplusplus
extern "C" {
#endif

#if defined(MI355GEMM_BUILDING)
#define MI355GEMM_API __attribute__((visibility("default")))
#else
#define MI355GEMM_API
#endif

enum {
  GEMM_OK = 0,
  GEMM_ERR_NEGATIVE_DIM = -1,      /* M, N or K < 0                                  */
  GEMM_ERR_BAD_LD = -2,            /* a leading dimension is too small               */
  GEMM_ERR_NULL_POINTER = -3,      /* NULL for an operand that would be read/written */
  GEMM_ERR_UNSUPPORTED_DEVICE = -4,/* no HIP device, or the current one is not gfx950 */
  GEMM_ERR_LAUNCH = -5,            /* the HIP runtime refused the kernel launch      */
  GEMM_ERR_BAD_ARG = -6,           /* an enumerated argument has no defined meaning  */
  GEMM_ERR_WORKSPACE = -7,         /* a workspace the call needs is NULL, smaller    */
                                   /*   than its size query, or not 16-byte aligned  */
  GEMM_ERR_SCRATCH_LIMIT = -8      /* gemm_f16_nt_splitk_static: the partial sums    */
                                   /*   need more than GEMM_STATIC_SCRATCH_BYTES     */
};

/*
 * fp32 SGEMM:  C = alpha * A * B + beta * C
 *
 * The operation of the cp.async SGEMM example on the page "异步拷贝与
 * Hopper/Blackwell 新特性" (section "cp.async 与多级流水"): every C[i][j]
 * becomes alpha times the dot product of row i of A with column j of B, plus
 * beta times its old value.  Page 1 ("第 6 章 Shared Memory & Tile", section
 * 6.1) fixes the row-major indexing.
 *
 *   A : float[M][lda], lda >= max(1, K)   (read)
 *   B : float[K][ldb], ldb >= max(1, N)   (read)
 *   C : float[M][ldc], ldc >= max(1, N)   (read if beta != 0, written)
 *
 * beta == 0 follows BLAS: C is then write-only and its old contents (NaN
 * included) never reach the result.  K == 0 or alpha == 0 gives C = beta * C
 * (C = 0 when beta == 0 too).  M == 0 or N == 0 is a no-op that accepts NULL
 * pointers.  The fp32 products are accumulated in fp32.
 */
MI355GEMM_API int gemm_f32(int M, int N, int K, float alpha,
                           const float* A, int lda,
                           const float* B, int ldb,
                           float beta, float* C, int ldc,
                           void* stream);

/*
 * fp16 "NT" GEMM:  C = A * B^T, fp32 accumulation, fp16 output.
 *
 * The product that the page "从零开始的 AI Infra: 算子基础与GPU架构" tunes,
 * as defined in its section "0. Naive Implementation": C[m][n] is the sum
 * over k of A[m][k] * B[n][k] accumulated in fp32 and rounded to half
 * (round to nearest, ties to even).  Section "19. 去掉转置" is the layout:
 * B is stored [N][K], so B[n][k] sits at n*ldb + k.
 *
 *   A : IEEE binary16 [M][lda], lda >= max(1, K)   (read)
 *   B : IEEE binary16 [N][ldb], ldb >= max(1, K)   (read)
 *   C : IEEE binary16 [M][ldc], ldc >= max(1, N)   (written only)
 *
 * K == 0 gives C = 0.  M == 0 or N == 0 is a no-op that accepts NULL
 * pointers.  Results overflow to +-inf like any fp32 -> fp16 conversion.
 */
MI355GEMM_API int gemm_f16_nt(int M, int N, int K,
                              const void* A, int lda,
                              const void* B, int ldb,
                              void* C, int ldc,
                              void* stream);

/*
 * fp16 "NT" GEMM with a fused write-back:
 *
 *     C = act(A * B^T + bias) + residual
 *
 * Page 1 ("第 6 章 Shared Memory & Tile", section 6.5.4, and exercise 6 of
 * section 6.9) folds the work that follows a GEMM into its write-back while
 * the accumulators are still in registers: the column's bias is added, the
 * sum goes through an activation, and (the page's attention-output case) the
 * residual stream is added, before the one store of C.  Here every output is
 *
 *     v = acc[i][j] + bias[j]          acc: the fp32 sum of gemm_f16_nt
 *     v = act(v)                       GEMM_ACT_NONE: v, GEMM_ACT_RELU:
 *                                      max(v, 0), GEMM_ACT_SILU: v / (1 + e^-v)
 *     C[i][j] = half(v + residual[i][j])
 *
 * evaluated in fp32 and rounded to half once (nearest, ties to even).  SiLU
 * uses the device's fast exponential.
 *
 *   A, B, C, lda, ldb, ldc : as for gemm_f16_nt
 *   bias     : IEEE binary16 [N] (read), or NULL for no bias
 *   act      : GEMM_ACT_NONE, GEMM_ACT_RELU or GEMM_ACT_SILU
 *   residual : IEEE binary16 [M][ldr], ldr >= max(1, N) (read), or NULL.
 *              It may be C itself (same pointer, ldr == ldc) for an in-place
 *              residual add; any other overlap with C is undefined.
 *
 * K == 0 gives C = act(bias) + residual.  M == 0 or N == 0 is a no-op.  An
 * unknown act is GEMM_ERR_BAD_ARG.
 */
enum { GEMM_ACT_NONE = 0, GEMM_ACT_RELU = 1, GEMM_ACT_SILU = 2 };

MI355GEMM_API int gemm_f16_nt_ex(int M, int N, int K,
                                 const void* A, int lda,
                                 const void* B, int ldb,
                                 const void* bias, int act,
                                 const void* residual, int ldr,
                                 void* C, int ldc,
                                 void* stream);

/*
 * Split-K with a caller-owned workspace.
 *
 * Page 1 ("第 6 章 Shared Memory & Tile", section 6.5.6) cuts the K dimension
 * of a product with few output tiles into ranges, computes each range's
 * partial sums in its own blocks and adds them afterwards.  Here the partial
 * sums of range s are fp32 tiles of 128 x 128 in the workspace, and a second
 * kernel adds the ranges in the fixed order 0, 1, ..., so results repeat
 * bitwise from run to run; the final write-back is the one of gemm_f32
 * (alpha * sum + beta * C) or of gemm_f16_nt (rounding to half).
 *
 *   M .. ldc, stream : as for gemm_f32 / gemm_f16_nt
 *   splits    : number of K ranges.  <= 0 lets the library choose: ranges
 *               only when K >= 2048 and the product has few output tiles of
 *               128 x 128 (16-bit: as many as keep tiles x ranges within 400
 *               workgroups, a power of two, at least 2, ranges at least 256
 *               deep; fp32: within 512, at least 3, at least 64 deep; at
 *               most 64), never for the matrix-vector shapes (M or N <= 8);
 *               1 never splits; larger values are cut to at most one range
 *               per 16 (fp32) or 64 (fp16) elements of K.  Without a split
 *               the call runs exactly as gemm_f32 / gemm_f16_nt.
 *   workspace : device memory, 16-byte aligned, of at least
 *               workspace_bytes >= gemm_*_splitk_workspace(M, N, K, splits)
 *               bytes; written and read by the call's kernels on `stream`,
 *               so it must not be in use by other work until they finish.
 *               May be NULL when that size is 0.
 *
 * Returns GEMM_ERR_WORKSPACE if a split is chosen and the workspace is NULL,
 * too small or misaligned; otherwise as gemm_f32 / gemm_f16_nt.
 */
MI355GEMM_API int gemm_f32_splitk(int M, int N, int K, float alpha,
                                  const float* A, int lda,
                                  const float* B, int ldb,
                                  float beta, float* C, int ldc,
                                  int splits, void* workspace,
                                  unsigned long long workspace_bytes,
                                  void* stream);

MI355GEMM_API int gemm_f16_nt_splitk(int M, int N, int K,
                                     const void* A, int lda,
                                     const void* B, int ldb,
                                     void* C, int ldc,
                                     int splits, void* workspace,
                                     unsigned long long workspace_bytes,
                                     void* stream);

/* Workspace bytes the calls above need for these sizes and `splits`; 0 when
 * they would not split (negative M, N, K or splits count as no split). */
MI355GEMM_API unsigned long long gemm_f32_splitk_workspace(int M, int N, int K, int splits);
MI355GEMM_API unsigned long long gemm_f16_nt_splitk_workspace(int M, int N, int K, int splits);

/*
 * gemm_f16_nt_splitk for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  It takes no workspace and allocates nothing; the fp32 partial
 * sums go to a static scratch area of GEMM_STATIC_SCRATCH_BYTES (32 MiB) that
 * the library's code object holds on every GPU it runs on, until the process
 * ends.
 *
 *   arguments  : as gemm_f16_nt_splitk, without workspace / workspace_bytes
 *   limit      : a split whose partial sums need more than
 *                GEMM_STATIC_SCRATCH_BYTES (gemm_f16_nt_splitk_workspace for
 *                the same M, N, K, splits) returns GEMM_ERR_SCRATCH_LIMIT
 *                before any work is enqueued.  Without a split the call runs
 *                exactly as gemm_f16_nt and uses no scratch.
 *   sharing    : every call on one GPU uses that GPU's one scratch area, and
 *                the area keeps the last call's partial sums.  Calls that
 *                overlap in time on one GPU (other streams, other host
 *                threads, replays of graphs on other streams) race on it:
 *                the caller must order them, e.g. on one stream.
 *
 * Results are bit for bit those of gemm_f16_nt_splitk with the same splits.
 */
#define GEMM_STATIC_SCRATCH_BYTES (32ull << 20)
MI355GEMM_API int gemm_f16_nt_splitk_static(int M, int N, int K,
                                            const void* A, int lda,
                                            const void* B, int ldb,
                                            void* C, int ldc,
                                            int splits, void* stream);

/*
 * 16-bit GEMM in any operand layout, fp16 or bf16, with the fused write-back:
 *
 *     C = act(op(A) * op(B) + bias) + residual
 *
 * Page 1 ("第 6 章 Shared Memory & Tile", section 6.3.3) drives the matrix
 * units through the library GEMM with a storage type (fp16 or bf16) and an
 * operation per operand; the NT page ("从零开始的 AI Infra: 算子基础与GPU架构",
 * section "19. 去掉转置") compares B stored [n][k] with its transpose stored
 * [k][n].  Here, all row-major:
 *
 *   type : GEMM_TYPE_F16 (IEEE binary16) or GEMM_TYPE_BF16 (bfloat16); A, B,
 *          C, bias and residual are all of this type.  Products accumulate
 *          in fp32; each output is rounded once to the type (nearest, ties
 *          to even).
 *   op_a : GEMM_OP_N: A is [M][lda], lda >= max(1, K), op(A) = A.
 *          GEMM_OP_T: A is [K][lda], lda >= max(1, M), op(A) = A^T.
 *   op_b : GEMM_OP_N: B is [K][ldb], ldb >= max(1, N), op(B) = B.
 *          GEMM_OP_T: B is [N][ldb], ldb >= max(1, K), op(B) = B^T.
 *   bias, act, residual, ldr, C, ldc : as for gemm_f16_nt_ex (bias NULL,
 *          GEMM_ACT_NONE and residual NULL give the plain product).
 *
 * (GEMM_TYPE_F16, GEMM_OP_N, GEMM_OP_T) is exactly gemm_f16_nt_ex.  NN
 * (B stored [K][N]), TT (A stored [K][M]) and TN (both) with A and B
 * 16-byte aligned and lda, ldb multiples of 8 read the K-major operands in
 * place, with no workspace: on whole tiles with K % 64 == 0 (256 x 256 for NN
 * and TT, 224 x 256 for NN or 256 x 224 for TT and TN, 128 x 128 or
 * 128 x 192; C 16-byte aligned, ldc a multiple of 8), or, for products of at
 * least 2^30 multiply-adds at least 128 wide and tall with K > 64 (and
 * K % 8 == 0 for NN and TT), on their ragged form (C anywhere) -- unless the
 * A * B^T tiles on transposed copies would take fewer rounds of the GPU (NN
 * 4096 x 3584, for one) (the NT page, section 19: the kernel consumes B
 * in its stored layout instead of transposing it first).  The other layouts
 * and shapes first copy each operand that is not K-contiguous (A for OP_T, B
 * for OP_N) into the workspace, transposed, then run the A * B^T kernels -- except on
 * the matrix-vector path (M <= 8 or N <= 8), where a long operand stored
 * K-major (B for OP_N when M is the small side, A for OP_T when N is) is read
 * in place, row by row, and the short one in either layout: its ranges of K
 * leave fp32 partial sums in the workspace and the split-K reduction adds
 * them in order.  A product of few output tiles and long K (the rule of
 * gemm_f16_nt_splitk's splits <= 0) is split into ranges of K -- on the
 * transposed copies in the other layouts -- with the fused write-back applied
 * by the ordered reduction, when the workspace also holds the ranges' fp32
 * partial sums; with a smaller one it runs unsplit.
 *
 *   workspace       : device memory, 16-byte aligned, of at least
 *                     gemm_ex_workspace(...) bytes for the same arguments
 *                     (written and read by the call's kernels on `stream`, so
 *                     not in use by other work until they finish); may be
 *                     NULL when that size is 0.
 *   workspace_bytes : its size.
 *
 * Unknown type, op or act values are GEMM_ERR_BAD_ARG; a workspace the call
 * needs that is NULL, too small or misaligned is GEMM_ERR_WORKSPACE (checked
 * before any work is enqueued).
 */
enum { GEMM_TYPE_F16 = 0, GEMM_TYPE_BF16 = 1 };
enum { GEMM_OP_N = 0, GEMM_OP_T = 1 };

MI355GEMM_API int gemm_ex(int type, int op_a, int op_b, int M, int N, int K,
                          const void* A, int lda,
                          const void* B, int ldb,
                          const void* bias, int act,
                          const void* residual, int ldr,
                          void* C, int ldc,
                          void* workspace, unsigned long long workspace_bytes,
                          void* stream);

/* Workspace bytes gemm_ex uses for these sizes, layouts and leading
 * dimensions, split-K partial sums included (0 when none, or for arguments
 * gemm_ex rejects).  Without the split-K part gemm_ex runs unsplit and needs
 * only the rest.  The figure holds for any pointers: for NN, TT and TN it
 * counts the transposed copies, which the calls that read the operand in place (see
 * gemm_ex) do not use -- they accept a NULL workspace. */
MI355GEMM_API unsigned long long gemm_ex_workspace(int type, int op_a, int op_b, int M, int N,
                                                   int K, int lda, int ldb);

/* A static, human-readable message for a GEMM_* status code. */
MI355GEMM_API const char* gemm_status_string(int status);

/*
 * Kernel selection, exposed for inspection and testing.  These are pure host
 * functions: they make no HIP call and never touch the pointed-to memory
 * (the pointers are only checked for alignment).  They return the GEMM_PATH_*
 * value that gemm_f32 / gemm_f16_nt / gemm_f16_nt_ex / gemm_ex would launch
 * for the same arguments, or a
 * negative GEMM_ERR_* code for arguments those calls would reject (a device
 * check excepted).
 *
 * The environment variable MI355GEMM_FORCE_PATH=general, read at every call,
 * forces the general kernels even where a fast path applies.
 */
enum {
  GEMM_PATH_NOOP = 0,           /* M == 0 or N == 0: nothing is launched          */
  GEMM_PATH_F32_SCALE = 1,      /* K == 0 or alpha == 0: C = beta * C             */
  GEMM_PATH_F32_GENERAL = 2,    /* v_mfma f32 tiles with predicated loads/stores: */
                                /*   any shape, leading dimension and alignment   */
                                /*   (16-byte aligned rows, K % 4 == 0, M, N >=   */
                                /*   128: streaming tiles with shifted edges)     */
  GEMM_PATH_F32_MFMA = 3,       /* v_mfma f32 full tiles, 16-byte aligned rows    */
  GEMM_PATH_F16_ZERO = 4,       /* K == 0: C = 0                                  */
  GEMM_PATH_F16_GENERAL = 5,    /* v_mfma f16 tiles with predicated loads/stores: */
                                /*   any shape, leading dimension and alignment   */
  GEMM_PATH_F16_MFMA = 6,       /* v_mfma f16 full tiles, 16-byte aligned rows    */
                                /*   (large ragged products with A and B rows at  */
                                /*   16-byte addresses and K % 8 == 0: shifted    */
                                /*   edge tiles, C anywhere; few output tiles:    */
                                /*   32 x 32 tiles, K split across the waves)     */
  GEMM_PATH_F16_GEMV = 7,       /* M <= 8 or N <= 8: matrix-vector kernel that    */
                                /*   streams the long operand once (any ld/align) */
  GEMM_PATH_F16_SPLITK = 8,     /* gemm_ex only, long K over few output tiles: K   */
                                /*   cut into ranges, fp32 partial sums in the    */
                                /*   workspace, ordered reduction                 */
  /* 9 is not used */
  GEMM_PATH_F16_STAGED = 10     /* large ragged or unaligned products: v_mfma     */
                                /*   wide tiles with register-staged loads (any   */
                                /*   shape, leading dimension, 2-byte alignment), */
                                /*   masked stores; the operands read in place    */
                                /*   (gemm_ex: after any transposed copy)         */
};

MI355GEMM_API int gemm_f32_path(int M, int N, int K, float alpha,
                                const float* A, int lda,
                                const float* B, int ldb,
                                float beta, const float* C, int ldc);

MI355GEMM_API int gemm_f16_nt_path(int M, int N, int K,
                                   const void* A, int lda,
                                   const void* B, int ldb,
                                   const void* C, int ldc);

MI355GEMM_API int gemm_f16_nt_ex_path(int M, int N, int K,
                                      const void* A, int lda,
                                      const void* B, int ldb,
                                      const void* bias, int act,
                                      const void* residual, int ldr,
                                      const void* C, int ldc);

/* For gemm_ex: the path of the kernels that run (after the transposed copies
 * of a smaller product in another layout, which are 16-byte aligned with rows
 * padded to a multiple of 8 elements). */
MI355GEMM_API int gemm_ex_path(int type, int op_a, int op_b, int M, int N, int K,
                               const void* A, int lda,
                               const void* B, int ldb,
                               const void* bias, int act,
                               const void* residual, int ldr,
                               const void* C, int ldc);

/* A static name for a GEMM_PATH_* value ("f32_mfma", ...); "?" if unknown. */
MI355GEMM_API const char* gemm_path_name(int path);

#ifdef __cplusplus
}
#endif

#endif /* MI355GEMM_H */
