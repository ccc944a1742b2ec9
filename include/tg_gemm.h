/*
 * tg_gemm -- tiled dense matrix multiply C = A * B on AMD Instinct MI355X
 * (gfx950), with fp32 accumulation.
 *
 * The operation is the one the pages build their tiled kernels around:
 * "Getting to know TileLang", first-GEMM section: fp16 operands, an fp32
 * fragment accumulator that is cleared, accumulated over the K loop and copied
 * (with a cast to the output type) into C once; "TileKernels deep dive",
 * section 3.1: the 128-tile loop computing C tile += A tile * B tile over K;
 * section 2.1: element addressing through per-dimension strides (stride_am,
 * stride_ak, stride_bk, stride_bn, stride_cm, stride_cn).  The same pages list
 * FP8 GEMM and block-scaled GEMM among TileLang's examples ("Getting to know
 * TileLang", operator-coverage section) and quantise to E4M3 with
 * scale = amax / 448 ("TileKernels deep dive", sections 4.3 and 7.2).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Matrices are addressed with ELEMENT strides:
 *      A[i,k] = A + i*sam + k*sak      (i < M, k < K)
 *      B[k,j] = B + k*sbk + j*sbn      (k < K, j < N)
 *      C[i,j] = C + i*scm + j*scn      (i < M, j < N)
 *    "B stored N x K" (each column of B contiguous) is sbk = 1, sbn = ldb;
 *    "B stored K x N row-major" is sbk = ldb, sbn = 1.
 *  - C = A * B overwrites C (no alpha/beta).  Accumulation is fp32; the result
 *    is rounded once to the output type, round-to-nearest-even.
 *  - A, B, C (and scales) are DEVICE pointers owned by the caller; they must
 *    stay valid until the work enqueued on `stream` has completed.
 *  - These entry points allocate nothing, keep no state between calls and
 *    never synchronise: each call validates its arguments on the host,
 *    enqueues one kernel on `stream` and returns.  They are reentrant and
 *    may be captured into HIP graphs.  Products that would run faster with
 *    K split across workgroups (M <= 64, grids that fill few CUs, a partial
 *    last wave) run allocation-free plans here; the *_ws entry points below
 *    take a caller-owned workspace for the split plans.
 *  - C must not overlap A, B or the scales (undefined behaviour otherwise).
 *
 * Errors (tg_status)
 * ------------------
 *  - Arguments are validated on the host BEFORE any HIP call; a failed
 *    validation has no side effects.
 *      TG_ERR_INVALID_VALUE: a negative dimension or stride, a NULL pointer for
 *        an operand with a non-empty extent, C rows that overlap (M > 1 and
 *        scm < N), or an address range that overflows 64-bit arithmetic.
 *      TG_ERR_UNSUPPORTED: scn != 1 (C must have unit stride along n), or a
 *        dimension of 2^31 or more.
 *  - M == 0 or N == 0 is a successful no-op.  K == 0 writes zeros to C.
 *  - TG_ERR_LAUNCH: the kernel launch failed (hipGetLastError after launch);
 *    asynchronous faults surface on the stream as usual for HIP.
 *  - Every valid call is computed: shapes, strides or alignments that the
 *    tuned kernels do not take go to a general masked kernel.
 */
#ifndef TG_GEMM_H
#define TG_GEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int tg_status;
enum {
  TG_SUCCESS = 0,
  TG_ERR_INVALID_VALUE = 1,
  TG_ERR_UNSUPPORTED = 2,
  TG_ERR_LAUNCH = 3,
  TG_ERR_SCRATCH_LIMIT = 4
};

/* A hipStream_t, passed as an opaque pointer; NULL = the null stream. */
typedef void* tg_stream_t;

/* Static, NUL-terminated description of a status code. */
const char* tg_status_string(tg_status s);

/* C = A * B with IEEE fp16 (binary16) A, B and C, fp32 accumulation.
 * The first-GEMM listing of "Getting to know TileLang" (fp16 in, float32
 * accumulator, fp16 out). */
tg_status tg_gemm_f16(int64_t M, int64_t N, int64_t K,
                      const void* A, int64_t sam, int64_t sak,
                      const void* B, int64_t sbk, int64_t sbn,
                      void* C, int64_t scm, int64_t scn, tg_stream_t stream);

/* C = A * B with bfloat16 A, B and C, fp32 accumulation.  Same contract as
 * tg_gemm_f16; bf16 is the type of the 4096 x 7168 x 16384 GEMM reported for
 * the Ascend release in "Getting to know TileLang" (six-piece section). */
tg_status tg_gemm_bf16(int64_t M, int64_t N, int64_t K,
                       const void* A, int64_t sam, int64_t sak,
                       const void* B, int64_t sbk, int64_t sbn,
                       void* C, int64_t scm, int64_t scn, tg_stream_t stream);

/* Block-scaled fp8 product with bfloat16 output:
 *   C[i,j] = sum_k (e4m3(A[i,k]) * SA[i, k/128]) * (e4m3(B[k,j]) * SB[j/128, k/128])
 * A and B hold OCP E4M3FN codes (1 byte; bias 7, max 448, no infinities),
 * the format of "TileKernels deep dive" section 4.3.  Scales are fp32, one per
 * 1 x 128 slice of each A row and one per 128 x 128 block of B (a block-scaled
 * GEMM as listed in "Getting to know TileLang", operator-coverage section),
 * addressed with element strides:
 *   SA[i, kb]  = SA + i*ssam + kb*ssak      (kb < ceil(K/128))
 *   SB[jb, kb] = SB + jb*ssbn + kb*ssbk     (jb < ceil(N/128))
 * A trailing partial block (K or N not a multiple of 128) has its own scale.
 * Within each 128-wide k block the code products are summed in fp32 and the
 * block sum is scaled by SA * SB into the fp32 accumulator; C is rounded once
 * to bf16 (nearest-even).  Errors as above; SA / SB are checked like A / B. */
tg_status tg_gemm_fp8_blockscaled(int64_t M, int64_t N, int64_t K,
                                  const void* A, int64_t sam, int64_t sak,
                                  const float* SA, int64_t ssam, int64_t ssak,
                                  const void* B, int64_t sbk, int64_t sbn,
                                  const float* SB, int64_t ssbn, int64_t ssbk,
                                  void* C, int64_t scm, int64_t scn, tg_stream_t stream);

/* The same products with a caller-owned workspace, for the plans that split
 * K across the workgroups of an output tile and add their fp32 partial
 * tiles in split order (deterministic): products with M <= 64 (64 x 128
 * strips of C, K split so that there is about one workgroup per CU -- where
 * that beats 32-column strips over all of K: a long K run per strip, or a
 * strip grid that fills at most half the CUs), grids
 * of output tiles that would fill at most half the CUs (one GPU's share of
 * a larger product, e.g. 4096 x 896 x 16384: 256 x 224 tiles, K split 4
 * ways), and grids of one whole wave of 256 x 224 tiles and a partial one
 * (the partial wave's tiles split).  The split is the K loop of
 * "TileKernels deep dive" section 3.1 cut into ranges whose tile sums are
 * added at the end.
 *   workspace:  device buffer of workspace_bytes bytes, 256-byte aligned,
 *               owned by the caller.  Its first 16 KiB hold completion
 *               counters that must be ZERO before the buffer's first use
 *               (e.g. allocate it with torch.zeros); every call leaves them
 *               zero again when its kernel completes.  The rest holds fp32
 *               partial tiles.  Calls whose work overlaps in time must not
 *               share a workspace (different streams, or graph replays that
 *               may run concurrently): they would race on the counters and
 *               partials.  It must not overlap A, B or C.
 *   workspace_bytes: 0 (no workspace: the call runs exactly as tg_gemm_f16
 *               / tg_gemm_bf16), or the buffer's size.  A call whose split
 *               plan needs more than workspace_bytes (tg_gemm_workspace_size)
 *               runs the allocation-free plan instead; it never fails for
 *               lack of workspace.
 * Results: within the same bound as the allocation-free plans, and bit for
 * bit equal to them when every fp32 partial sum is exact (integer inputs).
 * Errors: those of tg_gemm_f16, plus TG_ERR_INVALID_VALUE for
 * workspace_bytes > 0 with a NULL or not 256-byte aligned workspace.
 * Nothing is allocated; asynchronous on `stream`. */
tg_status tg_gemm_f16_ws(int64_t M, int64_t N, int64_t K,
                         const void* A, int64_t sam, int64_t sak,
                         const void* B, int64_t sbk, int64_t sbn,
                         void* C, int64_t scm, int64_t scn,
                         void* workspace, size_t workspace_bytes, tg_stream_t stream);
tg_status tg_gemm_bf16_ws(int64_t M, int64_t N, int64_t K,
                          const void* A, int64_t sam, int64_t sak,
                          const void* B, int64_t sbk, int64_t sbn,
                          void* C, int64_t scm, int64_t scn,
                          void* workspace, size_t workspace_bytes, tg_stream_t stream);

/* tg_gemm_fp8_blockscaled with a caller-owned workspace (same contract as
 * the 16-bit *_ws calls above).  Its split plan is for M <= 64 (a decode
 * step over fp8 weights): 64 x 128 strips of C, the K blocks split so that
 * there is about one workgroup per CU, each split's block sums folded in
 * with SA * SB as in tg_gemm_fp8_blockscaled and the fp32 partial tiles
 * added in split order.  It runs for M > 32 where it beats the strips (a
 * long K run per strip, or a strip grid of at most half the CUs with K of at
 * least 56 blocks); tg_gemm_workspace_size is 0 elsewhere.  Without workspace (or too little) it runs exactly
 * as tg_gemm_fp8_blockscaled.  Results: within the same bound, bit for bit
 * equal when every fp32 partial sum is exact.  Errors: those of
 * tg_gemm_fp8_blockscaled, plus TG_ERR_INVALID_VALUE for workspace_bytes > 0
 * with a NULL or not 256-byte aligned workspace.  Nothing is allocated;
 * asynchronous on `stream`. */
tg_status tg_gemm_fp8_blockscaled_ws(int64_t M, int64_t N, int64_t K,
                                     const void* A, int64_t sam, int64_t sak,
                                     const float* SA, int64_t ssam, int64_t ssak,
                                     const void* B, int64_t sbk, int64_t sbn,
                                     const float* SB, int64_t ssbn, int64_t ssbk,
                                     void* C, int64_t scm, int64_t scn,
                                     void* workspace, size_t workspace_bytes,
                                     tg_stream_t stream);

/* Workspace bytes the split plan of a call with these arguments uses (0: the
 * call has no split plan, so a workspace changes nothing).  op: 0 = f16,
 * 1 = bf16, 2 = fp8 block-scaled (scale pointers and strides do not change
 * the plan and are not taken).  Host only: no HIP call.
 * Errors: TG_ERR_INVALID_VALUE for a NULL `bytes`, an unknown op, or
 * arguments the product would reject (the same validation). */
tg_status tg_gemm_workspace_size(int op, int64_t M, int64_t N, int64_t K,
                                 const void* A, int64_t sam, int64_t sak,
                                 const void* B, int64_t sbk, int64_t sbn,
                                 void* C, int64_t scm, int64_t scn, size_t* bytes);

/* For callers that cannot allocate device memory at all (code under HIP
 * graph capture that may not create buffers, tight serving loops, harnesses
 * that forbid allocation): tg_gemm_bf16_ws with its workspace taken from a
 * fixed 64 MiB device array inside the library instead of a caller's
 * buffer.  Same arguments, plans and results as tg_gemm_bf16_ws given 64 MiB
 * of workspace (that covers every split plan of the skinny and tile kernels
 * except partial-wave splits of many tiles).  The array is a file-scope
 * device variable: each GPU the library runs on holds its own copy until the
 * process ends; the first call on a device looks up that copy's address and
 * clears its counters (a small kernel on `stream`).  Every call on one GPU
 * shares that GPU's array: calls whose work may overlap in time on one GPU
 * (different streams, concurrent graph replays) race on it and give
 * undefined results.  Nothing is allocated.  Errors: those of
 * tg_gemm_bf16_ws; TG_ERR_SCRATCH_LIMIT, with no side effects, when the
 * call's split plan needs more than 64 MiB (tg_gemm_workspace_size), and
 * TG_ERR_LAUNCH when the array's address cannot be had. */
tg_status tg_gemm_bf16_static_scratch(int64_t M, int64_t N, int64_t K,
                                      const void* A, int64_t sam, int64_t sak,
                                      const void* B, int64_t sbk, int64_t sbn,
                                      void* C, int64_t scm, int64_t scn, tg_stream_t stream);

/* Grouped product: G independent products sharing N and K, group g with its
 * own row count -- the grouped GEMM of the TileLang examples ("Getting to
 * know TileLang", operator-coverage section), as used for the experts of a
 * mixture-of-experts layer ("TileKernels deep dive", section 5).  For g < G:
 *   C[i, j] = sum_k A[i, k] * B_g[k, j]   for offsets[g] <= i < offsets[g+1]
 * A[i,k] at A + i*lda + k; B_g stored N x K: B_g[k,j] at B + g*sbg + j*ldb + k;
 * C[i,j] at C + i*ldc + j (elements; fp16 or bf16, fp32 accumulation, one
 * rounding, as for the single products).  `offsets` is a HOST array of G + 1
 * non-decreasing row indices (groups may be empty).  One launch covers all
 * groups when G <= 128, K % 8 == 0, lda, ldb, sbg are multiples of 8 and A,
 * B are 16-byte aligned; other calls run group by group through
 * tg_gemm_f16 / tg_gemm_bf16.  Errors: TG_ERR_INVALID_VALUE for negative
 * sizes or strides, decreasing offsets or offsets[0] < 0, NULL pointers for
 * non-empty extents, overlapping rows (more than one row of A or C with lda <
 * K or ldc < N, N > 1 with ldb < K) or overflowing address ranges; G == 0, no
 * rows or N == 0 is a no-op; K == 0 writes zeros.  C must not overlap A or
 * B.  Asynchronous on `stream`; nothing is allocated. */
tg_status tg_gemm_grouped_f16(int64_t G, const int64_t* offsets, int64_t N, int64_t K,
                              const void* A, int64_t lda, const void* B, int64_t ldb,
                              int64_t sbg, void* C, int64_t ldc, tg_stream_t stream);
tg_status tg_gemm_grouped_bf16(int64_t G, const int64_t* offsets, int64_t N, int64_t K,
                               const void* A, int64_t lda, const void* B, int64_t ldb,
                               int64_t sbg, void* C, int64_t ldc, tg_stream_t stream);

/* Grouped block-scaled fp8 product (e4m3fn codes, bf16 output) with the
 * scale conventions of tg_gemm_fp8_blockscaled: A's row scales follow A's
 * rows, SA[i, kb] at SA + i*ssam + kb*ssak; group g's B is B + g*sbg (stored
 * N x K, leading dimension ldb, codes are bytes) and its block scales are
 * SB_g[jb, kb] at SB + g*ssbg + jb*ssbn + kb*ssbk.  One launch covers all
 * groups when G <= 128 and every group's call would take the fp8 tile kernel
 * (K % 16 == 0, lda, ldb, sbg multiples of 16, A and B 16-byte aligned);
 * other calls run group by group through tg_gemm_fp8_blockscaled.  Errors
 * and no-ops as for the grouped fp16 / bf16 products (scale pointers and
 * strides checked like the codes'). */
tg_status tg_gemm_grouped_fp8_blockscaled(int64_t G, const int64_t* offsets, int64_t N,
                                          int64_t K, const void* A, int64_t lda,
                                          const float* SA, int64_t ssam, int64_t ssak,
                                          const void* B, int64_t ldb, int64_t sbg,
                                          const float* SB, int64_t ssbn, int64_t ssbk,
                                          int64_t ssbg, void* C, int64_t ldc,
                                          tg_stream_t stream);

/* How a grouped fp8 call would run: "grouped_tile_fp8_256x128" (one launch),
 * "per_group", "none" (no-op) or NULL (invalid arguments). */
const char* tg_gemm_grouped_fp8_plan(int64_t G, const int64_t* offsets, int64_t N, int64_t K,
                                     const void* A, int64_t lda, const float* SA, int64_t ssam,
                                     int64_t ssak, const void* B, int64_t ldb, int64_t sbg,
                                     const float* SB, int64_t ssbn, int64_t ssbk, int64_t ssbg,
                                     void* C, int64_t ldc);

/* How a grouped call would run: "grouped_tile_nt_256x224" or "_256x256" (one
 * launch), "per_group", "none" (no-op) or NULL (invalid arguments). */
const char* tg_gemm_grouped_plan(int64_t G, const int64_t* offsets, int64_t N, int64_t K,
                                 const void* A, int64_t lda, const void* B, int64_t ldb,
                                 int64_t sbg, void* C, int64_t ldc);

/* Block quantisation of fp32 to OCP E4M3FN codes with fp32 scales -- the
 * step that makes the operands of tg_gemm_fp8_blockscaled.  Per block the
 * scale is the absolute maximum over 448 and each code is x / scale cast to
 * E4M3 ("TileKernels deep dive", section 7.2, fused RMSNorm + FP8
 * quantisation; section 4.3, the E4M3 FN format):
 *   amax = max |x| over the block;  s = amax / 448, rounded to fp32;
 *   if s == 0 (an all-zero block, or amax / 448 underflows): s = 1 and every
 *     code of the block is 0;
 *   otherwise code = e4m3fn(clamp(x / s, -448, 448)), x / s the rounded fp32
 *     quotient, rounded to the nearest code with ties to the even fraction;
 *     the sign is kept (0x80 for -0 and for negatives that round to 0).
 * X (device, fp32): R x K, X[i,k] at X + i*ldx + k.  Q (device, bytes):
 * Q[i,k] at Q + i*ldq + k.  S (device, fp32): S[ib, kb] at S + ib*ssr +
 * kb*ssk, kb = k / 128 and
 *   tg_quant_fp8_1x128:   ib = i        (one scale per 1 x 128 row slice: the
 *                                        SA layout of the product),
 *   tg_quant_fp8_128x128: ib = i / 128  (one per 128 x 128 block: the SB
 *                                        layout for B stored N x K, R = N).
 * Blocks at the right and bottom edges cover what is left and have scales of
 * their own.  Inputs must be finite.  Errors: TG_ERR_INVALID_VALUE for a
 * negative size or stride, a NULL pointer when R, K > 0, rows that would
 * overlap (R > 1 and ldx < K or ldq < K), a zero scale stride along a
 * dimension with more than one block, or an address range that overflows;
 * TG_ERR_UNSUPPORTED for a grid beyond 2^31 workgroups; R == 0 or K == 0 is
 * a no-op.  Q and S must not overlap X or each other.  Asynchronous on
 * `stream`; nothing is allocated. */
tg_status tg_quant_fp8_1x128(int64_t R, int64_t K, const float* X, int64_t ldx,
                             void* Q, int64_t ldq, float* S, int64_t ssr, int64_t ssk,
                             tg_stream_t stream);
tg_status tg_quant_fp8_128x128(int64_t R, int64_t K, const float* X, int64_t ldx,
                               void* Q, int64_t ldq, float* S, int64_t ssr, int64_t ssk,
                               tg_stream_t stream);

/* Product with an fp8 output: C = A * B as tg_gemm_f16 / tg_gemm_bf16
 * compute it (fp32 accumulation), then each 1 x 128 row slice of the fp32
 * result quantised as tg_quant_fp8_1x128 quantises fp32 input, in the
 * product's own epilogue -- the fp32 values are not rounded to 16 bits first
 * and never reach memory.  Q and S are laid out as tg_gemm_fp8_blockscaled
 * takes its A operand and SA, so the output feeds the next block-scaled
 * product directly ("TileKernels deep dive", section 7.2: the fused kernel
 * that quantises its result to FP8, scale = row maximum over 448; and the
 * fused SwiGLU + FP8 example, which saves the wide result's write and read).
 * A, B: as for tg_gemm_f16 (device, element strides).  Q (device, bytes):
 * code of C[m,n] at Q + m*sqm + n.  S (device, fp32): scale of the slice of
 * columns 128j .. 128j+127 of row m at S + m*ssm + j*ssj, j < ceil(N / 128);
 * the last slice of a row covers the columns that are left.  Per slice:
 *   amax = max |C| over the slice;  s = amax / 448 rounded to fp32;
 *   s == 0: s = 1 and every code 0;  otherwise code = e4m3fn RNE of
 *   clamp(C / s, -448, 448) (the rounded fp32 quotient), sign kept.
 * Errors: those of tg_gemm_f16 with Q for C (sqm for scm, and sqm >= N when
 * M > 1); TG_ERR_INVALID_VALUE also for a negative scale stride, S == NULL
 * when M, N > 0, a zero scale stride along a dimension of more than one
 * slice, or a scale address range that overflows.  K == 0 gives zero codes
 * and scales of 1.  Q and S must not overlap A, B or each other.
 * Asynchronous on `stream`; nothing is allocated. */
tg_status tg_gemm_f16_quant_fp8(int64_t M, int64_t N, int64_t K,
                                const void* A, int64_t sam, int64_t sak,
                                const void* B, int64_t sbk, int64_t sbn,
                                void* Q, int64_t sqm, float* S, int64_t ssm, int64_t ssj,
                                tg_stream_t stream);
tg_status tg_gemm_bf16_quant_fp8(int64_t M, int64_t N, int64_t K,
                                 const void* A, int64_t sam, int64_t sak,
                                 const void* B, int64_t sbk, int64_t sbn,
                                 void* Q, int64_t sqm, float* S, int64_t ssm, int64_t ssj,
                                 tg_stream_t stream);

/* How a product with fp8 output would run: "tile_nt_256x256_q8" (B stored
 * N x K), "tile_nn_256x256_q8" (B stored K x N), "generic16_32x128_q8" (any
 * other call), "none" (no-op) or NULL (invalid arguments).  op: 0 = f16,
 * 1 = bf16. */
const char* tg_gemm_quant_fp8_plan(int op, int64_t M, int64_t N, int64_t K,
                                   const void* A, int64_t sam, int64_t sak,
                                   const void* B, int64_t sbk, int64_t sbn,
                                   void* Q, int64_t sqm, float* S, int64_t ssm, int64_t ssj);

/* Fused SwiGLU with an fp8 output: the gate product G = A * Bg and the up
 * product U = A * Bu of one input, combined as h = silu(g) * u with
 * silu(g) = g / (1 + e^-g), and each 1 x 128 row slice of h quantised as
 * tg_gemm_f16_quant_fp8 quantises C -- "TileKernels deep dive", section 4.3
 * (the SwiGLU result quantised straight to FP8 without a round trip through
 * a wide type) and section 7.2 (the FP8 quantisation's scale and cast).
 * Both products accumulate in fp32 as tg_gemm_f16 / tg_gemm_bf16 do; h is
 * formed in fp32 from the two accumulators (g * u / (1 + e^-g)); neither
 * product nor h reaches memory.  The output feeds the down projection as
 * the A operand (codes and SA) of tg_gemm_fp8_blockscaled.
 * A: as for tg_gemm_f16.  Bg, Bu (device): the gate and up weights,
 * K x N with the same strides, B[k,n] at B + k*sbk + n*sbn; the tiled kernel
 * takes them stored N x K (sbk = 1) as tg_gemm_f16 takes B.  Q, S: as for
 * tg_gemm_f16_quant_fp8 (code of h[m,n] at Q + m*sqm + n, scale of slice j
 * of row m at S + m*ssm + j*ssj).  Errors: those of tg_gemm_f16_quant_fp8
 * with Bg for B, and TG_ERR_INVALID_VALUE for Bu == NULL when M, N, K > 0.
 * K == 0 gives zero codes and scales of 1.  Q and S must not overlap the
 * inputs or each other.  Asynchronous on `stream`; nothing is allocated. */
tg_status tg_gemm_f16_swiglu_quant_fp8(int64_t M, int64_t N, int64_t K,
                                       const void* A, int64_t sam, int64_t sak,
                                       const void* Bg, const void* Bu, int64_t sbk, int64_t sbn,
                                       void* Q, int64_t sqm, float* S, int64_t ssm, int64_t ssj,
                                       tg_stream_t stream);
tg_status tg_gemm_bf16_swiglu_quant_fp8(int64_t M, int64_t N, int64_t K,
                                        const void* A, int64_t sam, int64_t sak,
                                        const void* Bg, const void* Bu, int64_t sbk, int64_t sbn,
                                        void* Q, int64_t sqm, float* S, int64_t ssm, int64_t ssj,
                                        tg_stream_t stream);

/* The fused SwiGLU with a caller-owned workspace (contract of
 * tg_gemm_f16_ws: 256-byte aligned, its first 16 KiB counters that must be
 * zero before first use and are left zero, no sharing between calls that
 * may overlap in time).  Its split plan is for M <= 64: the K slices of each
 * 128-column output slice are split over several workgroups, so that there
 * is about one workgroup per CU; the fp32 g and u partial sums are added in
 * split order before the activation, so h, the scales and the codes are
 * those of whole sums (bit for bit those of the call without a workspace
 * when every fp32 partial sum is exact).  Without workspace (or too little)
 * it runs exactly as tg_gemm_f16_swiglu_quant_fp8 / _bf16_.  Errors: those
 * of the call without a workspace, plus TG_ERR_INVALID_VALUE for
 * workspace_bytes > 0 with a NULL or not 256-byte aligned workspace.
 * Nothing is allocated; asynchronous on `stream`. */
tg_status tg_gemm_f16_swiglu_quant_fp8_ws(int64_t M, int64_t N, int64_t K,
                                          const void* A, int64_t sam, int64_t sak,
                                          const void* Bg, const void* Bu, int64_t sbk,
                                          int64_t sbn, void* Q, int64_t sqm, float* S,
                                          int64_t ssm, int64_t ssj, void* workspace,
                                          size_t workspace_bytes, tg_stream_t stream);
tg_status tg_gemm_bf16_swiglu_quant_fp8_ws(int64_t M, int64_t N, int64_t K,
                                           const void* A, int64_t sam, int64_t sak,
                                           const void* Bg, const void* Bu, int64_t sbk,
                                           int64_t sbn, void* Q, int64_t sqm, float* S,
                                           int64_t ssm, int64_t ssj, void* workspace,
                                           size_t workspace_bytes, tg_stream_t stream);

/* Workspace bytes the split plan of a fused SwiGLU call uses (0: no split
 * plan, so a workspace changes nothing).  op: 0 = f16, 1 = bf16.  Host only.
 * Errors: TG_ERR_INVALID_VALUE for a NULL `bytes`, an unknown op or
 * arguments the call would reject. */
tg_status tg_gemm_swiglu_quant_fp8_workspace_size(int op, int64_t M, int64_t N, int64_t K,
                                                  const void* A, int64_t sam, int64_t sak,
                                                  const void* Bg, const void* Bu, int64_t sbk,
                                                  int64_t sbn, void* Q, int64_t sqm, float* S,
                                                  int64_t ssm, int64_t ssj, size_t* bytes);

/* How a fused SwiGLU call would run: "skinny_64x128_swiglu_q8" (M <= 64,
 * both weights stored N x K: one workgroup per 128-column slice over the
 * whole of K), "skinny_64x128_swiglu_q8_splitkS" (the same with a workspace,
 * K split S ways), "tile_nt_256x256_swiglu_q8" (larger M, both weights
 * stored N x K and accepted by the N x K tile kernel),
 * "generic16_32x128_swiglu_q8" (any other call), "none" (no-op) or NULL
 * (invalid arguments).  op: 0 = f16, 1 = bf16.  tg_gemm_swiglu_quant_fp8_plan
 * names the plan without a workspace, tg_gemm_swiglu_quant_fp8_plan_ws with
 * one of workspace_bytes.  Host only. */
const char* tg_gemm_swiglu_quant_fp8_plan(int op, int64_t M, int64_t N, int64_t K,
                                          const void* A, int64_t sam, int64_t sak,
                                          const void* Bg, const void* Bu, int64_t sbk,
                                          int64_t sbn, void* Q, int64_t sqm, float* S,
                                          int64_t ssm, int64_t ssj);
const char* tg_gemm_swiglu_quant_fp8_plan_ws(int op, int64_t M, int64_t N, int64_t K,
                                             const void* A, int64_t sam, int64_t sak,
                                             const void* Bg, const void* Bu, int64_t sbk,
                                             int64_t sbn, void* Q, int64_t sqm, float* S,
                                             int64_t ssm, int64_t ssj, size_t workspace_bytes);

/* Name of the kernel a call with these arguments would launch ("none" for a
 * no-op, NULL if the arguments are invalid); nothing is launched.  op: 0 =
 * tg_gemm_f16, 1 = tg_gemm_bf16, 2 = tg_gemm_fp8_blockscaled (the scale
 * arguments do not affect the choice).  tg_gemm_plan names the plan of the
 * allocation-free entry points; tg_gemm_plan_ws the plan of
 * tg_gemm_f16_ws / tg_gemm_bf16_ws / tg_gemm_fp8_blockscaled_ws with a
 * workspace of workspace_bytes.  Host only.  For tests and benchmarks. */
const char* tg_gemm_plan(int op, int64_t M, int64_t N, int64_t K,
                         const void* A, int64_t sam, int64_t sak,
                         const void* B, int64_t sbk, int64_t sbn,
                         void* C, int64_t scm, int64_t scn);
const char* tg_gemm_plan_ws(int op, int64_t M, int64_t N, int64_t K,
                            const void* A, int64_t sam, int64_t sak,
                            const void* B, int64_t sbk, int64_t sbn,
                            void* C, int64_t scm, int64_t scn, size_t workspace_bytes);

#ifdef __cplusplus
}
#endif

#endif /* TG_GEMM_H */
