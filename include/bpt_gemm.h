/*
 * bpt_gemm.h -- C ABI of the MI355X (gfx950) pipelined half-precision GEMM.
 *
 * Operation (every entry point): C <- A * B, overwriting C, with
 *     C[i][j] = sum_{k=0}^{K-1} A[i][k] * B[k][j]
 * accumulated in fp32 on the matrix cores.  This is the tiled FP16 GEMM of
 * the "Xe2 ESIMD GEMM" page (its B_T[K,N] layout: B is K rows of N, row
 * major), rebuilt for CDNA4: K-tiles are staged global->LDS by LDS-DMA in a
 * ring of stages, published to the workgroup by a vmcnt wait plus one
 * s_barrier (the gfx950 form of the split arrive/wait barrier of the
 * "Xe2 Nbarrier Pipelining" page), and consumed by v_mfma_f32_32x32x16.
 * There is no alpha/beta.
 *
 * Layout: all matrices are row major.  A is M x K with leading dimension lda
 * (elements between the starts of consecutive rows, lda >= max(1, K)); B is
 * K x N with ldb >= max(1, N); C is M x N with ldc >= max(1, N).  Batch
 * strides are in elements.
 *
 * Element types: gemm_f16 / gemm_batched_f16 read IEEE binary16, gemm_bf16
 * reads bfloat16.  out_fp32 = 0 writes C in the input type (rounded to
 * nearest even from the fp32 sum); out_fp32 = 1 writes fp32.
 *
 * Ownership: A, B and C are DEVICE pointers owned by the caller.  C must not
 * overlap A or B.  The library keeps no per-call state; its one allocation is
 * a workspace used by three paths:
 *   - the split-K path for few rows of A (variants
 *     skinny_64x128_ring_k32_s4_splitk and skinny_64x128_w4_k32_s4_splitk
 *     when they split K over workgroups) keeps fp32 partial results there
 *     (at most 256 MiB);
 *   - the split-K path for few output tiles (variant splitk_pipelined: one
 *     matrix, more than 128 rows, at most 128 tiles of 128 x 128, N a
 *     multiple of 8, B in either layout) keeps the
 *     fp32 partial products of its 2 to 64 K ranges there (at most
 *     256 MiB);
 *   - the repack path (variant repack_pipelined: shapes the pipelined kernels
 *     cannot read in place -- K or N not a multiple of 8, leading dimensions,
 *     batch strides or bases not 16-byte granular -- with at least 2^24
 *     multiply-adds) copies A and/or B there, zero-padded and aligned
 *     (at most 1 GiB).
 * The buffers come from a pool per device.  Each carries an event recorded
 * on the caller's stream after the last kernel that used it, and a call
 * taking a buffer whose event has not completed first makes its stream wait
 * for it (hipStreamWaitEvent), whatever the stream handles: calls on
 * different streams -- hipStreamPerThread from several threads, a new
 * stream that got a destroyed one's handle -- never use a buffer at the same
 * time.  A buffer is allocated with hipMalloc only when no pooled one is
 * free and large enough (the first such call on a device, a call needing
 * more than before, calls in flight on more streams than the pool's 4
 * buffers); a grown-out buffer is kept until the process exits (hipFree
 * would synchronise the device).  A call made while its stream is being
 * captured into a graph, or one whose allocation fails, takes a path
 * without workspace (the skinny or pipelined kernel unsplit, the guarded
 * kernel instead of the repack) -- so a captured graph never refers to a
 * pooled buffer.
 *
 * Execution: the call validates its arguments on the host, enqueues the
 * kernel(s) on `stream` (NULL = the default stream) and returns without
 * waiting.  Completion is observed by synchronising the stream.  The split-K
 * path enqueues two kernels (the K-split products, then the in-order sum of
 * their fp32 partials), the repack path up to three (the copies of A and/or
 * B, then the product).
 *
 * Errors: nothing is launched unless the status is BPT_OK.
 *   BPT_ERR_INVALID_ARG  a size or stride is negative, a leading dimension is
 *                        too small, out_fp32 is not 0/1, or a pointer of a
 *                        non-empty operand is NULL;
 *   BPT_ERR_UNSUPPORTED  a dimension or leading dimension does not fit in 31
 *                        bits, or a forced variant cannot take the call;
 *   BPT_ERR_HIP          the HIP runtime reported an error at launch.
 * bpt_last_error() returns a message for the last failing call on the
 * calling thread.
 *
 * Degenerate shapes: M == 0, N == 0 or batch == 0 returns BPT_OK and
 * launches nothing; K == 0 writes zeros to C (the empty sum).
 */
#ifndef BPT_GEMM_H
#define BPT_GEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t; /* hipStream_t == struct ihipStream_t* */

typedef enum {
    BPT_OK = 0,
    BPT_ERR_INVALID_ARG = 1,
    BPT_ERR_UNSUPPORTED = 2,
    BPT_ERR_HIP = 3
} bpt_status;

/* fp16 GEMM, C (M x N) = A (M x K) * B (K x N); C is fp16 or fp32. */
bpt_status gemm_f16(int64_t M, int64_t N, int64_t K,
                    const void *A, int64_t lda,
                    const void *B, int64_t ldb,
                    void *C, int64_t ldc,
                    int out_fp32, struct ihipStream_t *stream);

/* bf16 GEMM; C is bf16 (out_fp32 = 0) or fp32 (out_fp32 = 1). */
bpt_status gemm_bf16(int64_t M, int64_t N, int64_t K,
                     const void *A, int64_t lda,
                     const void *B, int64_t ldb,
                     void *C, int64_t ldc,
                     int out_fp32, struct ihipStream_t *stream);

/* batch independent fp16 GEMMs; entry b uses A + b*strideA, B + b*strideB,
 * C + b*strideC (strides in elements, >= 0). */
bpt_status gemm_batched_f16(int64_t batch, int64_t M, int64_t N, int64_t K,
                            const void *A, int64_t lda, int64_t strideA,
                            const void *B, int64_t ldb, int64_t strideB,
                            void *C, int64_t ldc, int64_t strideC,
                            int out_fp32, struct ihipStream_t *stream);

/* The general entry point behind the three above, with the kernel variant
 * made explicit so that tests and benchmarks can pin one.
 * dtype: 0 = fp16 inputs, 1 = bf16 inputs.  variant: 0 chooses
 * automatically (what the three calls above do); 1 .. bpt_variant_count()
 * forces that variant and returns BPT_ERR_UNSUPPORTED when its shape,
 * alignment or type requirements are not met. */
bpt_status gemm_ex(int dtype, int64_t batch, int64_t M, int64_t N, int64_t K,
                   const void *A, int64_t lda, int64_t strideA,
                   const void *B, int64_t ldb, int64_t strideB,
                   void *C, int64_t ldc, int64_t strideC,
                   int out_fp32, int variant, struct ihipStream_t *stream);

/* For callers that cannot allocate device memory -- code being captured
 * into a HIP graph, serving loops that must not call hipMalloc, harnesses
 * that forbid it: gemm_ex with the same arguments, meaning and variant
 * choice, whose split-K partials and repack copies go into one fixed device
 * array of bpt_noalloc_scratch_bytes() (32 MiB) instead of the workspace
 * pool.  It calls no hipMalloc, hipFree or other allocating routine; each
 * GPU the library runs on holds its copy of the array until the process
 * ends.  A call whose path needs more scratch than that returns
 * BPT_ERR_UNSUPPORTED before launching anything (the message names the need
 * and the limit); calls needing none behave exactly as gemm_ex.  Every call
 * on a GPU shares that GPU's array: calls that overlap on one GPU (on
 * different streams, or from different host threads without ordering
 * between them) race and give wrong results.  Calls on one stream are
 * ordered by the stream.  Nothing in the array has to start at zero (every
 * partial and copy is written whole before it is read).  Under graph
 * capture the split paths keep their splits (gemm_ex runs them unsplit). */
bpt_status gemm_ex_noalloc(int dtype, int64_t batch, int64_t M, int64_t N, int64_t K,
                           const void *A, int64_t lda, int64_t strideA,
                           const void *B, int64_t ldb, int64_t strideB,
                           void *C, int64_t ldc, int64_t strideC,
                           int out_fp32, int variant, struct ihipStream_t *stream);

/* Bytes of the no-allocation entry point's device array. */
int64_t bpt_noalloc_scratch_bytes(void);

/* B given transposed: C (M x N) <- A * Bt^T, where Bt is N x K row major
 * with leading dimension ldbt >= max(1, K) and batch stride strideBt (B is
 * read as B[k][n] = Bt[n][k]).  This is the layout in which the pages' GEMM
 * keeps B for its "gather" kernel (its B[N,K]); the K-contiguous rows need
 * no transpose on the way to the matrix cores.  Everything else -- dtype,
 * batch, out_fp32, stream, errors, degenerate shapes -- as gemm_ex.
 * variant: 0 chooses automatically among the variants named
 * "pipelined_bt_*" and "generic_bt_*" (fast path: A and Bt 16-byte aligned,
 * lda, ldbt and the batch strides multiples of 8, K >= 128 and either a
 * multiple of 32 or of 8 with a tail; any N) and "splitk_pipelined", which
 * are the only ones this entry point takes; the others are for gemm_ex and
 * are rejected here with BPT_ERR_UNSUPPORTED, and vice versa
 * ("splitk_pipelined" serves both). */
bpt_status gemm_ex_bt(int dtype, int64_t batch, int64_t M, int64_t N, int64_t K,
                      const void *A, int64_t lda, int64_t strideA,
                      const void *Bt, int64_t ldbt, int64_t strideBt,
                      void *C, int64_t ldc, int64_t strideC,
                      int out_fp32, int variant, struct ihipStream_t *stream);

/* Fused scaled dot-product attention, forward (the pages' second workload:
 * the HD = 256 flash-attention "SDP" kernel of the "Xe2 Nbarrier Pipelining" page,
 * section "Proven Pattern: SDP Kernel Split Barrier B"):
 *     O[b][i][d] = sum_j p_j V[b][j][d] / sum_j p_j,
 *     p_j = exp(s_j - max_j s_j),  s_j = scale * sum_e Q[b][i][e] K[b][j][e]
 * for every b < batch_heads and query row i < seq_q, j over all seq_kv keys
 * (no mask).  Q is seq_q x head_dim, K and V are seq_kv x head_dim, O is
 * seq_q x head_dim, all row major with leading dimensions ldq, ldk, ldv,
 * ldo (>= head_dim) and strides strideQ .. strideO (>= 0) between the
 * batch_heads problems, in elements.  dtype: 0 = fp16, 1 = bf16 inputs; O
 * is the input type (round to nearest even) or fp32 (out_fp32 = 1).  The
 * logits and all sums are fp32; the weights enter the second product
 * rounded to the input type.  scale is typically 1/sqrt(head_dim).
 * Ownership, stream and errors as for the GEMMs; O must not overlap Q, K or
 * V.  head_dim must be 128 or 256, the bases 16-byte aligned and the
 * leading dimensions and strides multiples of 8 (else BPT_ERR_UNSUPPORTED);
 * a non-finite scale is BPT_ERR_INVALID_ARG.  batch_heads == 0 or
 * seq_q == 0 launches nothing; seq_kv == 0 writes zeros to O (an empty
 * softmax has no weights).  No workspace is used. */
bpt_status attention_fwd(int dtype, int64_t batch_heads, int64_t seq_q, int64_t seq_kv, int64_t head_dim,
                         const void *Q, int64_t ldq, int64_t strideQ,
                         const void *K, int64_t ldk, int64_t strideK,
                         const void *V, int64_t ldv, int64_t strideV,
                         void *O, int64_t ldo, int64_t strideO,
                         float scale, int out_fp32, struct ihipStream_t *stream);

/* Which variant gemm_ex(variant = 0) would run for these arguments (the
 * pointers are only inspected for alignment).  Returns 0 when the call
 * would be rejected or launch nothing. */
int bpt_select_variant(int dtype, int64_t batch, int64_t M, int64_t N, int64_t K,
                       const void *A, int64_t lda, const void *B, int64_t ldb,
                       int out_fp32);

/* The same for gemm_ex_bt (Bt is N x K with leading dimension ldbt). */
int bpt_select_variant_bt(int dtype, int64_t batch, int64_t M, int64_t N, int64_t K,
                          const void *A, int64_t lda, const void *Bt, int64_t ldbt,
                          int out_fp32);

/* Number of variants and the name of variant v (1-based); NULL if out of
 * range.  Names spell the tile shape, K-tile and stage count. */
int bpt_variant_count(void);
const char *bpt_variant_name(int v);

/* The workspace pool's choice of buffer, exported so that its policy can be
 * tested without a GPU (the library calls it internally; a caller never
 * needs to).  Input, for each of the n buffers of a device's pool: bytes[i];
 * busy[i] (1: taken by a call still on the host); state[i] (0: never used,
 * 1: its last use has completed, 2: its last use may still run); same[i] (1:
 * that last use was on the caller's stream handle).  Returns the buffer to
 * take, or n for a new one.  *wait is set to 1 when the caller's stream must
 * first wait for the buffer's last use -- always for state 2, since a handle
 * can name a different stream (hipStreamPerThread on another thread, a
 * destroyed stream's handle reused) -- and *grow to 1 when the buffer is too
 * small and is replaced by a larger one.  cap is the pool size above which
 * calls wait for each other's buffers rather than add one. */
int bpt_ws_choose(int n, const long long *bytes, const int *busy, const int *state, const int *same,
                  long long need, int cap, int *wait, int *grow);

/* Static text for a status code. */
const char *bpt_status_string(bpt_status s);

/* Message of the last non-OK status returned on the calling thread ("" if
 * none).  The pointer stays valid until the next call on that thread. */
const char *bpt_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* BPT_GEMM_H */
