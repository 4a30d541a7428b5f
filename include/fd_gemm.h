/*
 * fd_gemm.h -- C ABI of the flat GEMM of the decode linear layers (AMD
 * MI355X, gfx950), part of the same library as fd_attn.h.
 *
 * The operation (FlashDecoding++ theory page, section 2, the second
 * bottleneck, and section 4, the double-buffered flat GEMM and the heuristic
 * dataflow): the linear layers of a decoder block -- the Q/K/V projection,
 * the O projection and the two FFN products -- multiply a flat activation
 * matrix (M rows: the tokens of one decode step, M small) by a constant
 * weight matrix (N x K, fixed per layer):
 *
 *     C[m][n] = sum_k A[m][k] * W[n][k]          (C = A . W^T)
 *
 * A and W are bf16, the products are accumulated in fp32 and C is written in
 * fp32 or rounded to bf16.  M is padded only to a multiple of 16 inside the
 * kernel (no padded copy of A is made).  The weights stream from memory once
 * per call for M <= 64; beyond that they are read once per group of 64 rows.
 * Because W dominates the bytes moved for small M, the call is bound by
 * memory bandwidth and its kernel configuration depends only on M for a
 * given layer: the library picks it from a table keyed by (M, N, K) measured
 * offline, with a rule for shapes outside the table (fd_flat_gemm_plan shows
 * the pick).
 *
 * Rounding: each output is a sum of K exact bf16 x bf16 products accumulated
 * in fp32 in an unspecified order (within a K slice by the matrix cores, then
 * the slices in order), so |C - exact| <= gamma(K) * sum_k |A[m][k] W[n][k]|
 * with gamma(K) = K u / (1 - K u), u = 2^-24, plus half a bf16 ulp of C when
 * out_dtype is FD_BF16.
 *
 * Ownership and threading: every pointer is device memory owned by the
 * caller.  The call allocates nothing and never synchronises; it enqueues one
 * kernel on `stream`, or two when K is split over workgroups (a partial-sum
 * kernel writing fp32 partials into the workspace, then a reduce kernel).  C
 * is valid once the stream has completed the call.  Calls that share a
 * workspace must be ordered (one stream).
 *
 * Errors: FD_OK (0) or a negative FD_ERR_* code from fd_attn.h; on any error
 * nothing is enqueued.
 */
#ifndef FD_GEMM_H
#define FD_GEMM_H

#include "fd_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Problem descriptor.  Layouts (dense, row-major, bf16 = raw bit patterns of
 * bfloat16):
 *   a   [m][k]   a_dtype (FD_BF16)
 *   w   [n][k]   w_dtype (FD_BF16)     one output column per row of W
 *                (or its packed copy, w_layout = FD_GEMM_W_PACKED)
 *   c   [m][n]   out_dtype (FD_F32 or FD_BF16)
 * a, w and c must be 16-byte aligned.
 */
typedef struct {
    int32_t m;                  /* 1 .. 4096 */
    int32_t n;                  /* 1 .. 2^20 */
    int32_t k;                  /* 32 .. 2^20, a multiple of 32 */
    fd_dtype_t a_dtype;         /* FD_BF16 */
    fd_dtype_t w_dtype;         /* FD_BF16 */
    fd_dtype_t out_dtype;       /* FD_F32 or FD_BF16 */
    /* Tuning overrides, 0 = the library's pick: variant 1 .. FD_GEMM_VARIANTS
     * (see fd_flat_gemm_plan) and the number of K slices (1 .. k / 32). */
    int32_t variant;
    int32_t ksplit;
    /* Layout of w: FD_GEMM_W_ROWS ([n][k] row-major) or FD_GEMM_W_PACKED (the
     * output of fd_flat_gemm_pack_weights; variants 5 .. 12 only). */
    int32_t w_layout;
    void *workspace;            /* device, 256-byte aligned, >= fd_flat_gemm_workspace_size();
                                   may be NULL when that size is 0 */
    size_t workspace_bytes;
    /* Optional instrumentation: NULL, or 2 caller-created events stamped at
     * the start and the end of the partial-sum kernel by its own dispatch. */
    hipEvent_t *stage_events;
} fd_gemm_desc_t;

/* Kernel variants (a k-step is 32 of K):
 *   1..4   A staged in LDS; 4 wavefronts on 4 column blocks of 16 x
 *          {1, 2, 1, 2} columns; {8, 4, 16, 8} k-steps per load batch;
 *   5..12  A loaded directly; {4, 4, 4, 4, 8, 8, 16, 16} wavefronts on
 *          consecutive parts of the K slice of one column block of 16 x
 *          {4, 2, 1, 1, 1, 2, 1, 1} columns; {4, 8, 8, 16, 8, 4, 4, 8}
 *          k-steps per load batch (fewer when the rows of A need the
 *          registers);
 *   13, 14 weights moved by DMA into per-wavefront LDS rings of {3, 2}
 *          stages of 4 k-steps, A staged in LDS; 4 wavefronts on 4 column
 *          blocks of 16 columns.  K must be a multiple of 128. */
#define FD_GEMM_VARIANTS 14

#define FD_GEMM_W_ROWS 0
#define FD_GEMM_W_PACKED 1

/* Bytes of the packed copy of an n x k bf16 weight matrix: ceil(n / 16) * 16
 * * k * 2 (0 for invalid sizes). */
size_t fd_flat_gemm_packed_bytes(int32_t n, int32_t k);

/* Packs w ([n][k] row-major bf16, 16-byte aligned) into w_packed (device,
 * 16-byte aligned, fd_flat_gemm_packed_bytes long): ceil(n/16) blocks of 16
 * rows, each as k/32 steps of 1 KiB holding the 64 lanes' 16-byte operand
 * fragments of the 16x16x32 matrix-core instruction in lane order -- lane l
 * of block cb, step j gets row 16cb + l % 16, elements 32j + 8(l / 16) ..
 * +7; rows past n are zero.  Weights are fixed per layer, so this runs once,
 * when they are loaded; every weight-load instruction of the GEMM then reads
 * 1 KiB of consecutive bytes.  Asynchronous on `stream`; same size limits as
 * fd_flat_gemm.  Returns FD_OK or an FD_ERR_* code. */
int fd_flat_gemm_pack_weights(int32_t n, int32_t k, const void *w, void *w_packed, hipStream_t stream);

/* The configuration a call with this descriptor runs (the overrides applied):
 * variant, K slices, k-steps per slice and workgroups of the partial-sum
 * kernel.  Returns FD_OK or FD_ERR_SHAPE / FD_ERR_DTYPE for an invalid
 * descriptor.  Any output pointer may be NULL. */
int fd_flat_gemm_plan(const fd_gemm_desc_t *desc, int32_t *variant, int32_t *ksplit,
                      int32_t *steps_per_slice, int32_t *workgroups);

/* Bytes of workspace the call needs: ksplit * m * n * 4 when K is split,
 * 0 otherwise (and 0 for an invalid descriptor). */
size_t fd_flat_gemm_workspace_size(const fd_gemm_desc_t *desc);

/* C = A . W^T (see the top of this file).  Asynchronous on `stream`. */
int fd_flat_gemm(const fd_gemm_desc_t *desc, const void *a, const void *w, void *c,
                 hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FD_GEMM_H */
