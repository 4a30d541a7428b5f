/*
 * fd_prefill.h -- C ABI of causal prefill attention with the unified maximum
 * (AMD MI355X, gfx950), part of the same library as fd_attn.h.
 *
 * The operation (FlashDecoding++ theory page, section 3: the preset maximum
 * serves the prefill phase as it serves decode; section 1: prefill handles all
 * prompt tokens in one pass): for every batch entry b and query head h, a
 * block of q_len query vectors sits at the END of the sequence -- query j is
 * at position pos = kv_lens[b] - q_len + j -- and attends the keys of its KV
 * head (kvh = h / (Hq / Hkv)) at positions 0 .. pos:
 *
 *     s_t   = scale * <q_j, k_t>                            t = 0 .. pos
 *     out_j = sum_t exp(s_t - phi) v_t / sum_t exp(s_t - phi)
 *     flag_j = 1 if any s_t (t <= pos) lies outside [phi - a, phi + b]
 *
 * q_len == kv_len is a whole prompt; q_len < kv_len appends a block to a
 * cached prefix; a query with pos < 0 (kv_len < q_len) attends nothing and
 * gets a zero row with flag 0.  Weights are taken against the caller's
 * constant phi with no running maximum; once a score outside the band is seen
 * the computation continues with the ordinary running-maximum softmax (the
 * fallback rule of the same section), so the result is exact softmax attention
 * up to rounding either way.  Each attention weight enters the weight-value
 * product as a bf16 high part plus a bf16 remainder (together a relative
 * error of at most 2^-18) and the weight sums add the fp32 weights.
 *
 * The cache holds bf16 values or E4M3FN codes (value = code * the KV head's
 * k_scale / v_scale, which must be positive), contiguous per sequence or in
 * pages through a block table, as the decode call's caches do.
 *
 * Ownership and threading: every pointer is device memory owned by the
 * caller.  The call allocates nothing, needs no workspace, never
 * synchronises, and enqueues one kernel on `stream`; out and fallback_flags
 * are valid once the stream has completed it.  Calls on different streams
 * with distinct outputs may run concurrently.
 *
 * Errors: FD_OK (0) or a negative FD_ERR_* code from fd_attn.h; on any error
 * nothing is enqueued.  kv_lens[b] is device data and is clamped to
 * [0, max_seq_len]; a block_table entry outside [0, num_pages) that a key
 * needs is undefined behaviour.
 */
#ifndef FD_PREFILL_H
#define FD_PREFILL_H

#include "fd_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Problem descriptor.  Shapes and layouts (dense, row-major, bf16 = raw bit
 * patterns of bfloat16):
 *   q               [batch][num_q_heads][q_len][head_dim]           BF16
 *   contiguous k, v [batch][num_kv_heads][max_seq_len][head_dim]    kv_dtype  (page_size == 0)
 *   paged k, v      [num_pages][num_kv_heads][page_size][head_dim]  kv_dtype  (page_size  > 0)
 *                   key t of sequence b is in page block_table[b][t / page_size],
 *                   slot t % page_size
 *   block_table     int32 [batch][max_blocks_per_seq]               (paged only)
 *   kv_lens         int32 [batch]   keys of each sequence, the query block included
 *   out             [batch][num_q_heads][q_len][head_dim]           out_dtype
 *   fallback_flags  uint8 [batch][num_q_heads][q_len]
 * q, k, v and out must be 16-byte aligned.  Cache slots that no key of a
 * sequence uses may hold anything.
 */
typedef struct {
    int32_t batch;              /* 1 .. 65535 */
    int32_t num_q_heads;        /* >= 1, a multiple of num_kv_heads */
    int32_t num_kv_heads;       /* >= 1 */
    int32_t head_dim;           /* must be 128 */
    int32_t q_len;              /* 1 .. 2^23 */
    int32_t max_seq_len;        /* 1 .. 2^23: K/V capacity per sequence */
    float scale;                /* softmax scale; <= 0 selects 1/sqrt(head_dim) */
    fd_dtype_t dtype;           /* q: FD_BF16 */
    fd_dtype_t out_dtype;       /* FD_F32 or FD_BF16 */
    /* Optional instrumentation: NULL, or 2 caller-created events stamped at
     * the start and the end of the call's kernel by its own dispatch. */
    hipEvent_t *stage_events;
    fd_dtype_t kv_dtype;        /* k and v: FD_BF16 or FD_FP8_E4M3FN */
    int32_t page_size;          /* 0 = contiguous; else a power of two in [16, 256] */
    int32_t max_blocks_per_seq; /* paged: >= ceil(max_seq_len / page_size) */
    int32_t num_pages;          /* paged: pages in the K/V pool (>= 1) */
    const int32_t *block_table; /* paged: device int32 [batch][max_blocks_per_seq]; else NULL */
    const float *k_scale;       /* E4M3FN: device fp32 [num_kv_heads], > 0; else NULL */
    const float *v_scale;       /* E4M3FN: device fp32 [num_kv_heads], > 0; else NULL */
} fd_prefill_desc_t;

/* One prefill call (see the top of this file).  phi is the preset unified
 * maximum and [phi - a, phi + b] the safe band (closed).  Returns FD_OK or an
 * FD_ERR_* code; asynchronous on `stream`. */
int fd_attn_prefill(const fd_prefill_desc_t *desc, const void *q, const void *k, const void *v,
                    const int32_t *kv_lens, float phi, float a, float b, void *out,
                    uint8_t *fallback_flags, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FD_PREFILL_H */
