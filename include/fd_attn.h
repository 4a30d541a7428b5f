/*
 * fd_attn.h -- C ABI of the unified-max split-KV decode-attention library for
 * AMD MI355X (gfx950).
 *
 * The operation (FlashDecoding++ theory page, sections 1 and 3; the split-KV
 * figure credited there to the Flash-Decoding post): one decode step of
 * attention.  For every batch entry b and query head h, a single query vector
 * q[b][h] is scored against the first seq_lens[b] keys of its KV head
 * (kvh = h / (Hq / Hkv)), and the output is the softmax-weighted sum of the
 * matching values:
 *
 *     s_t = scale * <q, k_t>             (fp8 caches: k_t = k_scale[kvh] * code)
 *     out = sum_t exp(s_t - phi) v_t / sum_t exp(s_t - phi)
 *
 * The cache is cut into chunks of chunk_size tokens.  Each chunk is reduced on
 * its own against the caller's constant phi -- no chunk waits for another's
 * maximum -- and the chunk sums are merged by a plain addition (theory page,
 * section 3, the unified-max formula).  A (b, h) row in which any score leaves
 * the safe band [phi - a, phi + b] is reported in fallback_flags and its
 * out-of-band chunks are recomputed with the ordinary running-max online
 * softmax, then merged with the usual max rescale (same section, the fallback
 * rule).  With or without fallback the result equals exact softmax attention
 * up to fp32 rounding.
 *
 * Ownership and threading: every pointer is device memory owned by the
 * caller.  The library never allocates, frees or synchronises; its only
 * global state is a call counter that gives every call a fresh epoch.  A call
 * enqueues its kernels on `stream` and returns (one kernel where the merge
 * runs inside it -- small grids, the plan table's fused rows, balanced
 * shares; a chunk kernel and a merge kernel otherwise).  out,
 * fallback_flags and the
 * workspace are valid once the stream has completed the call.  Calls may run
 * concurrently on different streams as long as each has its own workspace
 * and outputs; calls that share a workspace must be ordered (one stream).
 *
 * Errors: a call returns FD_OK (0) or a negative FD_ERR_* code.  On any
 * host-detected error nothing is enqueued.  FD_ERR_LAUNCH comes from the
 * status of the call's own launches; the thread's HIP last-error state is
 * neither read nor cleared (an error the caller left there stays there).
 * Device-resident data cannot be checked without a synchronisation:
 * seq_lens[b] is clamped to [0, max_seq_len]; a block_table entry outside
 * [0, num_pages) that a valid token needs is undefined behaviour (it
 * addresses memory outside the cache).  Cache slots that no valid token uses
 * (past seq_lens[b] in a sequence's last page or in contiguous capacity, pages
 * no sequence uses) may hold anything, NaN included: they never reach a
 * result.
 */
#ifndef FD_ATTN_H
#define FD_ATTN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage formats.  FD_FP8_E4M3FN is the OCP 8-bit float with 4 exponent
 * bits (bias 7) and 3 mantissa bits, max +-448, no infinities, S.1111.111 =
 * NaN; a cached value is code * per-KV-head fp32 scale (the symmetric scale of
 * the quantisation background page). */
typedef enum {
    FD_F32 = 0,
    FD_BF16 = 1,
    FD_FP8_E4M3FN = 2
} fd_dtype_t;

enum {
    FD_OK = 0,
    FD_ERR_NULL = -1,         /* a required pointer is NULL */
    FD_ERR_SHAPE = -2,        /* a size is out of range or inconsistent */
    FD_ERR_DTYPE = -3,        /* unsupported storage format combination */
    FD_ERR_ALIGN = -4,        /* q, caches or out not 16-byte aligned */
    FD_ERR_BAND = -5,         /* phi, a or b not finite, a or b outside [0, 64] */
    FD_ERR_WORKSPACE = -6,    /* workspace NULL, unaligned or smaller than required */
    FD_ERR_LAUNCH = -7        /* the HIP runtime rejected a launch */
};

/*
 * Problem descriptor.  Shapes and layouts (all dense, row-major):
 *   q               [batch][num_q_heads][head_dim]          q_dtype (F32 or BF16)
 *   contiguous K/V  [batch][num_kv_heads][max_seq_len][head_dim]       (page_size == 0)
 *   paged K/V       [num_pages][num_kv_heads][page_size][head_dim]     (page_size  > 0)
 *                   token t of sequence b is in page block_table[b][t / page_size],
 *                   slot t % page_size
 *   block_table     int32 [batch][max_blocks_per_seq]           (paged only)
 *   seq_lens        int32 [batch]
 *   out             [batch][num_q_heads][head_dim]          out_dtype (F32 or BF16)
 *   fallback_flags  uint8 [batch][num_q_heads]: 1 if any score of the row left the band
 */
typedef struct {
    int32_t batch;              /* >= 1 */
    int32_t num_q_heads;        /* >= 1, a multiple of num_kv_heads */
    int32_t num_kv_heads;       /* >= 1 */
    int32_t head_dim;           /* must be 128 */
    int32_t max_seq_len;        /* 1 .. 2^23: contiguous capacity; seq_lens are clamped to it */
    int32_t chunk_size;         /* split size: a multiple of 32 (and of page_size), >= 32;
                                   0 = the library's pick from its table (fd_attn_plan),
                                   halved for calls with few rows (see fd_attn_plan) */
    int32_t page_size;          /* 0 = contiguous; else a power of two in [16, 256] */
    int32_t max_blocks_per_seq; /* paged: >= ceil(max_seq_len / page_size) */
    int32_t num_pages;          /* paged: number of pages in the K/V pool (>= 1) */
    float scale;                /* softmax scale; <= 0 selects 1/sqrt(head_dim) */
    fd_dtype_t q_dtype;         /* FD_F32 or FD_BF16 */
    fd_dtype_t kv_dtype;        /* FD_F32, FD_BF16 or FD_FP8_E4M3FN */
    fd_dtype_t out_dtype;       /* FD_F32 or FD_BF16 */
    const float *k_scale;       /* [num_kv_heads] device fp32, required iff kv_dtype is fp8 */
    const float *v_scale;       /* [num_kv_heads] device fp32, required iff kv_dtype is fp8 */
    void *workspace;            /* device, 256-byte aligned, >= fd_attn_workspace_size() bytes */
    size_t workspace_bytes;
    /* Optional instrumentation: NULL, or 2 caller-created events: start and
     * stop of the call's chunk kernel (which includes the merge when that runs
     * in the same launch), stamped by its own dispatch on `stream` (no extra
     * stream work). */
    hipEvent_t *stage_events;
    /* 0: the library's plan (see fd_attn_plan).  Otherwise, for tuning and
     * tests, FD_PLAN_SHAPE(k) forces kernel shape k of the call's family and
     * FD_PLAN_FUSED / FD_PLAN_SPLIT force the merge into the chunk launch or
     * into a second launch (either bit alone; the results are the same).
     * FD_PLAN_SHARES forces balanced shares (grouped families only; with
     * FD_PLAN_SPLIT, FD_ERR_SHAPE): instead of fixed chunks of chunk_size
     * tokens, a persistent grid of workgroups splits the call's tokens --
     * all row groups (sequence x block of query heads sharing a KV head)
     * laid end to end, counted in 64-token quanta, an empty sequence
     * counting one.  Calls of at least 4 quanta per workgroup put three
     * quarters of the quanta in equal contiguous shares, one per workgroup,
     * and the rest in 1024-token grains that workgroups claim in turn once
     * their share is done; smaller calls are all shares.  The cut depends
     * on the lengths only, so results do not depend on which workgroup
     * computes what.  A row group's chunks are then its pieces in the
     * shares and grains that touch it (cut at their edges, multiples of 64
     * tokens), reduced and band-checked on their own and merged in the
     * launch.  chunk_size still has to be valid but does not apply.  The
     * library also picks balanced shares for some calls with chunk_size 0
     * and nothing forced (fd_attn_plan). */
    int32_t plan;
} fd_attn_desc_t;

#define FD_PLAN_SHAPE(k) ((k) + 1)
#define FD_PLAN_SHAPE_MASK 0x0f
#define FD_PLAN_FUSED 0x10
#define FD_PLAN_SPLIT 0x20
#define FD_PLAN_SHARES 0x40 /* balanced shares (see plan above) */

/* Bytes of workspace a call with this descriptor needs (0 if desc is NULL or
 * its sizes are invalid; it depends on the plan, see fd_attn_plan).  The
 * workspace holds per-(row, chunk) partial sums (with balanced shares, per
 * (row, piece): a row group's piece in one share or pool grain), the counter
 * of claimed pool grains and per-row-group completion counters; it needs no
 * initialisation (the counters are tagged with a per-call epoch) and its
 * contents between calls are the library's.  After a call completes, its
 * first 4 bytes hold the uint32 number of (row, chunk) pairs (balanced
 * shares: (row, piece) pairs) that call recomputed with online softmax, and
 * the next 4 bytes that call's epoch.  A call captured into a
 * graph keeps the epoch it was captured with; every replay still counts from
 * zero, so after each replay the first 4 bytes hold that replay's count. */
size_t fd_attn_workspace_size(const fd_attn_desc_t *desc);

/* One decode-attention call (see the top of this file).  phi is the preset
 * unified maximum; [phi - a, phi + b] the safe band (closed; a NaN score is
 * outside it).  Returns FD_OK or an FD_ERR_* code; asynchronous on `stream`. */
int fd_attn_decode(const fd_attn_desc_t *desc, const void *q, const void *k_cache,
                   const void *v_cache, const int32_t *seq_lens, const int32_t *block_table,
                   float phi, float a, float b, void *out, uint8_t *fallback_flags,
                   hipStream_t stream);

/* The allocation-free variant of fd_attn_decode, for callers that cannot
 * allocate device memory: code under graph capture, tight serving loops,
 * harnesses that forbid allocation.  Same arguments and results as
 * fd_attn_decode, but desc->workspace and desc->workspace_bytes are ignored:
 * the workspace is a static device array of FD_ATTN_STATIC_WORKSPACE_BYTES
 * inside the library, one per GPU, held from the library's load until the
 * process ends.  A call whose fd_attn_workspace_size() exceeds that returns
 * FD_ERR_WORKSPACE and enqueues nothing.  The first call on a device looks up
 * that device's copy (FD_ERR_LAUNCH if the runtime cannot give its address);
 * no call allocates or frees anything.  Every call on one GPU shares the
 * array, which keeps the last call's partials (it needs no clearing: its
 * counters carry a per-call epoch), so calls that overlap on one GPU -- on
 * different streams, or from different threads -- race and give undefined
 * results; order them on one stream.  The recomputed-pair count of the last
 * call is in the array, not readable through this interface. */
#define FD_ATTN_STATIC_WORKSPACE_BYTES ((size_t)64 << 20)

int fd_attn_decode_static(const fd_attn_desc_t *desc, const void *q, const void *k_cache,
                          const void *v_cache, const int32_t *seq_lens, const int32_t *block_table,
                          float phi, float a, float b, void *out, uint8_t *fallback_flags,
                          hipStream_t stream);

/* The plan a call with this descriptor would run, from the library's table
 * of measured plans (or desc->plan where it forces one; with chunk_size 0,
 * the table may pick balanced shares, and does for calls of many row groups,
 * but only when each share gets at least 8192 tokens of work counted at
 * max_seq_len; and a call with few rows gets the table's chunk size halved,
 * down to 256 tokens, until it has 256 units -- the table was measured on
 * full batches, where a small call would leave most of the chip idle):
 * the chunk size, the
 * kernel family (0: grouped bf16 queries over a bf16 cache; 1: grouped bf16
 * queries over an E4M3FN cache; 2: one query per KV head, or fp32 operands),
 * the kernel shape within the family, whether the merge runs inside the
 * chunk launch (1) or in a second launch (0), and the number of balanced
 * shares (0: fixed chunks of the reported size; otherwise the workgroups
 * that split the call, see FD_PLAN_SHARES).  The table is keyed by family,
 * paging and max_seq_len (the offline table of shapes of the FlashDecoding++
 * theory page, section 4).  Any output pointer may be NULL.  Returns FD_OK or
 * FD_ERR_NULL / FD_ERR_SHAPE for an invalid descriptor. */
int fd_attn_plan(const fd_attn_desc_t *desc, int32_t *chunk_size, int32_t *family, int32_t *shape,
                 int32_t *fused, int32_t *shares);

/* Static text for a status code. */
const char *fd_attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FD_ATTN_H */
