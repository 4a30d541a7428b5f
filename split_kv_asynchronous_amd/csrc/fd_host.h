// Host-side checks shared by the C-ABI entry points.
#pragma once

#include <stdint.h>

#include "fd_attn.h"
#include "fd_common.h"

namespace fd {
namespace host {

inline bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// The chunk size of a call: the descriptor's, or for 0 the pick measured per
// kernel family on MI355X: 2048 tokens for grouped bf16 queries over a bf16
// cache (32K GQA workload 5.99 -> 6.26 TB/s against 1024), 1024 otherwise
// (the paged fp8 and the vector kernels lose at 2048), at least a page.
inline int chunk_of(const fd_attn_desc_t *d)
{
    if (d->chunk_size != 0) return d->chunk_size;
    const int group = d->num_kv_heads > 0 ? d->num_q_heads / d->num_kv_heads : 1;
    int c = (group > 1 && d->q_dtype == FD_BF16 && d->kv_dtype == FD_BF16) ? 2048 : 1024;
    return d->page_size > c ? d->page_size : c;
}

// Shape checks shared by the size query and the call.
inline int check_shape(const fd_attn_desc_t *d)
{
    if (d->batch < 1 || d->num_q_heads < 1 || d->num_kv_heads < 1) return FD_ERR_SHAPE;
    if (d->batch > 65535 || d->num_q_heads > 65535) return FD_ERR_SHAPE;   // grid limits
    if (d->num_q_heads % d->num_kv_heads) return FD_ERR_SHAPE;
    if (d->head_dim != fd::kHeadDim) return FD_ERR_SHAPE;
    if (d->max_seq_len < 1 || d->max_seq_len > (1 << 23)) return FD_ERR_SHAPE;
    const int chunk = chunk_of(d);
    if (chunk < 32 || chunk % 32) return FD_ERR_SHAPE;
    if (d->page_size) {
        if (!is_pow2(d->page_size) || d->page_size < 16 || d->page_size > 256) return FD_ERR_SHAPE;
        if (chunk % d->page_size) return FD_ERR_SHAPE;
        if (d->num_pages < 1) return FD_ERR_SHAPE;
        if ((int64_t)d->max_blocks_per_seq * d->page_size < d->max_seq_len) return FD_ERR_SHAPE;
    }
    const int64_t maxch = ((int64_t)d->max_seq_len + chunk - 1) / chunk;
    const int64_t slots = (int64_t)d->batch * d->num_q_heads * maxch;
    if (slots >= ((int64_t)1 << 31) || maxch >= ((int64_t)1 << 31)) return FD_ERR_SHAPE;
    if ((int64_t)d->batch * d->num_q_heads >= ((int64_t)1 << 31)) return FD_ERR_SHAPE;
    return FD_OK;
}

}  // namespace host
}  // namespace fd
