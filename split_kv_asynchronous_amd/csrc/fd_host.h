// Host-side checks shared by the C-ABI entry points.
#pragma once

#include <stdint.h>

#include "fd_attn.h"
#include "fd_common.h"

namespace fd {
namespace host {

inline bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Shape checks shared by the size query and the call.
inline int check_shape(const fd_attn_desc_t *d)
{
    if (d->batch < 1 || d->num_q_heads < 1 || d->num_kv_heads < 1) return FD_ERR_SHAPE;
    if (d->batch > 65535 || d->num_q_heads > 65535) return FD_ERR_SHAPE;   // grid limits
    if (d->num_q_heads % d->num_kv_heads) return FD_ERR_SHAPE;
    if (d->head_dim != fd::kHeadDim) return FD_ERR_SHAPE;
    if (d->max_seq_len < 1 || d->max_seq_len > (1 << 23)) return FD_ERR_SHAPE;
    if (d->chunk_size < 32 || d->chunk_size % 32) return FD_ERR_SHAPE;
    if (d->page_size) {
        if (!is_pow2(d->page_size) || d->page_size < 16 || d->page_size > 256) return FD_ERR_SHAPE;
        if (d->chunk_size % d->page_size) return FD_ERR_SHAPE;
        if (d->num_pages < 1) return FD_ERR_SHAPE;
        if ((int64_t)d->max_blocks_per_seq * d->page_size < d->max_seq_len) return FD_ERR_SHAPE;
    }
    const int64_t maxch = ((int64_t)d->max_seq_len + d->chunk_size - 1) / d->chunk_size;
    const int64_t slots = (int64_t)d->batch * d->num_q_heads * maxch;
    if (slots >= ((int64_t)1 << 31) || maxch >= ((int64_t)1 << 31)) return FD_ERR_SHAPE;
    if ((int64_t)d->batch * d->num_q_heads >= ((int64_t)1 << 31)) return FD_ERR_SHAPE;
    return FD_OK;
}

}  // namespace host
}  // namespace fd
