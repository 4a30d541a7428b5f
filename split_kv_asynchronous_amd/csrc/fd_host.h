// Host-side checks shared by the C-ABI entry points.
#pragma once

#include <hip/hip_ext.h>
#include <stdint.h>

#include <tuple>
#include <utility>

#include "fd_attn.h"
#include "fd_common.h"

namespace fd {
namespace host {

inline bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Launches k(args...) on stream s (optionally stamping events e0/e1 from the
// dispatch itself) and returns FD_OK or FD_ERR_LAUNCH from this launch's own
// status.  The thread's last-error state is neither read nor cleared, so an
// error that the caller's own earlier work left there stays for the caller.
template <typename... KArgs, typename... Args>
inline int launch(void (*k)(KArgs...), dim3 grid, dim3 block, size_t lds, hipStream_t s, hipEvent_t e0,
                  hipEvent_t e1, Args &&...args)
{
    static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
    std::tuple<KArgs...> held(std::forward<Args>(args)...);
    const hipError_t e = std::apply(
        [&](auto &...x) {
            void *argv[] = {static_cast<void *>(&x)...};
            return hipExtLaunchKernel(reinterpret_cast<const void *>(k), grid, block, argv, lds, s, e0, e1, 0);
        },
        held);
    return e == hipSuccess ? FD_OK : FD_ERR_LAUNCH;
}

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
