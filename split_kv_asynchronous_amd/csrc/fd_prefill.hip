// Host side of fd_attn_prefill (include/fd_prefill.h): validation and the
// launch of the causal prefill kernel.  No allocation, no synchronisation.
#include <hip/hip_ext.h>
#include <math.h>
#include <string.h>

#include "fd_host.h"
#include "fd_prefill.h"
#include "fd_prefill_kernel.h"

namespace {

#ifndef FD_PREFILL_WAVES
#define FD_PREFILL_WAVES 4
#endif
#ifndef FD_PREFILL_QBLOCKS
#define FD_PREFILL_QBLOCKS 2
#endif
#ifndef FD_PREFILL_STAGES
#define FD_PREFILL_STAGES 3
#endif

using PrefillShape = fd::prefill::Shape<FD_PREFILL_WAVES, FD_PREFILL_QBLOCKS, FD_PREFILL_STAGES>;
using fd::host::aligned16;

}  // namespace

namespace {

template <int KV, bool PAGED, bool OB>
int launch_prefill(const fd::prefill::PrefillParams &p, dim3 grid, dim3 block, hipStream_t s, hipEvent_t e0,
                   hipEvent_t e1)
{
    return fd::host::launch(
        fd::prefill::prefill_kernel<FD_PREFILL_WAVES, FD_PREFILL_QBLOCKS, FD_PREFILL_STAGES, KV, PAGED, OB>, grid,
        block, 0, s, e0, e1, p);
}

template <int KV, bool PAGED>
int launch_prefill(const fd::prefill::PrefillParams &p, bool out_bf16, dim3 grid, dim3 block, hipStream_t s,
                   hipEvent_t e0, hipEvent_t e1)
{
    return out_bf16 ? launch_prefill<KV, PAGED, true>(p, grid, block, s, e0, e1)
                    : launch_prefill<KV, PAGED, false>(p, grid, block, s, e0, e1);
}

}  // namespace

extern "C" int fd_attn_prefill(const fd_prefill_desc_t *d, const void *q, const void *k,
                               const void *v, const int32_t *kv_lens, float phi, float a,
                               float b, void *out, uint8_t *fallback_flags, hipStream_t stream)
{
    if (!d || !q || !k || !v || !kv_lens || !out || !fallback_flags) return FD_ERR_NULL;
    if (d->batch < 1 || d->batch > 65535 || d->num_q_heads < 1 || d->num_kv_heads < 1)
        return FD_ERR_SHAPE;
    if (d->num_q_heads % d->num_kv_heads) return FD_ERR_SHAPE;
    if (d->head_dim != fd::kHeadDim) return FD_ERR_SHAPE;
    if (d->q_len < 1 || d->q_len > (1 << 23)) return FD_ERR_SHAPE;
    if (d->max_seq_len < 1 || d->max_seq_len > (1 << 23)) return FD_ERR_SHAPE;
    if (!isfinite(d->scale)) return FD_ERR_SHAPE;
    const bool paged = d->page_size != 0;
    if (paged) {
        if (!fd::host::is_pow2(d->page_size) || d->page_size < 16 || d->page_size > 256) return FD_ERR_SHAPE;
        if (d->num_pages < 1) return FD_ERR_SHAPE;
        if ((int64_t)d->max_blocks_per_seq * d->page_size < d->max_seq_len) return FD_ERR_SHAPE;
        if (!d->block_table) return FD_ERR_NULL;
    }
    if (d->dtype != FD_BF16) return FD_ERR_DTYPE;
    if (d->kv_dtype != FD_BF16 && d->kv_dtype != FD_FP8_E4M3FN) return FD_ERR_DTYPE;
    if (d->out_dtype != FD_F32 && d->out_dtype != FD_BF16) return FD_ERR_DTYPE;
    const bool fp8 = d->kv_dtype == FD_FP8_E4M3FN;
    if (fp8 && (!d->k_scale || !d->v_scale)) return FD_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return FD_ERR_ALIGN;
    if (!isfinite(phi) || !isfinite(a) || !isfinite(b) || a < 0.f || b < 0.f || a > 64.f ||
        b > 64.f)
        return FD_ERR_BAND;

    const int64_t ntiles = ((int64_t)d->q_len + PrefillShape::rows - 1) / PrefillShape::rows;
    const int64_t total = (int64_t)d->batch * d->num_q_heads * ntiles;
    if (total > ((int64_t)1 << 31) - 8) return FD_ERR_SHAPE;

    fd::prefill::PrefillParams p;
    memset(&p, 0, sizeof p);
    p.q = static_cast<const uint16_t *>(q);
    p.k = k;
    p.v = v;
    p.kv_lens = kv_lens;
    p.block_table = paged ? d->block_table : nullptr;
    p.k_scale = fp8 ? d->k_scale : nullptr;
    p.v_scale = fp8 ? d->v_scale : nullptr;
    p.out = out;
    p.flags = fallback_flags;
    p.batch = d->batch;
    p.hq = d->num_q_heads;
    p.hkv = d->num_kv_heads;
    p.group = d->num_q_heads / d->num_kv_heads;
    p.q_len = d->q_len;
    p.max_seq_len = d->max_seq_len;
    p.page_shift = 0;
    if (paged)
        while ((1 << p.page_shift) < d->page_size) ++p.page_shift;
    p.max_blocks = d->max_blocks_per_seq;
    p.ntiles = (int)ntiles;
    p.total = (int)total;
    p.per_xcd = (int)((total + 7) / 8);
    // the kernel works on raw scores q.k: the softmax scale moves into the
    // exponent factor and the band edges are divided by it (E4M3FN: per KV
    // head on the GPU, with k_scale joining the scale)
    const double scale = d->scale > 0.f ? (double)d->scale : 1.0 / sqrt((double)fd::kHeadDim);
    const double log2e = 1.4426950408889634;
    p.c1 = (float)(scale * log2e);
    p.c0 = (float)(-(double)phi * log2e);
    p.lo_raw = (float)(((double)phi - (double)a) / scale);
    p.hi_raw = (float)(((double)phi + (double)b) / scale);
    p.phi_raw = (float)((double)phi / scale);
    p.scale = (float)scale;
    p.lo = (float)((double)phi - (double)a);
    p.hi = (float)((double)phi + (double)b);
    p.phi = phi;

    hipEvent_t *ev = d->stage_events;
    hipEvent_t ev0 = ev ? ev[0] : nullptr, ev1 = ev ? ev[1] : nullptr;
    const dim3 grid((unsigned)(8 * (int64_t)p.per_xcd)), block(PrefillShape::waves * 64);
    const bool ob = d->out_dtype == FD_BF16;
    if (fp8)
        return paged ? launch_prefill<FD_FP8_E4M3FN, true>(p, ob, grid, block, stream, ev0, ev1)
                     : launch_prefill<FD_FP8_E4M3FN, false>(p, ob, grid, block, stream, ev0, ev1);
    return paged ? launch_prefill<FD_BF16, true>(p, ob, grid, block, stream, ev0, ev1)
                 : launch_prefill<FD_BF16, false>(p, ob, grid, block, stream, ev0, ev1);
}
