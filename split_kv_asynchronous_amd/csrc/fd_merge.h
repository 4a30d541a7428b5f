// Merge of the chunk partials of each (b, h) row.
//
// Without recomputed chunks every partial was taken against the same constant
// phi, so the merge is a plain sum: out = sum_c o_c / sum_c l_c, no rescale
// (FlashDecoding++ theory page, section 3: after the unified maximum only a
// simple sum is left at the end).  A row with a recomputed chunk holds
// partials against different maxima (phi, or the chunk's own maximum) and is
// merged with the ordinary max rescale of split-KV softmax (the split-KV
// figure of section 1).
#pragma once

#include "fd_common.h"

namespace fd {

// Grid ceil(B*Hq / 4), 256 threads: one wavefront per row, 2 components per lane.
__global__ __launch_bounds__(256) void merge_kernel(Params p)
{
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= p.batch * p.hq) return;
    const int b = row / p.hq, h = row % p.hq;
    const int L = seq_len_of(p, b);
    const int nch = (L + p.chunk - 1) / p.chunk;
    const size_t base = (size_t)row * p.maxch;

    int any = 0;
    for (int c = lane; c < nch; c += 64) any |= p.cflag[base + c];
    any = __any(any);

    f32x2 o = {0.f, 0.f};
    float l = 0.f;
    if (!any) {
        for (int c = 0; c < nch; ++c) {
            const f32x2 oc = *reinterpret_cast<const f32x2 *>(p.o_part + (base + c) * kHeadDim + 2 * lane);
            o += oc;
            l += p.l_part[base + c];
        }
    } else {
        float M = -INFINITY;
        for (int c = 0; c < nch; ++c) M = fmaxf(M, p.m_part[base + c]);
        for (int c = 0; c < nch; ++c) {
            const float mc = p.m_part[base + c];
            const float f = (mc == M) ? 1.f : exp2_hw((mc - M) * kLog2e);
            const f32x2 oc = *reinterpret_cast<const f32x2 *>(p.o_part + (base + c) * kHeadDim + 2 * lane);
            o += oc * f;
            l = fmaf(p.l_part[base + c], f, l);
        }
    }
    float vs = 1.f;
    if (p.v_scale) vs = p.v_scale[h / p.group];
    f32x2 r = {0.f, 0.f};
    if (nch > 0) {
        const float inv = vs / l;
        r = o * inv;
    }
    if (p.out_bf16) {
        // round to nearest even
        uint32_t a = __float_as_uint(r.x), c2 = __float_as_uint(r.y);
        a = (r.x != r.x) ? 0x7fc0u : (a + 0x7fffu + ((a >> 16) & 1u)) >> 16;
        c2 = (r.y != r.y) ? 0x7fc00000u : (c2 + 0x7fffu + ((c2 >> 16) & 1u)) & 0xffff0000u;
        reinterpret_cast<uint32_t *>(p.out)[(size_t)row * (kHeadDim / 2) + lane] = a | c2;
    } else {
        reinterpret_cast<f32x2 *>(p.out)[(size_t)row * (kHeadDim / 2) + lane] = r;
    }
    if (lane == 0) p.flags[row] = any ? 1 : 0;
}

}  // namespace fd
