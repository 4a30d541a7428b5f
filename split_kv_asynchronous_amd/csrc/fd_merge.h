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

// RW wavefronts per row, 256 threads per workgroup (256 / (64 RW) rows each).
// In a wavefront, lanes 0..31 take one chunk and lanes 32..63 the next, 4
// components per lane, four chunk pairs in flight; the wavefronts of a row
// split its chunks and meet in LDS.  The kernel also counts the recomputed
// (row, chunk) pairs into the workspace counter (zeroed by this call's chunk
// kernel).
template <int RW>
__global__ __launch_bounds__(256) void merge_kernel(Params p)
{
    constexpr int ROWS = 4 / RW;
    __shared__ f32x4 red_o[4][32];
    __shared__ float red_l[4];
    __shared__ int red_n[4];
    __shared__ float red_m[4];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int sub = wave % RW;                       // wavefront inside its row
    const int row = blockIdx.x * ROWS + wave / RW;
    const bool live = row < p.batch * p.hq;
    const int b = live ? row / p.hq : 0, h = live ? row % p.hq : 0;
    const int L = live ? seq_len_of(p, b) : 0;
    const int nch = (L + p.chunk - 1) / p.chunk;
    const size_t base = part_slot(p, b, h, 0);   // chunk c at base + c * hq
    const size_t cs = p.hq;
    const int rw0 = (wave / RW) * RW;                // first wavefront of this row

    // flagged chunks of the row, and the largest chunk maximum if any
    int nflag = 0;
    for (int c = sub * 64 + lane; c < nch; c += 64 * RW) nflag += p.cflag[base + c * cs];
#pragma unroll
    for (int x = 1; x < 64; x <<= 1) nflag += __shfl_xor(nflag, x);
    if (RW > 1) {
        if (lane == 0) red_n[wave] = nflag;
        __syncthreads();
        nflag = 0;
#pragma unroll
        for (int w = 0; w < RW; ++w) nflag += red_n[rw0 + w];
    }
    const bool any = nflag != 0;
    float M = p.phi;
    if (any) {
        M = -INFINITY;
        for (int c = sub * 64 + lane; c < nch; c += 64 * RW) M = fmaxf(M, p.m_part[base + c * cs]);
#pragma unroll
        for (int x = 1; x < 64; x <<= 1) M = fmaxf(M, __shfl_xor(M, x));
    }
    if (RW > 1) {
        if (lane == 0) red_m[wave] = M;
        __syncthreads();
#pragma unroll
        for (int w = 0; w < RW; ++w) M = fmaxf(M, red_m[rw0 + w]);
    }

    const int half = lane >> 5, q4 = lane & 31;
    const float *op = p.o_part + base * kHeadDim + 4 * q4;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float lacc = 0.f;
    constexpr int STEP = 2 * RW;                     // chunks per pass of all row waves
    int c = 2 * sub + half;
    // without a recomputed chunk every partial is against phi: plain sum;
    // otherwise each is rescaled from its own maximum to M
    for (; c + 3 * STEP < nch; c += 4 * STEP) {
        f32x4 v[4];
        float l[4], f[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            v[u] = *reinterpret_cast<const f32x4 *>(op + (size_t)(c + u * STEP) * cs * kHeadDim);
            l[u] = p.l_part[base + (c + u * STEP) * cs];
            f[u] = any ? p.m_part[base + (c + u * STEP) * cs] : M;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float g = (f[u] == M) ? 1.f : exp2_hw((f[u] - M) * kLog2e);
            acc += v[u] * g;
            lacc = fmaf(l[u], g, lacc);
        }
    }
    for (; c < nch; c += STEP) {
        const float mc = any ? p.m_part[base + c * cs] : M;
        const float g = (mc == M) ? 1.f : exp2_hw((mc - M) * kLog2e);
        acc += *reinterpret_cast<const f32x4 *>(op + (size_t)c * cs * kHeadDim) * g;
        lacc = fmaf(p.l_part[base + c * cs], g, lacc);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] += __shfl_xor(acc[i], 32);
    lacc += __shfl_xor(lacc, 32);
    if (RW > 1) {
        if (half == 0) red_o[wave][q4] = acc;
        if (lane == 0) red_l[wave] = lacc;
        __syncthreads();
        if (sub != 0) return;
        acc = f32x4{0.f, 0.f, 0.f, 0.f};
        lacc = 0.f;
#pragma unroll
        for (int w = 0; w < RW; ++w) {
            acc += red_o[rw0 + w][q4];
            lacc += red_l[rw0 + w];
        }
    }
    if (!live) return;

    f32x4 r = {0.f, 0.f, 0.f, 0.f};
    if (nch > 0) {
        float vs = 1.f;
        if (p.v_scale) vs = p.v_scale[h / p.group];
        r = acc * (vs / lacc);
    }
    if (half == 0) {
        if (p.out_bf16) {
            uint32_t w[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t u = __float_as_uint(r[i]);
                w[i] = (r[i] != r[i]) ? 0x7fc0u : ((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
            }
            reinterpret_cast<u32x2 *>(p.out)[(size_t)row * (kHeadDim / 4) + q4] =
                u32x2{w[0] | (w[1] << 16), w[2] | (w[3] << 16)};
        } else {
            reinterpret_cast<f32x4 *>(p.out)[(size_t)row * (kHeadDim / 4) + q4] = r;
        }
    }
    if (lane == 0) {
        p.flags[row] = any ? 1 : 0;
        if (nflag) atomicAdd(p.counter, nflag);
    }
}

}  // namespace fd
