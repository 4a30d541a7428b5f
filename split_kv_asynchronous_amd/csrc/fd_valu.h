// Vector-ALU chunk reduction: one query head against one chunk of its KV head.
//
// Used for single-query-per-KV-head attention (MHA), for fp32 caches or
// queries, and -- in online mode -- for the fallback recompute of chunks whose
// scores left the safe band.
//
// Lane mapping: a wavefront splits into four 16-lane rows; each row owns one
// token at a time and each of its lanes owns 8 of the 128 components, so one
// load instruction reads 4 whole consecutive tokens (1 KiB of bf16).  The
// 16-lane dot product is finished with four DPP adds.
#pragma once

#include "fd_common.h"
#include "fd_merge.h"

namespace fd {

// Reduce tokens [t_begin, t_end) of row (b, h).
//  ONLINE == false: unified maximum -- p = exp(s - phi), no maximum search
//                   (FlashDecoding++ theory page, section 3, second formula);
//                   writes o, l, m = phi and the chunk's band flag.
//  ONLINE == true : ordinary online softmax with a running maximum (same
//                   section, first formula, used by the fallback rule);
//                   writes o, l and the chunk maximum m.
// NW = wavefronts in the workgroup; `red` is LDS of at least NW * 132 floats.
// direct: the row is this one chunk (or empty) in a fused call -- write its
// output (the merge's arithmetic: the chunk's sum times v_scale over its
// weight sum) instead of the partial; a unified pass that is flagged writes
// nothing (the online pass does).
template <int KV, int QT, bool PAGED, bool ONLINE, int NW>
FD_DEV bool valu_chunk(const Params &p, int b, int h, int c, int t_begin, int t_end, float *red, bool direct)
{
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int row = lane >> 4;     // token slot inside the wavefront
    const int sub = lane & 15;     // owns components 8*sub .. 8*sub+7
    const int kvh = h / p.group;
    const size_t qrow = ((size_t)b * p.hq + h) * kHeadDim;

    float q[8];
    load8<QT>(p.q, qrow + 8 * sub, q);
    float sc = p.scale;
    if constexpr (KV == FD_FP8_E4M3FN) sc *= p.k_scale[kvh];

    float o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = 0.f;
    float l = 0.f;
    float m = ONLINE ? -INFINITY : p.phi;
    bool bad = false;

    constexpr int U = 4;                       // tokens per row per step
    constexpr int STEP = NW * 4 * U;           // tokens per workgroup step
    for (int base = t_begin; base < t_end; base += STEP) {
        float kx[U][8], vx[U][8];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int t = base + (wave * U + u) * 4 + row;
            const int tl = t < t_end ? t : t_end - 1;    // stay inside the sequence
            const size_t off = kv_offset<PAGED>(p, b, kvh, tl) + 8 * sub;
            load8<KV, true>(p.k, off, kx[u]);
            load8<KV, true>(p.v, off, vx[u]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int t = base + (wave * U + u) * 4 + row;
            const bool valid = t < t_end;
            float part = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) part = fmaf(q[j], kx[u][j], part);
            const float s = row16_sum(part) * sc;
            if constexpr (!ONLINE) {
                bad |= valid && outside_band(s, p.lo, p.hi);
                const float w = valid ? exp2_hw((s - p.phi) * kLog2e) : 0.f;
                l += w;
#pragma unroll
                for (int j = 0; j < 8; ++j) o[j] = fmaf(w, vx[u][j], o[j]);
            } else if (valid) {
                const float m_new = fmaxf(m, s);
                const float r = (m == m_new) ? 1.f : exp2_hw((m - m_new) * kLog2e);
                const float w = (s == -INFINITY) ? 0.f : exp2_hw((s - m_new) * kLog2e);
                l = fmaf(l, r, w);
#pragma unroll
                for (int j = 0; j < 8; ++j) o[j] = fmaf(o[j], r, w * vx[u][j]);
                m = m_new;
            }
        }
    }

    // combine the four rows of the wavefront (lanes sub, sub+16, sub+32, sub+48)
#pragma unroll
    for (int x = 16; x <= 32; x <<= 1) {
        const float l2 = __shfl_xor(l, x);
        if constexpr (ONLINE) {
            const float m2 = __shfl_xor(m, x);
            const float mm = fmaxf(m, m2);
            const float r1 = (m == mm) ? 1.f : exp2_hw((m - mm) * kLog2e);
            const float r2 = (m2 == mm) ? 1.f : exp2_hw((m2 - mm) * kLog2e);
#pragma unroll
            for (int j = 0; j < 8; ++j) o[j] = o[j] * r1 + __shfl_xor(o[j], x) * r2;
            l = l * r1 + l2 * r2;
            m = mm;
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) o[j] += __shfl_xor(o[j], x);
            l += l2;
        }
    }
    const bool wave_bad = __any(bad);

    // combine the wavefronts through LDS: red[w][0..127] = o, [128] = l, [129] = m, [130] = bad
    if (lane < 16) {
#pragma unroll
        for (int j = 0; j < 8; ++j) red[wave * 132 + 8 * sub + j] = o[j];
    }
    if (lane == 0) {
        red[wave * 132 + 128] = l;
        red[wave * 132 + 129] = m;
        red[wave * 132 + 130] = wave_bad ? 1.f : 0.f;
    }
    __syncthreads();
    const size_t slot = part_slot(p, b, h, c);
    float M = p.phi;
    if constexpr (ONLINE) {
        M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, red[w * 132 + 129]);
    }
    bool flagged = false;
#pragma unroll
    for (int w = 0; w < NW; ++w) flagged |= red[w * 132 + 130] != 0.f;
    if (threadIdx.x < kHeadDim) {
        float acc = 0.f, lsum = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            float f = 1.f;
            if constexpr (ONLINE) {
                const float mw = red[w * 132 + 129];
                f = (mw == M) ? 1.f : exp2_hw((mw - M) * kLog2e);
            }
            acc += red[w * 132 + threadIdx.x] * f;
            lsum += red[w * 132 + 128] * f;
        }
        if (!direct) {
            part_store(p, p.o_part + slot * kHeadDim + threadIdx.x, acc);
        } else if (ONLINE || !flagged) {
            float vs = 1.f;
            if constexpr (KV == FD_FP8_E4M3FN) vs = p.v_scale[kvh];
            store_out(p, ((size_t)b * p.hq + h) * kHeadDim + threadIdx.x, t_end > t_begin ? acc * (vs / lsum) : 0.f);
        }
    }
    if (!direct && threadIdx.x == 0) {
        float lsum = 0.f;
        bool any = false;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            float f = 1.f;
            if constexpr (ONLINE) {
                const float mw = red[w * 132 + 129];
                f = (mw == M) ? 1.f : exp2_hw((mw - M) * kLog2e);
            }
            lsum += red[w * 132 + 128] * f;
            any |= red[w * 132 + 130] != 0.f;
        }
        part_store(p, p.l_part + slot, lsum);
        part_store(p, p.m_part + slot, M);
        if constexpr (!ONLINE) part_store(p, p.cflag + slot, (uint8_t)(any ? 1 : 0));
    }
    __syncthreads();   // `red` is reused by the caller
    return flagged;
}

// Grid (maxch, Hq, B): one workgroup per (chunk, query head, sequence).  The
// (x, y) position is read in dispatch order (x fastest) as query head fastest,
// then chunk, so consecutive workgroups write the partials of one chunk of a
// sequence, which are contiguous over the heads.
template <int KV, int QT, bool PAGED>
__global__ __launch_bounds__(256) void partial_valu_kernel(Params p)
{
    __shared__ float red[4 * 132];
    __shared__ int last_flag, merged;
    const size_t xy = (size_t)blockIdx.y * gridDim.x + blockIdx.x;
    const int h = (int)(xy % (size_t)p.hq), c = (int)(xy / (size_t)p.hq), b = blockIdx.z;
    if ((blockIdx.x | blockIdx.y | blockIdx.z | threadIdx.x) == 0) begin_call(p);
    const int L = seq_len_of(p, b);
    const int t0 = c * p.chunk;
    // chunks past the sequence have no unit; an empty sequence has one empty unit
    if (t0 >= L && !(c == 0 && L == 0)) return;
    const int t1 = min(t0 + p.chunk, L);
    // a score left the safe band: this workgroup redoes its chunk with online
    // softmax and overwrites the partial (the chunk flag stays set)
    // A row whose sequence is this one chunk (or empty) needs no merge: in a
    // fused call the workgroup writes its output and flag itself.
    const bool direct = p.fused && L <= p.chunk;
    const bool flagged = valu_chunk<KV, QT, PAGED, false, 4>(p, b, h, c, t0, t1, red, direct);
    if (flagged) valu_chunk<KV, QT, PAGED, true, 4>(p, b, h, c, t0, t1, red, direct);
    if (direct) {
        if (threadIdx.x == 0) {
            p.flags[(size_t)b * p.hq + h] = flagged ? 1 : 0;
            finish_group(p, flagged ? 1 : 0);
        }
    } else if (publish_unit(p, b * p.hq + h, units_of(p, L), last_flag)) {
        merge_group<4, 1>(p, b, h, 1, merged, chunk_parts(p, b, h, L));
    }
}

}  // namespace fd
