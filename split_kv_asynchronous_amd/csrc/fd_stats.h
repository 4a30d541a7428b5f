// Score statistics for choosing phi (FlashDecoding++ theory page, section 3:
// phi is set beforehand from the observed distribution of the scores).
//
// For every row (b, query head h) the largest and smallest valid score
// s_t = scale * <q, k_t> (fp8: k = code * k_scale), and optionally a histogram
// of all valid scores.  Only K is read.
//
// Work: one workgroup per (sequence b, KV head, block of query heads of that
// KV head, chunk of kStatsChunk tokens).  Grouped bf16 queries over bf16 or
// E4M3FN caches take the matrix-core kernel at the end of this file; the
// rest take the vector kernel, with the lane mapping of the vector decode
// kernel: a wavefront splits into four 16-lane rows,
// each row holds one token at a time with 8 of its 128 components per lane,
// and the 16-lane dot product is finished with four DPP adds, so all 16 lanes
// of a row hold the same score.  Extremes are combined over the rows and
// wavefronts in registers and LDS and leave the workgroup as one global
// atomic per query head; the histogram is accumulated in LDS (one atomic per
// score, issued by the row's first lane) and flushed with one global atomic
// per non-empty bin.
#pragma once

#include "fd_common.h"
#include "fd_mfma.h"
#include "fd_ring.h"

namespace fd {
namespace stats {

constexpr int kStatsHeads = 8;      // query heads per workgroup
constexpr int kStatsChunk = 2048;   // tokens per workgroup
constexpr int kStatsWaves = 4;

struct StatsParams {
    Params base;                   // q, k, lengths, block table, k_scale, shapes, scale
    float *row_max, *row_min;      // [B][Hq]
    uint32_t *hist;                // [nbins + 2] or nullptr
    int nbins;
    float hist_lo, hist_hi, inv_w; // inv_w = nbins / (hist_hi - hist_lo)
    int nchunk;                    // chunks per sequence (grid)
    int nhb;                       // head blocks per KV head
};

// Float max/min through compare-and-swap on the bit pattern (vector atomics).
FD_DEV void atomic_max_f32(float *addr, float v)
{
    unsigned *a = reinterpret_cast<unsigned *>(addr);
    unsigned old = __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    while (__uint_as_float(old) < v) {
        if (__hip_atomic_compare_exchange_strong(a, &old, __float_as_uint(v), __ATOMIC_RELAXED,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
            break;
    }
}

FD_DEV void atomic_min_f32(float *addr, float v)
{
    unsigned *a = reinterpret_cast<unsigned *>(addr);
    unsigned old = __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    while (__uint_as_float(old) > v) {
        if (__hip_atomic_compare_exchange_strong(a, &old, __float_as_uint(v), __ATOMIC_RELAXED,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
            break;
    }
}

// Outputs before the pass: extremes -inf / +inf, histogram 0.
__global__ __launch_bounds__(256) void stats_init_kernel(StatsParams p)
{
    const int rows = p.base.batch * p.base.hq;
    for (int i = blockIdx.x * 256 + threadIdx.x; i < rows; i += gridDim.x * 256) {
        p.row_max[i] = -INFINITY;
        p.row_min[i] = INFINITY;
    }
    if (p.hist)
        for (int i = blockIdx.x * 256 + threadIdx.x; i < p.nbins + 2; i += gridDim.x * 256) p.hist[i] = 0u;
}

// Histogram slot of a score: 0 below hist_lo (and NaN), 1 + i for bin i,
// nbins + 1 at or above hist_hi.
FD_DEV int hist_slot(const StatsParams &p, float s)
{
    if (!(s >= p.hist_lo)) return 0;
    if (s >= p.hist_hi) return p.nbins + 1;
    int i = (int)floorf((s - p.hist_lo) * p.inv_w);
    i = i < 0 ? 0 : (i >= p.nbins ? p.nbins - 1 : i);
    return 1 + i;
}

// Grid: one workgroup per unit, unit = ((b * Hkv + kvh) * nhb + hb) * nchunk + c.
// Dynamic LDS: nbins + 2 counters when a histogram is taken.
template <int KV, int QT, bool PAGED>
__global__ __launch_bounds__(kStatsWaves * 64) void score_stats_kernel(StatsParams sp)
{
    extern __shared__ uint32_t lhist[];
    __shared__ float red[kStatsWaves][2][kStatsHeads];
    const Params &p = sp.base;
    const int unit = blockIdx.x;
    const int c = unit % sp.nchunk;
    const int hb = (unit / sp.nchunk) % sp.nhb;
    const int bk = unit / (sp.nchunk * sp.nhb);
    const int b = bk / p.hkv, kvh = bk % p.hkv;
    const int L = seq_len_of(p, b);
    const int t_begin = c * kStatsChunk;
    if (t_begin >= L) return;                     // the whole workgroup leaves together
    const int t_end = min(t_begin + kStatsChunk, L);
    const int h0 = kvh * p.group + hb * kStatsHeads;
    const int nh = min(kStatsHeads, p.group - hb * kStatsHeads);

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int row = lane >> 4;          // token slot inside the wavefront
    const int sub = lane & 15;          // components 8*sub .. 8*sub+7

    if (sp.hist) {
        for (int i = threadIdx.x; i < sp.nbins + 2; i += kStatsWaves * 64) lhist[i] = 0u;
        __syncthreads();
    }

    float sc = p.scale;
    if constexpr (KV == FD_FP8_E4M3FN) sc *= as_const(p.k_scale)[kvh];
    float q[kStatsHeads][8];
#pragma unroll
    for (int hh = 0; hh < kStatsHeads; ++hh) {
        const int h = h0 + (hh < nh ? hh : 0);   // heads past the block repeat a valid one
        load8<QT>(p.q, ((size_t)b * p.hq + h) * kHeadDim + 8 * sub, q[hh]);
    }
    float mx[kStatsHeads], mn[kStatsHeads];
#pragma unroll
    for (int hh = 0; hh < kStatsHeads; ++hh) {
        mx[hh] = -INFINITY;
        mn[hh] = INFINITY;
    }

    constexpr int U = 2;                              // tokens per row per step
    constexpr int STEP = kStatsWaves * 4 * U;         // tokens per workgroup step
#pragma unroll 1
    for (int base = t_begin; base < t_end; base += STEP) {
        float kx[U][8];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int t = base + (wave * U + u) * 4 + row;
            const int tl = t < t_end ? t : t_end - 1;    // stay inside the sequence
            load8<KV, true>(p.k, kv_offset<PAGED>(p, b, kvh, tl) + 8 * sub, kx[u]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int t = base + (wave * U + u) * 4 + row;
            const bool valid = t < t_end;
#pragma unroll
            for (int hh = 0; hh < kStatsHeads; ++hh) {
                if (hh >= nh) break;
                float part = 0.f;
#pragma unroll
                for (int j = 0; j < 8; ++j) part = fmaf(q[hh][j], kx[u][j], part);
                const float s = row16_sum(part) * sc;
                if (valid) {
                    mx[hh] = fmaxf(mx[hh], s);
                    mn[hh] = fminf(mn[hh], s);
                    if (sp.hist && sub == 0) atomicAdd(&lhist[hist_slot(sp, s)], 1u);
                }
            }
        }
    }

    // extremes over the four rows of the wavefront, then over the wavefronts
#pragma unroll
    for (int hh = 0; hh < kStatsHeads; ++hh) {
        mx[hh] = fmaxf(mx[hh], __shfl_xor(mx[hh], 16));
        mx[hh] = fmaxf(mx[hh], __shfl_xor(mx[hh], 32));
        mn[hh] = fminf(mn[hh], __shfl_xor(mn[hh], 16));
        mn[hh] = fminf(mn[hh], __shfl_xor(mn[hh], 32));
    }
    if (lane == 0) {
#pragma unroll
        for (int hh = 0; hh < kStatsHeads; ++hh) {
            red[wave][0][hh] = mx[hh];
            red[wave][1][hh] = mn[hh];
        }
    }
    __syncthreads();
    if (threadIdx.x < nh) {
        const int hh = threadIdx.x;
        float M = -INFINITY, m = INFINITY;
#pragma unroll
        for (int w = 0; w < kStatsWaves; ++w) {
            M = fmaxf(M, red[w][0][hh]);
            m = fminf(m, red[w][1][hh]);
        }
        const size_t r = (size_t)b * p.hq + h0 + hh;
        atomic_max_f32(sp.row_max + r, M);
        atomic_min_f32(sp.row_min + r, m);
    }
    if (sp.hist) {
        for (int i = threadIdx.x; i < sp.nbins + 2; i += kStatsWaves * 64) {
            const uint32_t v = lhist[i];
            if (v) atomicAdd(sp.hist + i, v);
        }
    }
}

// Grouped queries with bf16 queries and a bf16 or E4M3FN cache: the scores of
// 16 tokens against up to 16 query heads come from four
// v_mfma_f32_16x16x32_bf16 (S^T = K . Q^T, A = K rows read straight from
// global memory, B = the heads' Q^T fragments held in registers; E4M3FN codes
// widened to bf16 exactly), so lane (n, g4) ends up holding 4 scores of head
// n: its extremes need no reduction across lanes of a token.  Workgroup unit
// as above with blocks of 16 heads; wavefront w takes the 16-token groups
// w, w + 4, ... of the chunk, GU groups per step.
constexpr int kStatsMfmaHeads = 16;

template <int KV, bool PAGED>
__global__ __launch_bounds__(kStatsWaves * 64) void score_stats_mfma_kernel(StatsParams sp)
{
    constexpr bool FP8 = KV == FD_FP8_E4M3FN;
    constexpr int GU = 4;                          // 16-token groups per wavefront per step
    extern __shared__ uint32_t lhist[];
    __shared__ float red[kStatsWaves][2][kStatsMfmaHeads];
    const Params &p = sp.base;
    const int unit = blockIdx.x;
    const int c = unit % sp.nchunk;
    const int hb = (unit / sp.nchunk) % sp.nhb;
    const int bk = unit / (sp.nchunk * sp.nhb);
    const int b = bk / p.hkv, kvh = bk % p.hkv;
    const int L = seq_len_of(p, b);
    const int t_begin = c * kStatsChunk;
    if (t_begin >= L) return;                     // the whole workgroup leaves together
    const int t_end = min(t_begin + kStatsChunk, L);
    const int h0 = kvh * p.group + hb * kStatsMfmaHeads;
    const int nh = min(kStatsMfmaHeads, p.group - hb * kStatsMfmaHeads);

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int n = lane & 15;
    const int g4 = lane >> 4;
    const bool head_ok = n < nh;

    if (sp.hist) {
        for (int i = threadIdx.x; i < sp.nbins + 2; i += kStatsWaves * 64) lhist[i] = 0u;
        __syncthreads();
    }

    // Q^T fragments: the k index of MFMA step kk is component 8*g4 + 32*kk + j;
    // heads past the block are zero
    u32x4 qf[4];
    {
        const u32x4 *qrow = reinterpret_cast<const u32x4 *>(
            static_cast<const uint16_t *>(p.q) + ((size_t)b * p.hq + h0 + (head_ok ? n : 0)) * kHeadDim);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) qf[kk] = head_ok ? qrow[g4 + 4 * kk] : u32x4{0u, 0u, 0u, 0u};
    }
    float sc = p.scale;
    if constexpr (FP8) sc *= as_const(p.k_scale)[kvh];

    float mx = -INFINITY, mn = INFINITY;
    const int ngroups = (t_end - t_begin + 15) / 16;
#pragma unroll 1
    for (int g0 = wave; g0 < ngroups; g0 += kStatsWaves * GU) {
        // K fragments of GU groups: lane (n, g4) reads row n of the group,
        // components 8*g4 + 32*kk .. +7 (bf16: 16 bytes; E4M3FN: 8 codes)
        u32x4 kb[GU][4];
        u32x2 k8[GU][4];
#pragma unroll
        for (int u = 0; u < GU; ++u) {
            const int g = g0 + u * kStatsWaves;
            int t = t_begin + 16 * g + n;
            t = t < t_end ? t : t_end - 1;             // stay inside the sequence
            const uint8_t *row = static_cast<const uint8_t *>(p.k) + kv_offset<PAGED>(p, b, kvh, t) * (FP8 ? 1 : 2);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                if constexpr (FP8)
                    k8[u][kk] = *reinterpret_cast<const u32x2 *>(row + 8 * g4 + 32 * kk);
                else
                    kb[u][kk] = *reinterpret_cast<const u32x4 *>(row + 2 * (8 * g4 + 32 * kk));
            }
        }
#pragma unroll
        for (int u = 0; u < GU; ++u) {
            const int g = g0 + u * kStatsWaves;
            if (g >= ngroups) break;                   // wave-uniform
            f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const u32x4 a = FP8 ? ring::e4m3x8_to_bf16(k8[u][kk].x, k8[u][kk].y) : kb[u][kk];
                s = mfma_bf16(a, qf[kk], s);
            }
            // lane (n, g4) holds tokens 16g + 4g4 + r of head n
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = t_begin + 16 * g + 4 * g4 + r;
                const float x = s[r] * sc;
                if (head_ok && t < t_end) {
                    mx = fmaxf(mx, x);
                    mn = fminf(mn, x);
                    if (sp.hist) atomicAdd(&lhist[hist_slot(sp, x)], 1u);
                }
            }
        }
    }

    // extremes of head n over the four lane groups, then over the wavefronts
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    mn = fminf(mn, __shfl_xor(mn, 16));
    mn = fminf(mn, __shfl_xor(mn, 32));
    if (g4 == 0) {
        red[wave][0][n] = mx;
        red[wave][1][n] = mn;
    }
    __syncthreads();
    if (threadIdx.x < nh) {
        const int hh = threadIdx.x;
        float M = -INFINITY, m = INFINITY;
#pragma unroll
        for (int w = 0; w < kStatsWaves; ++w) {
            M = fmaxf(M, red[w][0][hh]);
            m = fminf(m, red[w][1][hh]);
        }
        const size_t r = (size_t)b * p.hq + h0 + hh;
        atomic_max_f32(sp.row_max + r, M);
        atomic_min_f32(sp.row_min + r, m);
    }
    if (sp.hist) {
        for (int i = threadIdx.x; i < sp.nbins + 2; i += kStatsWaves * 64) {
            const uint32_t v = lhist[i];
            if (v) atomicAdd(sp.hist + i, v);
        }
    }
}

}  // namespace stats
}  // namespace fd
