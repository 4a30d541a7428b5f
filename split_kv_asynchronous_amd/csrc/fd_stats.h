// Score statistics for choosing phi (FlashDecoding++ theory page, section 3:
// phi is set beforehand from the observed distribution of the scores).
//
// For every row (b, query head h) the largest and smallest valid score
// s_t = scale * <q, k_t> (fp8: k = code * k_scale), and optionally a histogram
// of all valid scores.  Only K is read.
//
// Work: one workgroup per (sequence b, KV head, block of query heads of that
// KV head, chunk of sp.chunk tokens).  Grouped bf16 queries over bf16 or
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
constexpr int kStatsWaves = 4;
// Tokens per workgroup.  The matrix-core kernel's unit is 512 KiB of K in
// either cache format (2048 bf16 or 4096 E4M3FN tokens): measured, extremes
// only, units of 2048 / 4096 / 8192 tokens ran at 5.41 / 4.63 / 5.32 TB/s on
// the 32K GQA bf16 workload and at 3.95 / 4.52 / 4.38 on the paged 16K
// E4M3FN one.
constexpr int kStatsChunk = 2048;
template <int KV> constexpr int stats_dma_chunk() { return KV == FD_FP8_E4M3FN ? 4096 : 2048; }

struct StatsParams {
    Params base;                   // q, k, lengths, block table, k_scale, shapes, scale
    float *row_max, *row_min;      // [B][Hq]
    uint32_t *hist;                // [nbins + 2] or nullptr
    int nbins;
    float hist_lo, hist_hi, inv_w; // inv_w = nbins / (hist_hi - hist_lo)
    int chunk;                     // tokens per workgroup
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

// One count into an LDS histogram bin, written out: the compiler cannot tell
// the bin from the ring slots the DMA is still filling and would wait for
// every DMA in flight before an atomic of its own (one drain per score).  The
// bins and the ring are disjoint; the add returns nothing, so nothing waits.
FD_DEV void lds_count(uint32_t *bin)
{
    asm volatile("ds_add_u32 %0, %1" : : "v"((uint32_t)(uintptr_t)bin), "v"(1u) : "memory");
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
    const int t_begin = c * sp.chunk;
    if (t_begin >= L) return;                     // the whole workgroup leaves together
    const int t_end = min(t_begin + sp.chunk, L);
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

// Query heads one matrix-core workgroup serves.
constexpr int kStatsMfmaHeads = 16;

// Grouped bf16 queries over a bf16 or E4M3FN cache: the scores of 16 tokens
// against up to 16 query heads come from four v_mfma_f32_16x16x32_bf16
// (S^T = K . Q^T, Q^T fragments in registers), so lane (n, g4) ends up
// holding 4 scores of head n and its extremes need no reduction across the
// lanes of a token.  Workgroup unit as above with blocks of 16 heads.  K
// moves by DMA (register loads of the fragments would read 64 bytes, or 32,
// of each of 16 rows per instruction, part of every cache line they touch;
// measured 4.45 against 5.37 TB/s, bf16, extremes only): each wavefront
// streams its compute groups (w, w + 4, ...: 16
// bf16 or 32 E4M3FN tokens, 4 KiB) through a ring of NST LDS stages with
// non-temporal 1 KiB buffer->LDS instructions over whole rows (the decode
// kernels' K tile and piece rotation, so the fragment reads are
// conflict-free), and reads the fragments back with ds_read_b128; E4M3FN
// codes are widened to bf16 exactly in registers.  Scores, extremes,
// histogram and the workgroup's exit as above.
template <int KV, bool PAGED, int NST>
__global__ __launch_bounds__(kStatsWaves * 64, 2) void score_stats_dma_kernel(StatsParams sp)
{
    using F = ring::Fmt<KV>;
    constexpr bool FP8 = KV == FD_FP8_E4M3FN;
    constexpr int ROWB = F::row;                   // bytes per K row
    constexpr int GRP = F::group;                  // tokens per compute group
    constexpr int RPI = 1024 / ROWB;               // rows per DMA instruction
    constexpr int LPR = 64 / RPI;                  // lanes per row in a DMA instruction
    constexpr int NT = FP8 ? 2 : 1;                // 16-token score tiles per group
    constexpr int STAGE = ring::kGroupBytes;
    extern __shared__ __attribute__((aligned(16))) uint8_t dyn[];
    __shared__ float red[kStatsWaves][2][kStatsMfmaHeads];
    const Params &p = sp.base;
    const int unit = blockIdx.x;
    const int c = unit % sp.nchunk;
    const int hb = (unit / sp.nchunk) % sp.nhb;
    const int bk = unit / (sp.nchunk * sp.nhb);
    const int b = bk / p.hkv, kvh = bk % p.hkv;
    const int L = seq_len_of(p, b);
    const int t_begin = c * sp.chunk;
    if (t_begin >= L) return;                     // the whole workgroup leaves together
    const int t_end = min(t_begin + sp.chunk, L);
    const int h0 = kvh * p.group + hb * kStatsMfmaHeads;
    const int nh = min(kStatsMfmaHeads, p.group - hb * kStatsMfmaHeads);

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15;
    const int g4 = lane >> 4;
    const bool head_ok = n < nh;
    uint8_t *ring = dyn + wave * (NST * STAGE);
    uint32_t *lhist = reinterpret_cast<uint32_t *>(dyn + kStatsWaves * NST * STAGE);

    if (sp.hist) {
        for (int i = threadIdx.x; i < sp.nbins + 2; i += kStatsWaves * 64) lhist[i] = 0u;
        __syncthreads();
    }

    const int ngroups = (t_end - t_begin + GRP - 1) / GRP;
    const int nmine = ngroups > wave ? (ngroups - wave + kStatsWaves - 1) / kStatsWaves : 0;
    const uint8_t *kpool = static_cast<const uint8_t *>(p.k);
    // this wavefront's i-th group into ring slot `slot`: instruction q moves
    // rows RPI*q .. RPI*q + RPI-1, lane l fetching, of row RPI*q + l/LPR, the
    // piece that belongs in LDS slot l%LPR; rows past the sequence re-read its
    // last row (their scores are never used).  The rows of one instruction
    // never straddle a page (pages hold at least 16 tokens).
    auto issue = [&](int i, int slot) {
        const int tg = t_begin + GRP * (wave + kStatsWaves * i);
        const int last = t_end - 1 - tg;
        uint8_t *dst = ring + slot * STAGE;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = RPI * q + lane / LPR;                 // group row
            const int t = tg + (r < last ? r : last);           // its token (clamped)
            size_t row;
            if constexpr (PAGED) {
                // every clamped token of the instruction lies in the page of
                // tp: its 16-row half's first token, or the last valid token
                const int tp = min(tg + 16 * (RPI * q / 16), t_end - 1);
                const int P = 1 << p.page_shift;
                const int page = as_const(p.block_table)[(size_t)b * p.max_blocks + (tp >> p.page_shift)];
                row = ((size_t)page * p.hkv + kvh) * P + (t & (P - 1));
            } else {
                row = ((size_t)b * p.hkv + kvh) * p.max_seq_len + t;
            }
            const uint8_t *src = kpool + row * ROWB + 16 * ((lane % LPR - F::rot(r)) & (F::slots - 1));
            ring::lds_void *d = (ring::lds_void *)(dst + 1024 * q);
            __builtin_amdgcn_global_load_lds(src, d, 16, 0, ring::kStreamPolicy);
        }
    };
#pragma unroll
    for (int k = 0; k < NST; ++k)
        if (k < nmine) issue(k, k);

    // Q^T fragments, loaded after the prologue in one statement with their
    // wait; heads past the block read a valid row and are zeroed.  The k
    // index of MFMA step kk: bf16 component 8*g4 + 32*kk + j, E4M3FN
    // 16*(g4 + 4*(kk/2)) + 8*(kk%2) + j (the K pieces' map)
    u32x4 qf[4];
    {
        const uint16_t *qrow = static_cast<const uint16_t *>(p.q) +
                               ((size_t)b * p.hq + h0 + (head_ok ? n : 0)) * kHeadDim + (FP8 ? 16 : 8) * g4;
        if constexpr (FP8)
            asm volatile("global_load_dwordx4 %0, %4, off\n\t"
                         "global_load_dwordx4 %1, %4, off offset:16\n\t"
                         "global_load_dwordx4 %2, %4, off offset:128\n\t"
                         "global_load_dwordx4 %3, %4, off offset:144\n\t"
                         "s_waitcnt vmcnt(0)"
                         : "=&v"(qf[0]), "=&v"(qf[1]), "=&v"(qf[2]), "=&v"(qf[3])
                         : "v"(qrow)
                         : "memory");
        else
            asm volatile("global_load_dwordx4 %0, %4, off\n\t"
                         "global_load_dwordx4 %1, %4, off offset:64\n\t"
                         "global_load_dwordx4 %2, %4, off offset:128\n\t"
                         "global_load_dwordx4 %3, %4, off offset:192\n\t"
                         "s_waitcnt vmcnt(0)"
                         : "=&v"(qf[0]), "=&v"(qf[1]), "=&v"(qf[2]), "=&v"(qf[3])
                         : "v"(qrow)
                         : "memory");
        if (!head_ok) {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) qf[kk] = u32x4{0u, 0u, 0u, 0u};
        }
    }
    float sc = p.scale;
    if constexpr (FP8) sc *= as_const(p.k_scale)[kvh];
    // fragment reads: bf16 step kk -> row n, piece g4 + 4kk; E4M3FN tile tau,
    // half m -> row 16 tau + n, piece g4 + 4m (16 codes = steps 2m and 2m+1)
    uint32_t k_rd[4];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
        if constexpr (FP8) {
            const int r = 16 * (q4 >> 1) + n;
            k_rd[q4] = r * ROWB + 16 * ((g4 + 4 * (q4 & 1) + F::rot(r)) & (F::slots - 1));
        } else {
            k_rd[q4] = n * ROWB + 16 * ((g4 + 4 * q4 + F::rot(n)) & (F::slots - 1));
        }
    }

    float mx = -INFINITY, mn = INFINITY;
    int slot = 0;
#pragma unroll 1
    for (int i = 0; i < nmine; ++i) {
        // this group's DMAs done; up to NST - 1 later groups stay in flight
        const int ahead = min(NST - 1, nmine - 1 - i);
        ring::wait_ring<4, NST - 1>(ahead);
        const uint32_t sb = (uint32_t)(uintptr_t)(ring + slot * STAGE);
        uint32_t a4[4];
        u32x4 kr[4];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) a4[q4] = sb + k_rd[q4];
        ring::lds_read4(a4, kr);
        if (i + NST < nmine) issue(i + NST, slot);
        slot = slot + 1 == NST ? 0 : slot + 1;
        const int tg = t_begin + GRP * (wave + kStatsWaves * i);
#pragma unroll
        for (int tau = 0; tau < NT; ++tau) {
            f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                u32x4 kf;
                if constexpr (FP8) {
                    const u32x4 r = kr[2 * tau + (kk >> 1)];
                    kf = (kk & 1) ? ring::e4m3x8_to_bf16(r.z, r.w) : ring::e4m3x8_to_bf16(r.x, r.y);
                } else {
                    kf = kr[kk];
                }
                s = mfma_bf16(kf, qf[kk], s);
            }
            // lane (n, g4) holds tokens 16 tau + 4 g4 + r of the group, head n
            const int t0 = tg + 16 * tau + 4 * g4;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float x = s[r] * sc;
                if (head_ok && t0 + r < t_end) {
                    mx = fmaxf(mx, x);
                    mn = fminf(mn, x);
                    if (sp.hist) lds_count(&lhist[hist_slot(sp, x)]);
                }
            }
        }
    }

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
