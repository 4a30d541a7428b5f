// Grouped-query chunk kernel, bf16 cache: K and V stream through a per-wave
// LDS ring filled by coalesced buffer->LDS DMA; both contractions run on the
// matrix cores.
//
// Work decomposition.  A unit is (sequence b, head block hb, chunk c).  The
// grid is an upper bound on the number of units; workgroup i takes the i-th
// real unit of the list "all full chunks, then all partial last chunks", so
// workgroups past the end exit at once and no launch slot in the middle of the
// grid is wasted on a chunk beyond its sequence.
//
// Shape <NW, NSUB, NST>: NW wavefronts per workgroup; a ring block holds NSUB
// 16-token sub-tiles of K and of V; each wavefront owns an NST-stage ring.
// The blocks of a unit are dealt round-robin to the wavefronts.  Per block:
//   * 4*NSUB DMA instructions per tile, each moving 4 whole cache rows (1 KiB,
//     fully coalesced) into LDS; the 16-byte pieces of a row are rotated by
//     rot(t) so that the fragment reads below are free of bank conflicts;
//   * the block's fragments are read out of the stage at once (4 ds_read_b128
//     K fragments and 8 ds_read_b64_tr_b16 V^T fragments per sub-tile) and
//     the stage is refilled before any arithmetic;
//   * per sub-tile: S^T[16 tok x 16 heads] = K . Q^T on 4
//     v_mfma_f32_16x16x32_bf16; band test, p = exp(s - phi) and the weight sums
//     in registers; p split into a bf16 high part and a bf16 remainder;
//     O^T[128 x 16 heads] += V^T . P^T on 8 x 2 v_mfma_f32_16x16x16_bf16.
#pragma once

#include <type_traits>

#include "fd_common.h"
#include "fd_mfma.h"

#ifndef FD_CHUNK_WAVES
#define FD_CHUNK_WAVES 4
#endif
#ifndef FD_CHUNK_SUBTILES
#define FD_CHUNK_SUBTILES 1
#endif
#ifndef FD_CHUNK_STAGES
#define FD_CHUNK_STAGES 2
#endif

namespace fd {

namespace chunk {

constexpr int kRow = kHeadDim * 2;                 // bytes per bf16 cache row
constexpr int kSubTile = 16 * kRow;                // 16 rows: 4 KiB
constexpr int kRedStride = 16 * kHeadDim + 32;     // one wave's O^T, then l and flag-or-max per head

template <int NW, int NSUB, int NST>
struct Shape {
    static constexpr int waves = NW;
    static constexpr int nsub = NSUB;
    static constexpr int nst = NST;
    static constexpr int blk = 16 * NSUB;              // tokens per ring block
    static constexpr int tile = NSUB * kSubTile;       // K (or V) part of a block
    static constexpr int stage = 2 * tile;
    static constexpr int wave_lds = NST * stage;
    static constexpr int lds = NW * wave_lds;
    static constexpr int dma_per_block = 2 * (blk / 4);  // 1 KiB per DMA instruction
    static_assert(NST * dma_per_block < 64, "vmcnt cannot count that deep");
    static_assert(NW * kRedStride * 4 <= lds, "epilogue reduction must fit in the ring");
    static_assert(lds <= 160 * 1024, "LDS per workgroup");
};

using DefaultShape = Shape<FD_CHUNK_WAVES, FD_CHUNK_SUBTILES, FD_CHUNK_STAGES>;

typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8])
template <int N>
FD_DEV void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// wait until at most k ring blocks (of D DMA instructions each) are in flight
template <int D, int KMAX>
FD_DEV void wait_ring(int k)
{
    if (KMAX > 3 && k >= 4) wait_vmcnt<(KMAX > 3 ? 4 * D : 0)>();
    else if (KMAX > 2 && k == 3) wait_vmcnt<(KMAX > 2 ? 3 * D : 0)>();
    else if (KMAX > 1 && k == 2) wait_vmcnt<(KMAX > 1 ? 2 * D : 0)>();
    else if (KMAX > 0 && k == 1) wait_vmcnt<D>();
    else wait_vmcnt<0>();
}

// rotation of the 16-byte pieces of row t (0..15) of a sub-tile
FD_DEV int rot_of(int t) { return 2 * (t & 3) + ((t >> 2) & 1); }

FD_DEV f32x4 mfma16(u32x2 a, u32x2 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                     __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

// wave-wide inclusive prefix sum
FD_DEV int wave_scan(int x, int lane)
{
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d);
        if (lane >= d) x += y;
    }
    return x;
}

struct Unit {
    int b, hb, c;
    bool ok;
};

// The u-th unit of "full chunks of every sequence, then the partial last
// chunks", sequence-major inside each part, head blocks outer, chunks inner.
FD_DEV Unit find_unit(const Params &p, int u, int nhb, int lane)
{
    Unit r = {0, 0, 0, false};
    int base = 0;
#pragma unroll 1
    for (int part = 0; part < 2; ++part) {
#pragma unroll 1
        for (int b0 = 0; b0 < p.batch; b0 += 64) {
            const int b = b0 + lane;
            int cnt = 0;
            if (b < p.batch) {
                const int L = seq_len_of(p, b);
                cnt = part == 0 ? (L / p.chunk) * nhb : ((L % p.chunk) ? nhb : 0);
            }
            const int incl = wave_scan(cnt, lane);
            const int total = __shfl(incl, 63);
            if (u < base + total) {
                const uint64_t m = __ballot(base + incl > u);
                const int hit = __builtin_ctzll(m);
                const int before = base + __shfl(incl - cnt, hit);
                const int bb = b0 + hit;
                const int L = seq_len_of(p, bb);
                const int rem = u - before;
                r.b = bb;
                if (part == 0) {
                    const int F = L / p.chunk;
                    r.hb = rem / F;
                    r.c = rem % F;
                } else {
                    r.hb = rem;
                    r.c = L / p.chunk;
                }
                r.ok = true;
                return r;
            }
            base += total;
        }
    }
    return r;
}

template <bool PAGED, typename S>
__global__ __launch_bounds__(S::waves * 64, 2) void chunk_bf16_kernel(Params p)
{
    constexpr int NW = S::waves;
    constexpr int NSUB = S::nsub;
    constexpr int NST = S::nst;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[S::lds];
    __shared__ int flagged_heads;
    if ((blockIdx.x | threadIdx.x) == 0) *p.counter = 0;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15;
    const int g4 = lane >> 4;
    const int GB = p.heads_per_block;
    const int nhb = p.hq / GB;

    const Unit U = find_unit(p, blockIdx.x, nhb, lane);
    if (!U.ok) return;
    const int b = __builtin_amdgcn_readfirstlane(U.b);
    const int hb = __builtin_amdgcn_readfirstlane(U.hb);
    const int c = __builtin_amdgcn_readfirstlane(U.c);
    const int L = seq_len_of(p, b);
    const int t_begin = c * p.chunk;
    const int t_end = min(t_begin + p.chunk, L);
    const int h0 = hb * GB;
    const int kvh = h0 / p.group;
    const bool head_ok = n < GB;

    // Q^T fragments (B operand of the S product)
    u32x4 qf[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        qf[kk] = u32x4{0u, 0u, 0u, 0u};
        if (head_ok)
            qf[kk] = *reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(p.q) +
                                                      ((size_t)b * p.hq + h0 + n) * kHeadDim +
                                                      8 * g4 + 32 * kk);
    }
    const float sc = p.scale;
    const float nphi = -p.phi * kLog2e;

    // ---- DMA addressing: instruction i of a tile moves rows 4i .. 4i+3; lane
    // (n, g4) fetches piece (n - rot) & 15 of row 4i + g4 so that LDS slot n of
    // that row holds it (rot depends on the row's parity within a sub-tile)
    const uint32_t dma_voff_even = g4 * kRow + 16 * ((n - rot_of(g4)) & 15);
    const uint32_t dma_voff_odd = g4 * kRow + 16 * ((n - rot_of(4 + g4)) & 15);
    uint8_t *ring = lds + wave * S::wave_lds;

    __amdgpu_buffer_rsrc_t krs, vrs;
    const uint8_t *kpool = static_cast<const uint8_t *>(p.k);
    const uint8_t *vpool = static_cast<const uint8_t *>(p.v);
    const __attribute__((address_space(4))) int32_t *btab = as_const(p.block_table);
    if constexpr (!PAGED) {
        const size_t slice = ((size_t)b * p.hkv + kvh) * (size_t)p.max_seq_len * kRow;
        const int nrec = (int)((uint32_t)L * kRow);
        krs = __builtin_amdgcn_make_buffer_rsrc((void *)(kpool + slice), (short)0, nrec, 0x00020000);
        vrs = __builtin_amdgcn_make_buffer_rsrc((void *)(vpool + slice), (short)0, nrec, 0x00020000);
    } else {
        btab += (size_t)b * p.max_blocks;
    }
    const int last_page = (L - 1) >> p.page_shift;
    const int pmask = (1 << p.page_shift) - 1;

    const int nblk = (t_end - t_begin + S::blk - 1) / S::blk;

    auto issue = [&](int j, int stage) {
        uint8_t *kt = ring + stage * S::stage;
        uint8_t *vt = kt + S::tile;
#pragma unroll
        for (int u = 0; u < NSUB; ++u) {
            const int t0 = t_begin + S::blk * j + 16 * u;
            size_t page_off = 0;
            if constexpr (PAGED) {
                // a 16-token sub-tile never straddles a page (pages hold >= 16 tokens)
                int idx = t0 >> p.page_shift;
                idx = idx < last_page ? idx : last_page;
                page_off = (((size_t)btab[idx] * p.hkv + kvh) * (size_t)(pmask + 1) + (t0 & pmask)) * kRow;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t vo = (i & 1) ? dma_voff_odd : dma_voff_even;
                lds_void *kd = (lds_void *)(kt + u * kSubTile + i * 1024);
                lds_void *vd = (lds_void *)(vt + u * kSubTile + i * 1024);
                if constexpr (PAGED) {
                    __builtin_amdgcn_global_load_lds(kpool + page_off + i * 4 * kRow + vo, kd, 16, 0, 0);
                    __builtin_amdgcn_global_load_lds(vpool + page_off + i * 4 * kRow + vo, vd, 16, 0, 0);
                } else {
                    const int so = (int)((uint32_t)(t0 + 4 * i) * kRow);
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, kd, 16, vo, so, 0, 0);
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, vd, 16, vo, so, 0, 0);
                }
            }
        }
    };

    // fragment read addresses inside a sub-tile (bytes)
    // K: lane (n, g4), k-step kk: row n, piece g4 + 4kk
    uint32_t k_rd[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) k_rd[kk] = n * kRow + 16 * ((g4 + 4 * kk + rot_of(n)) & 15);
    // V (transposing read): lane i of group g4 addresses row 4g4 + i/4,
    // components 16dt + 4(i%4) .. +3, i.e. half (i & 1) of piece 2dt + (i%4)/2
    const int vt_tok = 4 * g4 + (n >> 2);
    uint32_t v_rd[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
        v_rd[dt] = vt_tok * kRow + 8 * (n & 1) + 16 * ((2 * dt + ((n & 3) >> 1) + rot_of(vt_tok)) & 15);

    float *red = reinterpret_cast<float *>(lds);

    // One pass over the unit's blocks.  ONLINE == false: weights exp(s - phi)
    // against the preset constant, band test per head.  ONLINE == true: the
    // ordinary running-maximum softmax, the maximum advanced once per
    // sub-tile.  Leaves this wave's O^T, weight sum, and band flag (or running
    // maximum) in red[wave].
    auto run = [&](auto online_tag) {
        constexpr bool ONLINE = decltype(online_tag)::value;
        f32x4 o[8];
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        float lsum = 0.f;
        float mrun = -INFINITY;     // ONLINE: running maximum of head n (same in all 4 lane groups)
        int bad = 0;

        int j = wave;
        int issued = 0;
#pragma unroll
        for (int k = 0; k < NST; ++k)
            if (j + k * NW < nblk) {
                issue(j + k * NW, k);
                ++issued;
            }
        // the query loads were issued before the ring prologue: once at most
        // the prologue's DMAs are outstanding, the queries have arrived
        wait_ring<S::dma_per_block, NST>(issued);
        int stage = 0;
#pragma unroll 1
        for (; j < nblk; j += NW) {
            // this block's DMAs done; up to NST-1 later blocks stay in flight
            const int ahead = (nblk - 1 - j) / NW;
            wait_ring<S::dma_per_block, NST - 1>(ahead < NST - 1 ? ahead : NST - 1);
            const uint8_t *kt = ring + stage * S::stage;
            const uint8_t *vt = kt + S::tile;

            // Pull the whole block out of the stage first and hand the stage
            // back to the DMA engine before any arithmetic.  The reads are
            // inline assembly: the compiler cannot tell them apart from ring
            // slots still being filled and would drain every DMA in flight
            // before them; the explicit waits here do the ordering instead.
            u32x4 kf[NSUB][4];
            u32x2 va[NSUB][8];
#pragma unroll
            for (int u = 0; u < NSUB; ++u) {
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const uint32_t addr = (uint32_t)(uintptr_t)(kt + u * kSubTile + k_rd[kk]);
                    asm volatile("ds_read_b128 %0, %1" : "=v"(kf[u][kk]) : "v"(addr) : "memory");
                }
#pragma unroll
                for (int dt = 0; dt < 8; ++dt) {
                    const uint32_t addr = (uint32_t)(uintptr_t)(vt + u * kSubTile + v_rd[dt]);
                    asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(va[u][dt]) : "v"(addr) : "memory");
                }
            }
            // all reads of the stage have returned (the fragments are tied to
            // this wait so no use moves above it); refill the stage
#pragma unroll
            for (int u = 0; u < NSUB; ++u)
                asm volatile("s_waitcnt lgkmcnt(0)"
                             : "+v"(va[u][0]), "+v"(va[u][1]), "+v"(va[u][2]), "+v"(va[u][3]),
                               "+v"(va[u][4]), "+v"(va[u][5]), "+v"(va[u][6]), "+v"(va[u][7]),
                               "+v"(kf[u][0]), "+v"(kf[u][1]), "+v"(kf[u][2]), "+v"(kf[u][3])
                             :
                             : "memory");
            if (j + NST * NW < nblk) issue(j + NST * NW, stage);
            stage = stage + 1 == NST ? 0 : stage + 1;

#pragma unroll
            for (int u = 0; u < NSUB; ++u) {
                // S^T: rows = tokens 4*g4 + r of the sub-tile, column = head n
                f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) s = mfma_bf16(kf[u][kk], qf[kk], s);
                const int t0 = t_begin + S::blk * j + 16 * u;
                float w[4];
                if constexpr (!ONLINE) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const bool valid = t0 + 4 * g4 + r < t_end;
                        const float sv = s[r] * sc;
                        bad |= (int)valid & (int)outside_band(sv, p.lo, p.hi);
                        const float e = exp2_hw(fmaf(sv, kLog2e, nphi));
                        w[r] = valid ? e : 0.f;
                        lsum += w[r];
                    }
                } else {
                    float sv[4], mx = -INFINITY;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const bool valid = t0 + 4 * g4 + r < t_end;
                        sv[r] = valid ? s[r] * sc : -INFINITY;
                        mx = fmaxf(mx, sv[r]);
                    }
                    mx = fmaxf(mx, __shfl_xor(mx, 16));
                    mx = fmaxf(mx, __shfl_xor(mx, 32));
                    const float mnew = fmaxf(mrun, mx);
                    const float f = (mrun == mnew) ? 1.f : exp2_hw((mrun - mnew) * kLog2e);
#pragma unroll
                    for (int dt = 0; dt < 8; ++dt) o[dt] *= f;
                    lsum *= f;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        w[r] = (sv[r] == -INFINITY) ? 0.f : exp2_hw((sv[r] - mnew) * kLog2e);
                        lsum += w[r];
                    }
                    mrun = mnew;
                }
                uint32_t h01, h23, l01, l23;
                split_pair(w[0], w[1], h01, l01);
                split_pair(w[2], w[3], h23, l23);
                const u32x2 ph = {h01, h23}, pl = {l01, l23};
#pragma unroll
                for (int dt = 0; dt < 8; ++dt) {
                    o[dt] = mfma16(va[u][dt], ph, o[dt]);
                    o[dt] = mfma16(va[u][dt], pl, o[dt]);
                }
            }
        }

        // per-head weight sums and flags over the 4 lane groups
        lsum += __shfl_xor(lsum, 16);
        lsum += __shfl_xor(lsum, 32);
        int badi = head_ok ? bad : 0;
        badi |= __shfl_xor(badi, 16);
        badi |= __shfl_xor(badi, 32);

        // publish this wave's partial in LDS (the ring is idle once all waves arrive)
        __syncthreads();
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[wave * kRedStride + (16 * dt + 4 * g4 + r) * 16 + n] = o[dt][r];
        if (g4 == 0) {
            red[wave * kRedStride + 2048 + n] = lsum;
            red[wave * kRedStride + 2064 + n] = ONLINE ? mrun : (float)badi;
        }
        __syncthreads();
    };

    // ---- unified-max pass: plain sums over the waves
    run(std::false_type{});
    for (int idx = threadIdx.x; idx < GB * kHeadDim; idx += NW * 64) {
        const int hh = idx >> 7, d = idx & 127;
        float acc = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < NW; ++w2) acc += red[w2 * kRedStride + d * 16 + hh];
        const size_t slot = ((size_t)b * p.hq + h0 + hh) * p.maxch + c;
        p.o_part[slot * kHeadDim + d] = acc;
    }
    if (wave == 0) {
        int f = 0;
        float l = 0.f;
        if (lane < GB) {
#pragma unroll
            for (int w2 = 0; w2 < NW; ++w2) {
                l += red[w2 * kRedStride + 2048 + lane];
                f |= red[w2 * kRedStride + 2064 + lane] != 0.f;
            }
            const size_t slot = ((size_t)b * p.hq + h0 + lane) * p.maxch + c;
            p.l_part[slot] = l;
            p.m_part[slot] = p.phi;
            p.cflag[slot] = f;
        }
        const uint64_t m = __ballot(f);
        if (lane == 0) flagged_heads = (int)(uint32_t)m;
    }
    __syncthreads();
    const int fmask = flagged_heads;
    if (fmask == 0) return;

    // ---- a score of this chunk left the safe band (FlashDecoding++ theory
    // page, section 3): redo the chunk with online softmax and replace the
    // partials of the flagged heads
    __syncthreads();   // everyone has read red[] before the ring is refilled
    run(std::true_type{});
    for (int idx = threadIdx.x; idx < GB * kHeadDim; idx += NW * 64) {
        const int hh = idx >> 7, d = idx & 127;
        if (!((fmask >> hh) & 1)) continue;
        float M = -INFINITY;
#pragma unroll
        for (int w2 = 0; w2 < NW; ++w2) M = fmaxf(M, red[w2 * kRedStride + 2064 + hh]);
        float acc = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < NW; ++w2) {
            const float mw = red[w2 * kRedStride + 2064 + hh];
            const float f = (mw == M) ? 1.f : exp2_hw((mw - M) * kLog2e);
            acc += red[w2 * kRedStride + d * 16 + hh] * f;
        }
        const size_t slot = ((size_t)b * p.hq + h0 + hh) * p.maxch + c;
        p.o_part[slot * kHeadDim + d] = acc;
    }
    if (threadIdx.x < GB && ((fmask >> threadIdx.x) & 1)) {
        const int hh = threadIdx.x;
        float M = -INFINITY;
#pragma unroll
        for (int w2 = 0; w2 < NW; ++w2) M = fmaxf(M, red[w2 * kRedStride + 2064 + hh]);
        float l = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < NW; ++w2) {
            const float mw = red[w2 * kRedStride + 2064 + hh];
            const float f = (mw == M) ? 1.f : exp2_hw((mw - M) * kLog2e);
            l += red[w2 * kRedStride + 2048 + hh] * f;
        }
        const size_t slot = ((size_t)b * p.hq + h0 + hh) * p.maxch + c;
        p.l_part[slot] = l;
        p.m_part[slot] = M;
    }
}

}  // namespace chunk
}  // namespace fd
