// Cooperative grouped-query chunk kernel (used for E4M3FN caches; it also
// takes bf16): K and V stream through an LDS ring shared by the workgroup,
// filled by coalesced buffer->LDS DMA; both contractions run on the matrix
// cores.  Against the per-wavefront-ring kernel it trades redundant score
// work for a small LDS footprint, so more workgroups share a compute unit --
// the better trade for E4M3FN, whose units carry half the bytes.
//
// Work decomposition.  A unit is (sequence b, head block hb, chunk c): up to
// 16 query heads that share one KV head, over one chunk.  The grid is an upper
// bound on the number of units; workgroup i takes the i-th real unit of the
// list "all full chunks, then all partial last chunks", so workgroups past the
// end exit at once and no launch slot in the middle of the grid is wasted on a
// chunk beyond its sequence.
//
// Inside a workgroup the NW wavefronts split the 128 output components, not
// the tokens: every wavefront scores every token of the unit against all heads
// of the block (S^T = K . Q^T is cheap next to streaming K and V) and reduces
// its own 128 / NW components of O.  So the wavefronts need no reduction with
// each other, they all reach the same weight sums, band flags and running
// maxima, and each writes its share of the partial result straight to the
// workspace.
//
// Ring.  Shape <NW, NSUB, NST>: NST stages, each holding one block of NSUB
// compute groups of K and of V (a group is 16 tokens for bf16, 32 tokens for E4M3FN:
// 4 KiB either way).  Every wavefront issues its share of each block's DMAs --
// 1 KiB instructions moving whole cache rows (4 bf16 rows or 8 E4M3FN rows,
// fully coalesced), the 16-byte pieces of a row rotated by rot(t) so the
// fragment reads below are free of bank conflicts.  One barrier per block: at
// block s every wavefront has its own DMAs of block s done and has finished
// reading block s-1, whose stage then takes block s + NST - 1.  Per block:
//   * K fragments with ds_read_b128, V^T fragments with the transposing reads
//     ds_read_b64_tr_b16 / ds_read_b64_tr_b8; E4M3FN codes are widened to bf16
//     in registers (exact);
//   * S^T[16 tok x 16 heads] = K . Q^T on v_mfma_f32_16x16x32_bf16; band
//     test, p = exp(s - phi) and the weight sums in registers; p split into a
//     bf16 high part and a bf16 remainder; O^T[128/NW x 16 heads] += V^T . P^T
//     on v_mfma_f32_16x16x16_bf16 (bf16: 16-token groups) or
//     v_mfma_f32_16x16x32_bf16 (E4M3FN: 32-token groups).
#pragma once

#include <type_traits>

#include "fd_ring.h"

namespace fd {

namespace coop {

using namespace ring;

template <int NW, int NSUB, int NST>
struct Shape {
    static constexpr int waves = NW;           // each reduces 128 / NW output components
    static constexpr int nsub = NSUB;
    static constexpr int nst = NST;
    static constexpr int tile = NSUB * kGroupBytes;    // K (or V) part of a block
    static constexpr int stage = 2 * tile;
    static constexpr int lds = NST * stage;
    static constexpr int dma_per_group = 4 / NW;       // 1 KiB DMA instructions per wave per K (or V) group
    static constexpr int dma_per_wave = 2 * NSUB * dma_per_group;
    static_assert(NW == 2 || NW == 4, "two or four wavefronts");
    static_assert(NST >= 2, "the ring needs two stages");
    static_assert((NST - 1) * dma_per_wave < 64, "vmcnt cannot count that deep");
    static_assert(lds <= 64 * 1024, "LDS per workgroup");
};

template <int KV, bool PAGED, typename S>
__global__ __launch_bounds__(S::waves * 64) void chunk_kernel(Params p)
{
    using F = Fmt<KV>;
    constexpr bool FP8 = KV == FD_FP8_E4M3FN;
    constexpr int NSUB = S::nsub;
    constexpr int NST = S::nst;
    constexpr int ROW = F::row;
    constexpr int GRP = F::group;                  // tokens per compute group
    constexpr int BLK = NSUB * GRP;                // tokens per ring block
    constexpr int RPI = 1024 / ROW;                // rows per DMA instruction
    constexpr int LPR = 64 / RPI;                  // lanes per row in a DMA instruction
    constexpr int DPW = S::dma_per_wave;
    constexpr int IPG = S::dma_per_group;
    constexpr int DT = 8 / S::waves;               // 16-component tiles of O per wavefront
    constexpr int NT = FP8 ? 2 : 1;                // 16-token score tiles per group
    __shared__ __attribute__((aligned(1024))) uint8_t ring[S::lds];
    __shared__ int last_flag, merged;
    if ((blockIdx.x | blockIdx.y | threadIdx.x) == 0) begin_call(p);

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15;
    const int g4 = lane >> 4;
    const int GB = p.heads_per_block;
    const int nhb = p.hq / GB;

    const Unit U = find_unit(p, blockIdx.y * gridDim.x + blockIdx.x, nhb, lane);
    if (!U.ok) return;
    const int b = __builtin_amdgcn_readfirstlane(U.b);
    const int hb = __builtin_amdgcn_readfirstlane(U.hb);
    const int c = __builtin_amdgcn_readfirstlane(U.c);
    const int L = __builtin_amdgcn_readfirstlane(U.L);
    const int t_begin = c * p.chunk;
    const int t_end = min(t_begin + p.chunk, L);
    const int h0 = hb * GB;
    const int kvh = h0 / p.group;
    const bool head_ok = n < GB;

    // Q^T fragments (B operand of the score product).  The k index of MFMA
    // step kk maps to query components 8*g4 + 32*kk + j (bf16) or
    // 16*(g4 + 4*(kk/2)) + 8*(kk%2) + j (E4M3FN, matching 16-byte K pieces);
    // K uses the same map.  They are loaded after the ring prologue has been
    // issued (see run below); heads past the block read a valid row and are
    // zeroed.
    u32x4 qf[4];
    const uint16_t *qlane = static_cast<const uint16_t *>(p.q) +
                            ((size_t)b * p.hq + h0 + (head_ok ? n : 0)) * kHeadDim + (FP8 ? 16 : 8) * g4;
    float sc = p.scale;
    if constexpr (FP8) sc *= as_const(p.k_scale)[kvh];
    const float nphi = -p.phi * kLog2e;

    // ---- DMA: wavefront w issues instructions i = IPG*w .. IPG*w + IPG-1 of
    // every group of K and of V, instruction i moving group rows RPI*i ..
    // RPI*i + RPI-1; lane l fetches, of group row RPI*i + l/LPR, the piece
    // that belongs in LDS slot l%LPR.
    uint32_t dma_vo[IPG];
#pragma unroll
    for (int q = 0; q < IPG; ++q) {
        const int r = RPI * (IPG * wave + q) + lane / LPR;
        dma_vo[q] = (lane / LPR) * ROW + 16 * ((lane % LPR - F::rot(r)) & (F::slots - 1));
    }

    __amdgpu_buffer_rsrc_t krs, vrs;
    const uint8_t *kpool = static_cast<const uint8_t *>(p.k);
    const uint8_t *vpool = static_cast<const uint8_t *>(p.v);
    const __attribute__((address_space(4))) int32_t *btab = as_const(p.block_table);
    if constexpr (!PAGED) {
        const size_t slice = ((size_t)b * p.hkv + kvh) * (size_t)p.max_seq_len * ROW;
        const int nrec = (int)((uint32_t)L * ROW);
        krs = __builtin_amdgcn_make_buffer_rsrc((void *)(kpool + slice), (short)0, nrec, 0x00020000);
        vrs = __builtin_amdgcn_make_buffer_rsrc((void *)(vpool + slice), (short)0, nrec, 0x00020000);
    } else {
        btab += (size_t)b * p.max_blocks;
    }
    // last page a valid token uses (0 for an empty sequence, whose table row
    // is read but never used: the unit issues no DMA)
    const int last_page = L > 0 ? (L - 1) >> p.page_shift : 0;
    const int pmask = (1 << p.page_shift) - 1;

    const int nblk = (t_end - t_begin + BLK - 1) / BLK;

    // Page-table entries of this wavefront's rows of block jb, one per group.
    // Blocks past the unit read the last valid page's entry.
    constexpr int NPG = PAGED ? NSUB : 1;
    auto load_pages = [&](int jb, int (&pg)[NPG]) {
        if constexpr (PAGED) {
#pragma unroll
            for (int u = 0; u < NSUB; ++u) {
                const int idx = (t_begin + BLK * jb + GRP * u + RPI * IPG * wave) >> p.page_shift;
                pg[u] = btab[idx < last_page ? idx : last_page];
            }
        } else {
            pg[0] = 0;
        }
    };

    auto issue = [&](int jb, int stage, const int (&pg)[NPG]) {
        uint8_t *kt = ring + stage * S::stage + IPG * wave * 1024;
#pragma unroll
        for (int u = 0; u < NSUB; ++u) {
#pragma unroll
            for (int q = 0; q < IPG; ++q) {
                // first row of the instruction
                const int t0 = t_begin + BLK * jb + GRP * u + RPI * (IPG * wave + q);
                lds_void *kd = (lds_void *)(kt + u * kGroupBytes + q * 1024);
                lds_void *vd = (lds_void *)(kt + S::tile + u * kGroupBytes + q * 1024);
                if constexpr (PAGED) {
                    // a wavefront's rows of a group never straddle a page (pages hold >= 16 tokens)
                    const size_t off =
                        (((size_t)pg[u] * p.hkv + kvh) * (size_t)(pmask + 1) + (t0 & pmask)) * ROW + dma_vo[q];
                    __builtin_amdgcn_global_load_lds(kpool + off, kd, 16, 0, kStreamPolicy);
                    __builtin_amdgcn_global_load_lds(vpool + off, vd, 16, 0, kStreamPolicy);
                } else {
                    const int so = (int)((uint32_t)t0 * ROW);
                    const uint32_t vo = dma_vo[q];
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, kd, 16, vo, so, 0, kStreamPolicy);
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, vd, 16, vo, so, 0, kStreamPolicy);
                }
            }
        }
    };

    // ---- fragment read addresses inside a compute group (bytes)
    // K, bf16: step kk -> row n, piece g4 + 4kk.  E4M3FN: for tile tau and
    // half m, row 16*tau + n, piece g4 + 4m (16 codes = steps 2m and 2m+1).
    uint32_t k_rd[4];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
        if constexpr (FP8) {
            const int tau = q4 >> 1, m = q4 & 1, r = 16 * tau + n;
            k_rd[q4] = r * ROW + 16 * ((g4 + 4 * m + F::rot(r)) & (F::slots - 1));
        } else {
            k_rd[q4] = n * ROW + 16 * ((g4 + 4 * q4 + F::rot(n)) & (F::slots - 1));
        }
    }
    // V^T (transposing reads) for this wavefront's dim tiles dt = DT*w + dl.
    // bf16: lane i of group g4 addresses row 4g4 + i/4, components
    //   16dt + 4(i%4) .. +3 (half i&1 of piece 2dt + (i%4)/2); lane k then holds
    //   component 16dt + k of rows 4g4 .. 4g4+3.
    // E4M3FN: lane i of group g4 addresses row T(i/2), components 16dt +
    //   8(i%2) .. +7 (half i&1 of piece dt), with T(j) = 4g4 + j (j < 4) or
    //   16 + 4g4 + j - 4; lane k then holds component 16dt + k of rows T(0..7),
    //   the token order in which the two score tiles hand over their weights.
    uint32_t v_rd[DT];
#pragma unroll
    for (int dl = 0; dl < DT; ++dl) {
        const int dt = DT * wave + dl;
        if constexpr (FP8) {
            const int jj = n >> 1;
            const int r = jj < 4 ? 4 * g4 + jj : 16 + 4 * g4 + jj - 4;
            v_rd[dl] = r * ROW + 8 * (n & 1) + 16 * ((dt + F::rot(r)) & (F::slots - 1));
        } else {
            const int r = 4 * g4 + (n >> 2);
            v_rd[dl] = r * ROW + 8 * (n & 1) + 16 * ((2 * dt + ((n & 3) >> 1) + F::rot(r)) & (F::slots - 1));
        }
    }

    f32x4 o[DT];
    float lsum, mrun;
    int bad;

    // One pass over the unit's blocks.  ONLINE == false: weights exp(s - phi)
    // against the preset constant, band test per head.  ONLINE == true: the
    // ordinary running-maximum softmax, the maximum advanced once per compute
    // group.  Leaves this wavefront's 16*DT components of O^T in o, and the
    // weight sum, band flag and running maximum of head n in lsum, bad, mrun
    // (identical in every wavefront).
    auto run = [&](auto online_tag) {
        constexpr bool ONLINE = decltype(online_tag)::value;
#pragma unroll
        for (int dl = 0; dl < DT; ++dl) o[dl] = f32x4{0.f, 0.f, 0.f, 0.f};
        lsum = 0.f;
        mrun = -INFINITY;
        bad = 0;

        int issued = 0;
        {
            int pg[NST - 1][NPG];
#pragma unroll
            for (int k = 0; k < NST - 1; ++k) load_pages(k, pg[k]);
#pragma unroll
            for (int k = 0; k < NST - 1; ++k)
                if (k < nblk) {
                    issue(k, k, pg[k]);
                    ++issued;
                }
        }
        // page-table entries are fetched one ring refill ahead of their use
        int pg_next[NPG];
        load_pages(NST - 1, pg_next);
        // The query loads and their wait sit in one assembly statement
        // (early-clobber outputs), so the compiler never holds a register that
        // a load still in flight will write; issued after the prologue, they
        // overlap its DMAs, which the same wait also covers.
        if constexpr (!ONLINE) {
            if constexpr (FP8)
                asm volatile("global_load_dwordx4 %0, %4, off\n\t"
                             "global_load_dwordx4 %1, %4, off offset:16\n\t"
                             "global_load_dwordx4 %2, %4, off offset:128\n\t"
                             "global_load_dwordx4 %3, %4, off offset:144\n\t"
                             "s_waitcnt vmcnt(0)"
                             : "=&v"(qf[0]), "=&v"(qf[1]), "=&v"(qf[2]), "=&v"(qf[3])
                             : "v"(qlane)
                             : "memory");
            else
                asm volatile("global_load_dwordx4 %0, %4, off\n\t"
                             "global_load_dwordx4 %1, %4, off offset:64\n\t"
                             "global_load_dwordx4 %2, %4, off offset:128\n\t"
                             "global_load_dwordx4 %3, %4, off offset:192\n\t"
                             "s_waitcnt vmcnt(0)"
                             : "=&v"(qf[0]), "=&v"(qf[1]), "=&v"(qf[2]), "=&v"(qf[3])
                             : "v"(qlane)
                             : "memory");
            if (!head_ok) {
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) qf[kk] = u32x4{0u, 0u, 0u, 0u};
            }
        }

        int stage = 0;
#pragma unroll 1
        for (int s = 0; s < nblk; ++s) {
            // this wavefront's DMAs of block s are done (later blocks may
            // still be in flight) ...
            const int ahead = issued - s - 1;
            wait_ring<DPW, NST - 2>(ahead);
            // ... and so are everyone else's; everyone is done reading block s-1
            __builtin_amdgcn_s_barrier();
            if (s + NST - 1 < nblk) {
                issue(s + NST - 1, stage == 0 ? NST - 1 : stage - 1, pg_next);
                ++issued;
            }
            load_pages(s + NST, pg_next);

            // Read the block's fragments.  The reads are inline assembly: the
            // compiler cannot tell them apart from ring slots still being
            // filled and would drain every DMA in flight before them; the
            // explicit waits here do the ordering instead.
            const uint8_t *kt = ring + stage * S::stage;
            const uint8_t *vt = kt + S::tile;
            u32x4 kraw[NSUB][4];
            u32x2 vraw[NSUB][DT];
#pragma unroll
            for (int u = 0; u < NSUB; ++u) {
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const uint32_t addr = (uint32_t)(uintptr_t)(kt + u * kGroupBytes + k_rd[q4]);
                    asm volatile("ds_read_b128 %0, %1" : "=v"(kraw[u][q4]) : "v"(addr) : "memory");
                }
#pragma unroll
                for (int dl = 0; dl < DT; ++dl) {
                    const uint32_t addr = (uint32_t)(uintptr_t)(vt + u * kGroupBytes + v_rd[dl]);
                    if constexpr (FP8)
                        asm volatile("ds_read_b64_tr_b8 %0, %1" : "=v"(vraw[u][dl]) : "v"(addr) : "memory");
                    else
                        asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(vraw[u][dl]) : "v"(addr) : "memory");
                }
            }
            // the fragments are tied to this wait so that no use moves above it
#pragma unroll
            for (int u = 0; u < NSUB; ++u) {
                asm volatile("s_waitcnt lgkmcnt(0)"
                             : "+v"(kraw[u][0]), "+v"(kraw[u][1]), "+v"(kraw[u][2]), "+v"(kraw[u][3])
                             :
                             : "memory");
#pragma unroll
                for (int dl = 0; dl < DT; ++dl) asm volatile("" : "+v"(vraw[u][dl]) : : "memory");
            }
            stage = stage + 1 == NST ? 0 : stage + 1;

#pragma unroll
            for (int u = 0; u < NSUB; ++u) {
                const int tg = t_begin + BLK * s + GRP * u;      // first token of the group
                if (tg + GRP > t_end) {       // the unit ends inside this group
                    const u32x2 vm = v_tail_mask<FP8>(tg, g4, t_end);
#pragma unroll
                    for (int dl = 0; dl < DT; ++dl) vraw[u][dl] &= vm;
                }
                // S^T tiles: rows = tokens 16*tau + 4*g4 + r of the group, column = head n
                f32x4 sacc[NT];
#pragma unroll
                for (int tau = 0; tau < NT; ++tau) {
                    sacc[tau] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk) {
                        u32x4 kf;
                        if constexpr (FP8) {
                            const u32x4 r = kraw[u][2 * tau + (kk >> 1)];
                            kf = (kk & 1) ? e4m3x8_to_bf16(r.z, r.w) : e4m3x8_to_bf16(r.x, r.y);
                        } else {
                            kf = kraw[u][kk];
                        }
                        sacc[tau] = mfma_bf16(kf, qf[kk], sacc[tau]);
                    }
                }
                float w[NT][4];
                if constexpr (!ONLINE) {
#pragma unroll
                    for (int tau = 0; tau < NT; ++tau)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const bool valid = tg + 16 * tau + 4 * g4 + r < t_end;
                            const float sv = sacc[tau][r] * sc;
                            bad |= (int)valid & (int)outside_band(sv, p.lo, p.hi);
                            const float e = exp2_hw(fmaf(sv, kLog2e, nphi));
                            w[tau][r] = valid ? e : 0.f;
                            lsum += w[tau][r];
                        }
                } else {
                    float sv[NT][4], mx = -INFINITY;
#pragma unroll
                    for (int tau = 0; tau < NT; ++tau)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const bool valid = tg + 16 * tau + 4 * g4 + r < t_end;
                            sv[tau][r] = valid ? sacc[tau][r] * sc : -INFINITY;
                            mx = fmaxf(mx, sv[tau][r]);
                        }
                    mx = fmaxf(mx, __shfl_xor(mx, 16));
                    mx = fmaxf(mx, __shfl_xor(mx, 32));
                    const float mnew = fmaxf(mrun, mx);
                    const float f = (mrun == mnew) ? 1.f : exp2_hw((mrun - mnew) * kLog2e);
#pragma unroll
                    for (int dl = 0; dl < DT; ++dl) o[dl] *= f;
                    lsum *= f;
#pragma unroll
                    for (int tau = 0; tau < NT; ++tau)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            w[tau][r] = (sv[tau][r] == -INFINITY) ? 0.f
                                                                  : exp2_hw((sv[tau][r] - mnew) * kLog2e);
                            lsum += w[tau][r];
                        }
                    mrun = mnew;
                }
                if constexpr (FP8) {
                    // P^T over 32 tokens: k = 8*g4 + j <-> tile j/4, row 4*g4 + j%4
                    uint32_t h0w, h1w, h2w, h3w, l0w, l1w, l2w, l3w;
                    split_pair(w[0][0], w[0][1], h0w, l0w);
                    split_pair(w[0][2], w[0][3], h1w, l1w);
                    split_pair(w[NT - 1][0], w[NT - 1][1], h2w, l2w);
                    split_pair(w[NT - 1][2], w[NT - 1][3], h3w, l3w);
                    const u32x4 ph = {h0w, h1w, h2w, h3w}, pl = {l0w, l1w, l2w, l3w};
#pragma unroll
                    for (int dl = 0; dl < DT; ++dl) {
                        const u32x4 va = e4m3x8_to_bf16(vraw[u][dl].x, vraw[u][dl].y);
                        o[dl] = mfma_bf16(va, ph, o[dl]);
                        o[dl] = mfma_bf16(va, pl, o[dl]);
                    }
                } else {
                    uint32_t h01, h23, l01, l23;
                    split_pair(w[0][0], w[0][1], h01, l01);
                    split_pair(w[0][2], w[0][3], h23, l23);
                    const u32x2 ph = {h01, h23}, pl = {l01, l23};
#pragma unroll
                    for (int dl = 0; dl < DT; ++dl) {
                        o[dl] = mfma16(vraw[u][dl], ph, o[dl]);
                        o[dl] = mfma16(vraw[u][dl], pl, o[dl]);
                    }
                }
            }
        }
        // per-head weight sums and flags over the 4 lane groups
        lsum += __shfl_xor(lsum, 16);
        lsum += __shfl_xor(lsum, 32);
        bad = head_ok ? bad : 0;
        bad |= __shfl_xor(bad, 16);
        bad |= __shfl_xor(bad, 32);
    };

    // lane (g4, n) holds components 16*(DT*w + dl) + 4*g4 .. +3 of head h0 + n
    const size_t slot = part_slot(p, b, h0 + (head_ok ? n : 0), c);
    float *orow = p.o_part + slot * kHeadDim + 16 * DT * wave + 4 * g4;
    // Partials of a fused call are read by another workgroup during the
    // launch: one 16-byte device-coherent store per piece, through a buffer
    // range over the block's heads (the partials of one chunk of a sequence
    // are contiguous over the heads), instead of four 4-byte coherent stores.
    const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
        p.o_part + part_slot(p, b, h0, c) * kHeadDim, (short)0, GB * kHeadDim * 4, 0x00020000);
    const int ooff = 4 * ((head_ok ? n : 0) * kHeadDim + 16 * DT * wave + 4 * g4);
    auto store_o = [&](int dl) {
        if (p.fused) __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o[dl]), prs, ooff + 64 * dl, 0,
                                                            kCoherentPolicy);
        else __builtin_nontemporal_store(o[dl], reinterpret_cast<f32x4 *>(orow + 16 * dl));
    };

    // A row group whose sequence is this one chunk (or empty) needs no merge:
    // in a fused call each wavefront writes its components of the rows'
    // outputs itself, in the merge's arithmetic (the chunk's sum times
    // v_scale over its weight sum; an empty row is zero), and no partial is
    // stored.
    const bool direct = p.fused && L <= p.chunk;
    const float vs = FP8 ? p.v_scale[kvh] : 1.f;
    const size_t row = (size_t)b * p.hq + h0 + (head_ok ? n : 0);
    auto out_o = [&](int dl) {
        store_out4(p, row * kHeadDim + 16 * DT * wave + 4 * g4 + 16 * dl,
                   L > 0 ? o[dl] * (vs / lsum) : f32x4{0.f, 0.f, 0.f, 0.f});
    };

    // ---- unified-max pass
    run(std::false_type{});
    const uint64_t fmask = __ballot(g4 == 0 && bad != 0);   // the same in every wavefront
    if (head_ok) {
        if (direct) {
            if (!((fmask >> n) & 1)) {                         // flagged heads: after the recompute
#pragma unroll
                for (int dl = 0; dl < DT; ++dl) out_o(dl);
            }
        } else {
#pragma unroll
            for (int dl = 0; dl < DT; ++dl) store_o(dl);
            if (wave == 0 && g4 == 0) {
                part_store(p, p.l_part + slot, lsum);
                part_store(p, p.m_part + slot, p.phi);
                part_store(p, p.cflag + slot, (uint8_t)(bad != 0));
            }
        }
    }

    // ---- a score of this chunk left the safe band (FlashDecoding++ theory
    // page, section 3): redo the chunk with online softmax and replace the
    // partials (or outputs) of the flagged heads
    if (fmask != 0) {
        __builtin_amdgcn_s_barrier();   // everyone is done with the ring
        run(std::true_type{});
        if (head_ok && ((fmask >> n) & 1)) {
#pragma unroll
            for (int dl = 0; dl < DT; ++dl) {
                if (direct) out_o(dl);
                else store_o(dl);
            }
            if (!direct && wave == 0 && g4 == 0) {
                part_store(p, p.l_part + slot, lsum);
                part_store(p, p.m_part + slot, mrun);
            }
        }
    }

    // ---- publish the unit; the last unit of the row group merges it
    if (direct) {
        if (head_ok && wave == 0 && g4 == 0) p.flags[row] = (uint8_t)((fmask >> n) & 1);
        if (threadIdx.x == 0) finish_group(p, __popcll(fmask));
    } else if (publish_unit(p, b * p.hq + h0, units_of(p, L), last_flag)) {
        merge_group<S::waves, 1>(p, b, h0, GB, merged, chunk_parts(p, b, h0, L));
    }
}

}  // namespace coop
}  // namespace fd
