// Grouped-query chunk kernel for bf16 and E4M3FN caches: K and V stream
// through a per-wave LDS ring filled by coalesced buffer->LDS DMA; both
// contractions run on the matrix cores.
//
// Work decomposition (chunk_kernel).  A unit is (sequence b, head block hb,
// chunk c).  The grid is an upper bound on the number of units; workgroup i
// takes the i-th real unit of the list "all full chunks, then all partial
// last chunks", so workgroups past the end exit at once and no launch slot in
// the middle of the grid is wasted on a chunk beyond its sequence.
// share_kernel runs the same unit body over balanced shares of the call
// instead (see there).
//
// Shape <NW, NSUB, NST>: NW wavefronts per workgroup, each owning an
// NST-stage ring; a ring block holds NSUB compute groups of K and of V (a
// group is 16 tokens for bf16, 32 tokens for E4M3FN: 4 KiB either way).  The
// blocks of a unit are dealt round-robin to the wavefronts.  Per block:
//   * 1 KiB DMA instructions, each moving whole cache rows (4 bf16 rows or 8
//     E4M3FN rows, fully coalesced) into LDS; the 16-byte pieces of a row are
//     rotated by rot(t) so that the fragment reads below are free of bank
//     conflicts;
//   * the block's fragments are read out of the stage at once -- K fragments
//     with ds_read_b128, V^T fragments with the transposing reads
//     ds_read_b64_tr_b16 / ds_read_b64_tr_b8 -- and the stage is refilled
//     before any arithmetic; E4M3FN fragments are widened to bf16 in
//     registers (exact);
//   * S^T[16 tok x 16 heads] = K . Q^T on v_mfma_f32_16x16x32_bf16; band
//     test, p = exp(s - phi) and the weight sums in registers; p split into a
//     bf16 high part and a bf16 remainder; O^T[128 x 16 heads] += V^T . P^T
//     on v_mfma_f32_16x16x16_bf16 (bf16: 16-token groups) or
//     v_mfma_f32_16x16x32_bf16 (E4M3FN: 32-token groups).
#pragma once

#include <type_traits>

#include "fd_ring.h"

namespace fd {

namespace chunk {

using namespace ring;

constexpr int kRedStride = 16 * kHeadDim + 32;     // one wave's O^T, then l and flag-or-max per head

template <int NW, int NSUB, int NST>
struct Shape {
    static constexpr int waves = NW;
    static constexpr int nsub = NSUB;
    static constexpr int nst = NST;
    static constexpr int tile = NSUB * kGroupBytes;    // K (or V) part of a ring block
    static constexpr int stage = 2 * tile;
    static constexpr int wave_lds = NST * stage;
    static constexpr int lds = NW * wave_lds;
    static constexpr int dma_per_block = 2 * tile / 1024;  // 1 KiB per DMA instruction
    static_assert(NST * dma_per_block < 64, "vmcnt cannot count that deep");
    static_assert(NW * kRedStride * 4 <= lds, "epilogue reduction must fit in the ring");
    static_assert(lds <= 160 * 1024, "LDS per workgroup");
    static constexpr int per_cu = lds > 80 * 1024 ? 1 : 2;      // workgroups the LDS lets share a compute unit
};

// One unit of work: tokens [t_begin, t_end) of the row group (sequence b,
// head block hb), whose partials are `parts` (this unit's index idx there).
// A direct unit is the whole row group of a call that merges in the launch:
// it writes the rows' outputs and flags and stores no partial.
struct Seg {
    int b, hb, L;          // L = the sequence's clamped length
    int t_begin, t_end;
    int idx;
    bool direct;
    Parts parts;
};

// Reduces one unit with the whole workgroup, stores its partials (or, for a
// direct unit, the outputs), publishes it, and merges the row group if it
// was the row group's last unit.  `lds` is the workgroup's ring (S::lds
// bytes); the three ints are workgroup-shared.  Every thread must call it;
// it leaves the ring and those ints in use until all threads have returned.
// With `claim` set, thread 0 adds 1 to *claim with a fetch-and-add once its
// wave has issued the unit's last ring refill, and leaves the returned word
// in claim_v: issued there, the round trip is older than no DMA that a later
// ring wait waits for (a wave's vector-memory counter counts returns in issue
// order), so it delays none of them.
template <int KV, bool PAGED, typename S>
FD_DEV void run_unit(const Params &p, const Seg &sg, uint8_t *lds, int &flagged_heads, int &last_flag, int &merged,
                     unsigned long long *claim = nullptr, unsigned long long *claim_v = nullptr)
{
    using F = Fmt<KV>;
    constexpr bool FP8 = KV == FD_FP8_E4M3FN;
    constexpr int NW = S::waves;
    constexpr int NSUB = S::nsub;
    constexpr int NST = S::nst;
    constexpr int ROW = F::row;
    constexpr int GRP = F::group;                  // tokens per compute group
    constexpr int BLK = NSUB * GRP;                // tokens per ring block
    constexpr int RPI = 1024 / ROW;                // rows per DMA instruction
    constexpr int LPR = 64 / RPI;                  // lanes per row in a DMA instruction
    constexpr int DMA_TILE = S::tile / 1024;       // DMA instructions per K (or V) tile

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15;
    const int g4 = lane >> 4;
    const int GB = p.heads_per_block;
    const int b = sg.b, hb = sg.hb, L = sg.L;
    const int t_begin = sg.t_begin, t_end = sg.t_end;
    const int h0 = hb * GB;
    // workspace slot of this unit's partial of head h0 + hh
    auto slot_of = [&](int hh) { return sg.parts.base + (size_t)sg.idx * sg.parts.stride + hh; };
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

    // ---- DMA addressing: instruction i of a tile moves rows RPI*i .. +RPI-1;
    // lane l fetches, of row RPI*i + l/LPR, the piece that belongs in LDS slot
    // l%LPR.  The rotation depends on i only through i%4 (period 2 for bf16,
    // 4 for E4M3FN), so four offsets per lane cover every instruction.
    uint32_t dma_voff[4];
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
        const int r = (RPI * i4 + lane / LPR) % GRP;          // group row
        const int slot = lane % LPR;
        dma_voff[i4] = (lane / LPR) * ROW + 16 * ((slot - F::rot(r)) & (F::slots - 1));
    }
    uint8_t *ring = lds + wave * S::wave_lds;

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

    // Page-table entries of ring block jb, one per 16 tokens (a page holds at
    // least 16).  Blocks past the unit read the last valid page's entry.
    constexpr int NPG = PAGED ? BLK / 16 : 1;
    auto load_pages = [&](int jb, int (&pg)[NPG]) {
        if constexpr (PAGED) {
#pragma unroll
            for (int g = 0; g < NPG; ++g) {
                const int idx = (t_begin + BLK * jb + 16 * g) >> p.page_shift;
                pg[g] = btab[idx < last_page ? idx : last_page];
            }
        } else {
            pg[0] = 0;
        }
    };

    auto issue = [&](int j, int stage, const int (&pg)[NPG]) {
        uint8_t *kt = ring + stage * S::stage;
        uint8_t *vt = kt + S::tile;
        const int tb = t_begin + BLK * j;
        size_t page_off = 0;
#pragma unroll
        for (int i = 0; i < DMA_TILE; ++i) {
            const int t0 = tb + RPI * i;                        // first row of this instruction
            if constexpr (PAGED) {
                // the rows of one instruction never straddle a page
                if (i * RPI % 16 == 0)
                    page_off = (((size_t)pg[i * RPI / 16] * p.hkv + kvh) * (size_t)(pmask + 1) + (t0 & pmask)) * ROW;
            }
            const uint32_t vo = dma_voff[i & 3];
            lds_void *kd = (lds_void *)(kt + i * 1024);
            lds_void *vd = (lds_void *)(vt + i * 1024);
            if constexpr (PAGED) {
                const size_t off = page_off + (size_t)((i * RPI) % 16) * ROW + vo;
                __builtin_amdgcn_global_load_lds(kpool + off, kd, 16, 0, kStreamPolicy);
                __builtin_amdgcn_global_load_lds(vpool + off, vd, 16, 0, kStreamPolicy);
            } else {
                const int so = (int)((uint32_t)t0 * ROW);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, kd, 16, vo, so, 0, kStreamPolicy);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, vd, 16, vo, so, 0, kStreamPolicy);
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
    // V^T (transposing reads), dim tile dt.
    // bf16: lane i of group g4 addresses row 4g4 + i/4, components
    //   16dt + 4(i%4) .. +3 (half i&1 of piece 2dt + (i%4)/2); lane k then holds
    //   component 16dt + k of rows 4g4 .. 4g4+3.
    // E4M3FN: lane i of group g4 addresses row T(i/2), components 16dt +
    //   8(i%2) .. +7 (half i&1 of piece dt), with T(j) = 4g4 + j (j < 4) or
    //   16 + 4g4 + j - 4; lane k then holds component 16dt + k of rows T(0..7),
    //   the token order in which the two S tiles hand over their weights.
    uint32_t v_rd[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
        if constexpr (FP8) {
            const int jj = n >> 1;
            const int r = jj < 4 ? 4 * g4 + jj : 16 + 4 * g4 + jj - 4;
            v_rd[dt] = r * ROW + 8 * (n & 1) + 16 * ((dt + F::rot(r)) & (F::slots - 1));
        } else {
            const int r = 4 * g4 + (n >> 2);
            v_rd[dt] = r * ROW + 8 * (n & 1) + 16 * ((2 * dt + ((n & 3) >> 1) + F::rot(r)) & (F::slots - 1));
        }
    }

    float *red = reinterpret_cast<float *>(lds);

    // One pass over the unit's blocks.  ONLINE == false: weights exp(s - phi)
    // against the preset constant, band test per head.  ONLINE == true: the
    // ordinary running-maximum softmax, the maximum advanced once per compute
    // group.  Leaves this wave's O^T, weight sum, and band flag (or running
    // maximum) in red[wave].
    bool claim_sent = false;
    auto run = [&](auto online_tag) {
        constexpr bool ONLINE = decltype(online_tag)::value;
        constexpr int NT = FP8 ? 2 : 1;            // S tiles per compute group
        f32x4 o[8];
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        float lsum = 0.f;
        float mrun = -INFINITY;     // ONLINE: running maximum of head n (same in all 4 lane groups)
        int bad = 0;

        int j = wave;
        {
            int pg[NST][NPG];
#pragma unroll
            for (int k = 0; k < NST; ++k) load_pages(j + k * NW, pg[k]);
#pragma unroll
            for (int k = 0; k < NST; ++k)
                if (j + k * NW < nblk) issue(j + k * NW, k, pg[k]);
        }
        // page-table entries are fetched one ring refill ahead of their use
        int pg_next[NPG];
        load_pages(j + NST * NW, pg_next);
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
            u32x4 kraw[NSUB][4];
            u32x2 vraw[NSUB][8];
#pragma unroll
            for (int u = 0; u < NSUB; ++u) {
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const uint32_t addr = (uint32_t)(uintptr_t)(kt + u * kGroupBytes + k_rd[q4]);
                    asm volatile("ds_read_b128 %0, %1" : "=v"(kraw[u][q4]) : "v"(addr) : "memory");
                }
#pragma unroll
                for (int dt = 0; dt < 8; ++dt) {
                    const uint32_t addr = (uint32_t)(uintptr_t)(vt + u * kGroupBytes + v_rd[dt]);
                    if constexpr (FP8)
                        asm volatile("ds_read_b64_tr_b8 %0, %1" : "=v"(vraw[u][dt]) : "v"(addr) : "memory");
                    else
                        asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(vraw[u][dt]) : "v"(addr) : "memory");
                }
            }
            // all reads of the stage have returned (the fragments are tied to
            // this wait so no use moves above it); refill the stage
#pragma unroll
            for (int u = 0; u < NSUB; ++u)
                asm volatile("s_waitcnt lgkmcnt(0)"
                             : "+v"(vraw[u][0]), "+v"(vraw[u][1]), "+v"(vraw[u][2]), "+v"(vraw[u][3]),
                               "+v"(vraw[u][4]), "+v"(vraw[u][5]), "+v"(vraw[u][6]), "+v"(vraw[u][7]),
                               "+v"(kraw[u][0]), "+v"(kraw[u][1]), "+v"(kraw[u][2]), "+v"(kraw[u][3])
                             :
                             : "memory");
            if (j + NST * NW < nblk) {
                issue(j + NST * NW, stage, pg_next);
            } else if (!ONLINE && claim && !claim_sent) {
                if (threadIdx.x == 0) *claim_v = fetch_add64(claim, 1);
                claim_sent = true;
            }
            load_pages(j + (NST + 1) * NW, pg_next);
            stage = stage + 1 == NST ? 0 : stage + 1;

#pragma unroll
            for (int u = 0; u < NSUB; ++u) {
                const int tg = t_begin + BLK * j + GRP * u;      // first token of the group
                if (tg + GRP > t_end) {       // the unit ends inside this group
                    const u32x2 vm = v_tail_mask<FP8>(tg, g4, t_end);
#pragma unroll
                    for (int dt = 0; dt < 8; ++dt) vraw[u][dt] &= vm;
                }
                // S^T tiles: rows = tokens 16*tau + 4*g4 + r of the group, column = head n
                f32x4 s[NT];
#pragma unroll
                for (int tau = 0; tau < NT; ++tau) {
                    s[tau] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk) {
                        u32x4 kf;
                        if constexpr (FP8) {
                            const u32x4 r = kraw[u][2 * tau + (kk >> 1)];
                            kf = (kk & 1) ? e4m3x8_to_bf16(r.z, r.w) : e4m3x8_to_bf16(r.x, r.y);
                        } else {
                            kf = kraw[u][kk];
                        }
                        s[tau] = mfma_bf16(kf, qf[kk], s[tau]);
                    }
                }
                float w[NT][4];
                if constexpr (!ONLINE) {
#pragma unroll
                    for (int tau = 0; tau < NT; ++tau)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const bool valid = tg + 16 * tau + 4 * g4 + r < t_end;
                            const float sv = s[tau][r] * sc;
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
                            sv[tau][r] = valid ? s[tau][r] * sc : -INFINITY;
                            mx = fmaxf(mx, sv[tau][r]);
                        }
                    mx = fmaxf(mx, __shfl_xor(mx, 16));
                    mx = fmaxf(mx, __shfl_xor(mx, 32));
                    const float mnew = fmaxf(mrun, mx);
                    const float f = (mrun == mnew) ? 1.f : exp2_hw((mrun - mnew) * kLog2e);
#pragma unroll
                    for (int dt = 0; dt < 8; ++dt) o[dt] *= f;
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
                    for (int dt = 0; dt < 8; ++dt) {
                        const u32x4 va = e4m3x8_to_bf16(vraw[u][dt].x, vraw[u][dt].y);
                        o[dt] = mfma_bf16(va, ph, o[dt]);
                        o[dt] = mfma_bf16(va, pl, o[dt]);
                    }
                } else {
                    uint32_t h01, h23, l01, l23;
                    split_pair(w[0][0], w[0][1], h01, l01);
                    split_pair(w[0][2], w[0][3], h23, l23);
                    const u32x2 ph = {h01, h23}, pl = {l01, l23};
#pragma unroll
                    for (int dt = 0; dt < 8; ++dt) {
                        o[dt] = mfma16(vraw[u][dt], ph, o[dt]);
                        o[dt] = mfma16(vraw[u][dt], pl, o[dt]);
                    }
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

    // A row group whose sequence is this one chunk (or empty) needs no merge:
    // in a fused call the unit writes its rows' outputs and flags itself, in
    // the merge's arithmetic (the chunk's sum times v_scale over its weight
    // sum; an empty row is zero), and stores no partial.
    const bool direct = sg.direct;
    const float vs = FP8 ? p.v_scale[kvh] : 1.f;
    const size_t row0 = (size_t)b * p.hq + h0;

    // ---- unified-max pass: plain sums over the waves
    run(std::false_type{});
    if (claim && !claim_sent && threadIdx.x == 0) *claim_v = fetch_add64(claim, 1);   // no loop iteration
    if (wave == 0) {
        int f = 0;
        float l = 0.f;
        if (lane < GB) {
#pragma unroll
            for (int w2 = 0; w2 < NW; ++w2) {
                l += red[w2 * kRedStride + 2048 + lane];
                f |= red[w2 * kRedStride + 2064 + lane] != 0.f;
            }
            if (!direct) {
                const size_t slot = slot_of(lane);
                part_store(p, p.l_part + slot, l);
                part_store(p, p.m_part + slot, p.phi);
                part_store(p, p.cflag + slot, (uint8_t)f);
            }
        }
        const uint64_t m = __ballot(f);
        if (lane == 0) flagged_heads = (int)(uint32_t)m;
    }
    __syncthreads();
    const int fmask = flagged_heads;
    for (int idx = threadIdx.x; idx < GB * kHeadDim; idx += NW * 64) {
        const int hh = idx >> 7, d = idx & 127;
        float acc = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < NW; ++w2) acc += red[w2 * kRedStride + d * 16 + hh];
        if (direct) {
            if ((fmask >> hh) & 1) continue;          // written after the recompute
            float l = 0.f;
#pragma unroll
            for (int w2 = 0; w2 < NW; ++w2) l += red[w2 * kRedStride + 2048 + hh];
            store_out(p, (row0 + hh) * kHeadDim + d, L > 0 ? acc * (vs / l) : 0.f);
        } else {
            const size_t slot = slot_of(hh);
            part_store(p, p.o_part + slot * kHeadDim + d, acc);
        }
    }

    // ---- a score of this chunk left the safe band (FlashDecoding++ theory
    // page, section 3): redo the chunk with online softmax and replace the
    // partials (or outputs) of the flagged heads
    if (fmask != 0) {
        __syncthreads();   // everyone has read red[] before the ring is refilled
        run(std::true_type{});
        for (int idx = threadIdx.x; idx < GB * kHeadDim; idx += NW * 64) {
            const int hh = idx >> 7, d = idx & 127;
            if (!((fmask >> hh) & 1)) continue;
            float M = -INFINITY;
#pragma unroll
            for (int w2 = 0; w2 < NW; ++w2) M = fmaxf(M, red[w2 * kRedStride + 2064 + hh]);
            float acc = 0.f, l = 0.f;
#pragma unroll
            for (int w2 = 0; w2 < NW; ++w2) {
                const float mw = red[w2 * kRedStride + 2064 + hh];
                const float f = (mw == M) ? 1.f : exp2_hw((mw - M) * kLog2e);
                acc += red[w2 * kRedStride + d * 16 + hh] * f;
                l += red[w2 * kRedStride + 2048 + hh] * f;
            }
            if (direct) {
                store_out(p, (row0 + hh) * kHeadDim + d, acc * (vs / l));
            } else {
                const size_t slot = slot_of(hh);
                part_store(p, p.o_part + slot * kHeadDim + d, acc);
            }
        }
        if (!direct && threadIdx.x < GB && ((fmask >> threadIdx.x) & 1)) {
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
            const size_t slot = slot_of(hh);
            part_store(p, p.l_part + slot, l);
            part_store(p, p.m_part + slot, M);
        }
    }

    // ---- publish the unit; the last unit of the row group merges it
    if (direct) {
        if (threadIdx.x < GB) p.flags[row0 + threadIdx.x] = (uint8_t)((fmask >> threadIdx.x) & 1);
        if (threadIdx.x == 0) finish_group(p, __popc(fmask));
    } else if (publish_unit(p, b * p.hq + h0, sg.parts.n, last_flag)) {
        merge_group<NW>(p, b, h0, GB, merged, sg.parts);
    }
}

template <int KV, bool PAGED, typename S>
__global__ __launch_bounds__(S::waves * 64, S::per_cu) void chunk_kernel(Params p)
{
    __shared__ __attribute__((aligned(1024))) uint8_t lds[S::lds];
    __shared__ int flagged_heads, last_flag, merged;
    if ((blockIdx.x | blockIdx.y | threadIdx.x) == 0) begin_call(p);
    const int GB = p.heads_per_block;
    const Unit U = find_unit(p, blockIdx.y * gridDim.x + blockIdx.x, p.hq / GB, threadIdx.x & 63);
    if (!U.ok) return;
    Seg sg;
    sg.b = __builtin_amdgcn_readfirstlane(U.b);
    sg.hb = __builtin_amdgcn_readfirstlane(U.hb);
    sg.L = __builtin_amdgcn_readfirstlane(U.L);
    const int c = __builtin_amdgcn_readfirstlane(U.c);
    sg.t_begin = c * p.chunk;
    sg.t_end = min(sg.t_begin + p.chunk, sg.L);
    sg.idx = c;
    sg.direct = p.fused && sg.L <= p.chunk;
    sg.parts = chunk_parts(p, sg.b, sg.hb * GB, sg.L);
    run_unit<KV, PAGED, S>(p, sg, lds, flagged_heads, last_flag, merged);
}

// Balanced shares (a persistent grid): the call's work -- every row group's
// tokens, row groups in (sequence, head block) order, in quanta of kQuantum
// tokens -- is cut into segments (cut_of: one static share per workgroup,
// then pool grains that workgroups claim as they finish).  A workgroup walks
// the row groups each of its segments touches and reduces its units there,
// each with the whole workgroup as in chunk_kernel.  Two kinds of unit:
//  * pieces (p.share_chunks == 0): a row group's piece in a segment, cut at
//    the segment's edges; the pieces are the row group's chunks, merged in
//    the launch by the one that completes last (a row group inside one
//    segment is written directly).  Piece (segment s, row group r) keeps its
//    partials in slots (s + r) GB ..: along the cut, s + r grows strictly
//    from piece to piece.
//  * whole chunks of p.chunk tokens (p.share_chunks == 1, p.chunk a multiple
//    of kQuantum): chunk c of a row group belongs to the segment holding its
//    first quantum; partials, merge and one-chunk rows as in chunk_kernel.
template <int KV, bool PAGED, typename S>
__global__ __launch_bounds__(S::waves * 64, S::per_cu) void share_kernel(Params p)
{
    __shared__ __attribute__((aligned(1024))) uint8_t lds[S::lds];
    __shared__ int flagged_heads, last_flag, merged;
    __shared__ uint32_t claimed;
    const int GB = p.heads_per_block;
    const int nhb = p.hq / GB;
    const int lane = threadIdx.x & 63;
    if ((blockIdx.x | threadIdx.x) == 0) begin_call(p);
    const int cq = p.share_chunks ? p.chunk / kQuantum : 0;       // quanta per chunk
    const Cut cut = cut_of(call_quanta(p, nhb, lane), gridDim.x, cq > kGrainQuanta ? cq : kGrainQuanta);
    if ((int)blockIdx.x >= cut.W) return;
    // Pool grains are claimed with one fetch-and-add (thread 0) on the call's
    // epoch-tagged claim counter (fd_merge.h), issued in the segment's last
    // unit once its ring is fully issued and settled after the unit, so the
    // round trip overlaps the unit's last blocks and epilogue (a segment with
    // no unit -- whole chunks, none starting in it -- claims at its end).
    // Every workgroup claims until it draws past the pool: the call makes
    // exactly ngrains + W claims, and the last one resets the counter for the
    // next call.
    uint32_t seg = blockIdx.x;
    unsigned long long pending = 0;
    bool first = true;
    for (;;) {
        uint64_t lo, hi;
        seg_range(cut, seg, lo, hi);
        RowGroup g = seek(p, nhb, lane, lo);
        bool sent = false;
        while (g.A < hi) {
            const uint64_t end = hi < g.A + g.nq ? hi : g.A + g.nq;    // this segment's part of the row group
            Seg sg;
            sg.b = g.b;
            sg.hb = g.hb;
            sg.L = g.L;
            if (cq) {
                // chunks of the row group whose first quantum lies in [lo, end)
                const uint64_t from = lo > g.A ? lo - g.A : 0;
                const int nch = units_of(p, g.L);
                for (int c = (int)((from + cq - 1) / cq); c < nch && (uint64_t)c * cq < end - g.A; ++c) {
                    if (!first) __syncthreads();   // the last unit's epilogue is done with the ring
                    first = false;
                    sg.t_begin = c * p.chunk;
                    sg.t_end = min(sg.t_begin + p.chunk, g.L);
                    sg.idx = c;
                    sg.direct = p.fused && g.L <= p.chunk;
                    sg.parts = chunk_parts(p, g.b, g.hb * GB, g.L);
                    const bool last_unit = (uint64_t)(c + 1) * cq >= end - g.A && g.A + g.nq >= hi;
                    run_unit<KV, PAGED, S>(p, sg, lds, flagged_heads, last_flag, merged,
                                           cut.ngrains && last_unit ? p.claim_word : nullptr, &pending);
                    sent |= last_unit;
                }
            } else {
                if (!first) __syncthreads();
                first = false;
                const uint64_t plo = lo > g.A ? lo : g.A;
                const uint32_t sf = seg_of(cut, g.A), sl = seg_of(cut, g.A + g.nq - 1);
                sg.t_begin = (int)(plo - g.A) * kQuantum;
                sg.t_end = min((int)(end - g.A) * kQuantum, g.L);
                sg.idx = (int)(seg - sf);
                sg.direct = sf == sl;
                sg.parts = Parts{((size_t)sf + (size_t)g.b * nhb + g.hb) * GB, GB, (int)(sl - sf + 1)};
                const bool last_unit = hi <= g.A + g.nq;
                run_unit<KV, PAGED, S>(p, sg, lds, flagged_heads, last_flag, merged,
                                       cut.ngrains && last_unit ? p.claim_word : nullptr, &pending);
                sent |= last_unit;
            }
            // next row group
            g.A += g.nq;
            if (++g.hb == nhb) {
                g.hb = 0;
                if (++g.b == p.batch) break;
                g.L = __builtin_amdgcn_readfirstlane(seq_len_of(p, g.b));
                g.nq = quanta_of(g.L);
            }
        }
        if (!cut.ngrains) break;
        __syncthreads();   // every wave is past the last unit's use of the shared ints
        if (threadIdx.x == 0) {
            if (!sent) pending = fetch_add64(p.claim_word, 1);
            const uint32_t k = epoch_settle(p.claim_word, p.epoch, 1, pending) - 1;
            if (k == cut.ngrains + (uint32_t)cut.W - 1) put(p.claim_word, next_tag(p.epoch));
            claimed = k;
        }
        __syncthreads();
        const uint32_t k = claimed;
        if (k >= cut.ngrains) break;
        seg = (uint32_t)cut.W + k;
    }
}

}  // namespace chunk
}  // namespace fd
