// Causal prefill attention with the unified maximum (gfx950): bf16 queries
// over a bf16 or E4M3FN cache, contiguous or paged.
//
// The prefill form of the method (FlashDecoding++ theory page, section 3: the
// preset maximum serves prefill as it serves decode): a block of q_len query
// tokens per sequence, query j at position kv_len - q_len + j attending keys
// 0 .. position.  Every weight is exp(s - phi) against the caller's constant,
// so the key loop carries no running maximum and never rescales the output
// accumulators.  A score outside [phi - a, phi + b] sets the row's flag; from
// the first key tile in which a wavefront sees one, that wavefront continues
// with the ordinary running-maximum online softmax, starting from its
// unified-max sums (reference phi), so the result stays exact (the fallback
// rule of the same section).
//
// Work decomposition.  A workgroup owns one (sequence b, query head h, tile of
// M = NW * 16 * QB consecutive queries) and walks all the keys its last query
// sees; wavefront w owns queries 16*QB*w .. 16*QB*w + 16*QB - 1 of the tile in
// QB blocks of 16.  Work items are ordered (sequence, kv head) outer, query
// tiles heaviest first, the heads of a KV group innermost, and dealt to the
// eight XCDs in contiguous ranges (a launch places workgroup i on XCD i % 8),
// so the query heads and tiles that read the same K/V share one L2.
//
// Ring.  NST stages of 32 keys (K and V: two 16-row groups of bf16 or one
// 32-row group of E4M3FN, 4 KiB per group) shared by the workgroup and filled
// by 1 KiB DMA instructions, each moving 4 (8) whole cache rows -- buffer->LDS
// over the sequence's contiguous slice, or global->LDS per page through the
// block table; the 16-byte pieces of a row are rotated so the fragment reads
// are free of bank conflicts.  One barrier per stage.  Per stage and wavefront:
//   * K fragments with ds_read_b128, V^T fragments with ds_read_b64_tr_b16
//     (ds_read_b64_tr_b8 for E4M3FN, whose codes are widened to bf16 in
//     registers, exactly; k_scale joins the softmax scale, v_scale the output);
//   * S^T[16 keys x 16 queries] = K . Q^T on v_mfma_f32_16x16x32_bf16 (Q^T
//     fragments stay in registers), scale, causal mask, band test, weights;
//   * weights split into a bf16 high part and a bf16 remainder (together a
//     relative 2^-18); the weight sums add the fp32 weights in registers;
//   * O^T[128 x 16 queries] += V^T . P^T on v_mfma_f32_16x16x32_bf16 over the
//     stage's 32 keys, once per part, taken in the order the two score tiles
//     hand them over.
#pragma once

#include <type_traits>

#include "fd_ring.h"

namespace fd {
namespace prefill {

using namespace ring;

// Everything one prefill call's kernel needs, passed by value.
struct PrefillParams {
    const uint16_t *q;             // bf16 bit patterns
    const void *k, *v;             // bf16 bit patterns or E4M3FN codes
    const int32_t *kv_lens;
    const int32_t *block_table;    // [B][max_blocks] (paged caches)
    const float *k_scale, *v_scale;   // [Hkv] (E4M3FN caches)
    void *out;
    uint8_t *flags;
    int batch, hq, hkv, group;     // group = hq / hkv
    int q_len, max_seq_len;
    int page_shift, max_blocks;    // paged caches: log2(page size), row stride of block_table
    int ntiles;                    // query tiles per (sequence, head)
    int total;                     // work items
    int per_xcd;                   // ceil(total / 8)
    float c1;                      // scale * log2(e): raw score -> exponent units
    float c0;                      // -phi * log2(e)
    float lo_raw, hi_raw, phi_raw; // band edges and phi in raw score units (divided by scale)
    float scale, lo, hi, phi;      // the same in score units (E4M3FN: divided per KV head on the GPU)
};

// Two floats -> packed bf16 pair, round to nearest even.
FD_DEV uint32_t pack_bf16(float a, float b)
{
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

// Stage geometry per cache format: a stage holds 32 keys of K and of V, as
// two 16-row groups of 256-byte bf16 rows or one 32-row group of 128-byte
// E4M3FN rows (4 KiB per group either way, the decode kernels' formats and
// LDS piece rotations).
template <int NW, int QB, int NST, int KV = FD_BF16>
struct Shape {
    static constexpr int waves = NW;
    static constexpr int qblocks = QB;                 // 16-query blocks per wavefront
    static constexpr int nst = NST;
    static constexpr int rows = NW * 16 * QB;          // queries per workgroup
    static constexpr int keys = 32;                    // keys per stage
    static constexpr int groups = KV == FD_FP8_E4M3FN ? 1 : 2;   // compute groups per stage
    static constexpr int tile = groups * kGroupBytes;  // K (or V) part of a stage
    static constexpr int stage = 2 * tile;
    static constexpr int lds = NST * stage;
    static constexpr int dma_per_group = 4 / NW;       // 1 KiB DMA instructions per wave per K (or V) group
    static constexpr int dma_per_wave = 2 * groups * dma_per_group;
    static_assert(NW == 2 || NW == 4, "two or four wavefronts");
    static_assert(NST >= 2, "the ring needs two stages");
    static_assert((NST - 1) * dma_per_wave < 64, "vmcnt cannot count that deep");
    static_assert(lds <= 80 * 1024, "two workgroups per compute unit");
    static_assert(QB >= 1 && QB <= 4, "query blocks per wavefront");
};

template <int NW, int QB, int NST, int KV, bool PAGED, bool OUT_BF16>
__global__ __launch_bounds__(NW * 64, QB > 2 ? 1 : 2) void prefill_kernel(PrefillParams p)
{
    using S = Shape<NW, QB, NST, KV>;
    using F = Fmt<KV>;
    constexpr bool FP8 = KV == FD_FP8_E4M3FN;
    constexpr int ROW = F::row;                    // bytes per cache row
    constexpr int GRP = F::group;                  // rows per compute group
    constexpr int NG = S::groups;                  // compute groups per stage
    constexpr int RPI = 1024 / ROW;                // rows per DMA instruction
    constexpr int LPR = 64 / RPI;                  // lanes per row in a DMA instruction
    constexpr int BLK = S::keys;
    constexpr int IPG = S::dma_per_group;
    constexpr int DPW = S::dma_per_wave;
    constexpr int M = S::rows;
    __shared__ __attribute__((aligned(1024))) uint8_t ring[S::lds];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15;
    const int g4 = lane >> 4;

    // ---- work item: contiguous ranges per XCD
    const int wi = (int)(blockIdx.x & 7) * p.per_xcd + (int)(blockIdx.x >> 3);
    if (wi >= p.total) return;
    const int per_pair = p.ntiles * p.group;
    const int pair = wi / per_pair;
    const int rem = wi - pair * per_pair;
    const int td = rem / p.group;
    const int b = pair / p.hkv;
    const int kvh = pair - b * p.hkv;
    const int h = kvh * p.group + (rem - td * p.group);
    const int j0 = (p.ntiles - 1 - td) * M;        // first query of the tile

    int kv = as_const(p.kv_lens)[b];
    kv = kv < 0 ? 0 : (kv > p.max_seq_len ? p.max_seq_len : kv);

    // raw scores are q . k with K as stored: for E4M3FN the KV head's k_scale
    // joins the softmax scale (both positive), and v_scale the output
    float c1 = p.c1, lo_raw = p.lo_raw, hi_raw = p.hi_raw, phi_raw = p.phi_raw, vsc = 1.f;
    if constexpr (FP8) {
        const float eff = p.scale * as_const(p.k_scale)[kvh];
        c1 = eff * kLog2e;
        lo_raw = p.lo / eff;
        hi_raw = p.hi / eff;
        phi_raw = p.phi / eff;
        vsc = as_const(p.v_scale)[kvh];
    }
    const int off = kv - p.q_len;                  // position of query j is off + j
    const int jw0 = j0 + wave * 16 * QB;           // this wavefront's first query
    const int jw_end = min(jw0 + 16 * QB, p.q_len);
    const int kend_w = jw_end > jw0 ? max(0, min(kv, off + jw_end)) : 0;   // keys the wave sees
    const int j_end = min(j0 + M, p.q_len);
    const int kend = max(0, min(kv, off + j_end));                        // keys the workgroup sees
    const int nblk = (kend + BLK - 1) / BLK;
    // every query of the wave sees keys 0 .. pos_min (stages below need no mask)
    const int pos_min = jw0 + 16 * QB <= p.q_len ? off + jw0 : -1;

    // position of query row n of block qb; -1 (no keys) past the query block
    int pos[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int j = jw0 + 16 * qb + n;
        pos[qb] = j < p.q_len ? off + j : -1;
    }

    // ---- DMA: wavefront w issues instructions IPG*w .. IPG*w + IPG-1 of each
    // group of K and of V; instruction i moves group rows RPI*i .. RPI*i +
    // RPI-1, lane l fetching, of row RPI*i + l/LPR, the piece that belongs in
    // LDS slot l%LPR.
    uint32_t dma_vo[IPG];
#pragma unroll
    for (int qd = 0; qd < IPG; ++qd) {
        const int r = RPI * (IPG * wave + qd) + lane / LPR;
        dma_vo[qd] = (lane / LPR) * ROW + 16 * ((lane % LPR - F::rot(r)) & (F::slots - 1));
    }
    const uint8_t *kpool = static_cast<const uint8_t *>(p.k);
    const uint8_t *vpool = static_cast<const uint8_t *>(p.v);
    __amdgpu_buffer_rsrc_t krs, vrs;
    const __attribute__((address_space(4))) int32_t *btab = as_const(p.block_table);
    if constexpr (!PAGED) {
        const size_t slice = ((size_t)b * p.hkv + kvh) * (size_t)p.max_seq_len * ROW;
        const int nrec = (int)((uint32_t)kv * ROW);    // rows past kv read as zeros
        krs = __builtin_amdgcn_make_buffer_rsrc((void *)(kpool + slice), (short)0, nrec, 0x00020000);
        vrs = __builtin_amdgcn_make_buffer_rsrc((void *)(vpool + slice), (short)0, nrec, 0x00020000);
    } else {
        btab += (size_t)b * p.max_blocks;
    }
    // last page a key of the sequence uses; an instruction whose rows lie
    // past kv reads through that page's table entry with an empty range
    const int last_page = kv > 0 ? (kv - 1) >> p.page_shift : 0;
    const int pmask = (1 << p.page_shift) - 1;

    auto issue = [&](int jb, int stage) {
        uint8_t *kt = ring + stage * S::stage + IPG * wave * 1024;
#pragma unroll
        for (int u = 0; u < NG; ++u) {
#pragma unroll
            for (int qd = 0; qd < IPG; ++qd) {
                const int t0 = BLK * jb + GRP * u + RPI * (IPG * wave + qd);
                lds_void *kd = (lds_void *)(kt + u * kGroupBytes + qd * 1024);
                lds_void *vd = (lds_void *)(kt + S::tile + u * kGroupBytes + qd * 1024);
                const uint32_t vo = dma_vo[qd];
                if constexpr (PAGED) {
                    // A buffer range over the page's rows of this KV head that
                    // hold keys (rows past kv read as zeros, like the
                    // contiguous slice past kv).  The rows of one instruction
                    // never straddle a page (pages hold >= 16 rows).
                    const int idx = t0 >> p.page_shift;
                    const int page = btab[idx < last_page ? idx : last_page];
                    const int valid = min(max(kv - (idx << p.page_shift), 0), pmask + 1);
                    const size_t base = ((size_t)page * p.hkv + kvh) * (size_t)(pmask + 1) * ROW;
                    const __amdgpu_buffer_rsrc_t kp = __builtin_amdgcn_make_buffer_rsrc(
                        (void *)(kpool + base), (short)0, valid * ROW, 0x00020000);
                    const __amdgpu_buffer_rsrc_t vp = __builtin_amdgcn_make_buffer_rsrc(
                        (void *)(vpool + base), (short)0, valid * ROW, 0x00020000);
                    const int so = (t0 & pmask) * ROW;
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(kp, kd, 16, vo, so, 0, 0);
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(vp, vd, 16, vo, so, 0, 0);
                } else {
                    const int so = (int)((uint32_t)t0 * ROW);
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, kd, 16, vo, so, 0, 0);
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, vd, 16, vo, so, 0, 0);
                }
            }
        }
    };

    // ---- fragment read addresses inside a compute group (bytes)
    // K, bf16: step kk -> row n, piece g4 + 4kk.  E4M3FN: for score tile tau
    // and half m, row 16*tau + n, piece g4 + 4m (16 codes = steps 2m, 2m+1).
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
    // V^T, dim tile dt.  bf16: lane i of group g4 addresses row 4g4 + i/4,
    // components 16dt + 4(i%4) .. +3; lane k then holds component 16dt + k of
    // rows 4g4 .. 4g4+3 of the group.  E4M3FN: lane i addresses row T(i/2),
    // components 16dt + 8(i%2) .. +7, with T(j) = 4g4 + j (j < 4) or
    // 16 + 4g4 + j - 4; lane k then holds component 16dt + k of rows T(0..7).
    // Either way the keys come in the order the two score tiles hand over
    // their weights.
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

    f32x4 o[QB][8];      // O^T: lane (n, g4) holds components 16dt + 4g4 + i of query n
    float lacc[QB];      // weight sums: lane (n, g4) holds query n's sum over its keys 4g4 .. 4g4+3
    float mrun[QB];      // online softmax: running maximum (raw score units)
    bool bad[QB];        // some visible score of query n left the band
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) o[qb][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        lacc[qb] = 0.f;
        mrun[qb] = -INFINITY;
        bad[qb] = false;
    }

    // ---- ring prologue
#pragma unroll
    for (int k = 0; k < NST - 1; ++k)
        if (k < nblk) issue(k, k);
    int issued = nblk < NST - 1 ? nblk : NST - 1;

    // Q^T fragments (B operand of the score product): k index of MFMA step kk
    // = component 8*g4 + 32*kk + j (bf16) or 16*(g4 + 4*(kk/2)) + 8*(kk%2) + j
    // (E4M3FN, matching its 16-byte K pieces); the K fragments use the same map.  Rows
    // past the block read the last row and are never stored.  The loads and
    // their wait sit in one assembly statement (early-clobber outputs): the
    // compiler never sees a register that a load still in flight will write.
    // The wait also covers the prologue's DMAs, which overlap the loads.
    u32x4 qf[QB][4];
    {
        const size_t head_row = ((size_t)b * p.hq + h) * p.q_len;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const uint16_t *qrow = p.q + (head_row + min(jw0 + 16 * qb + n, p.q_len - 1)) * kHeadDim +
                                   (FP8 ? 16 : 8) * g4;
            if constexpr (FP8)
                asm volatile("global_load_dwordx4 %0, %4, off\n\t"
                             "global_load_dwordx4 %1, %4, off offset:16\n\t"
                             "global_load_dwordx4 %2, %4, off offset:128\n\t"
                             "global_load_dwordx4 %3, %4, off offset:144\n\t"
                             "s_waitcnt vmcnt(0)"
                             : "=&v"(qf[qb][0]), "=&v"(qf[qb][1]), "=&v"(qf[qb][2]), "=&v"(qf[qb][3])
                             : "v"(qrow)
                             : "memory");
            else
                asm volatile("global_load_dwordx4 %0, %4, off\n\t"
                             "global_load_dwordx4 %1, %4, off offset:64\n\t"
                             "global_load_dwordx4 %2, %4, off offset:128\n\t"
                             "global_load_dwordx4 %3, %4, off offset:192\n\t"
                             "s_waitcnt vmcnt(0)"
                             : "=&v"(qf[qb][0]), "=&v"(qf[qb][1]), "=&v"(qf[qb][2]), "=&v"(qf[qb][3])
                             : "v"(qrow)
                             : "memory");
        }
    }

    // ---- per-stage pieces
    // Wait for stage s (this wavefront's DMAs, then everyone's, through the
    // barrier, after which everyone is also done reading stage s-1) and refill
    // the stage that s-1 used.
    auto sync_stage = [&](int s) {
        wait_ring<DPW, NST - 2>(issued - s - 1);
        __builtin_amdgcn_s_barrier();
        if (s + NST - 1 < nblk) {
            issue(s + NST - 1, (s + NST - 1) % NST);
            ++issued;
        }
    };

    // The stage's operands: K fragments per score tile and MFMA step, V^T
    // fragments per dim tile over the stage's 32 keys (bf16; E4M3FN codes are
    // widened exactly in registers).
    u32x4 kop[2][4];
    u32x2 vraw[2][8];                  // bf16: the two groups' V^T fragments
    u32x4 vop[FP8 ? 8 : 1];            // E4M3FN: the widened V^T fragments
    auto vfrag = [&](int dt) -> u32x4 {
        if constexpr (FP8) return vop[dt];
        else return u32x4{vraw[0][dt].x, vraw[0][dt].y, vraw[1][dt].x, vraw[1][dt].y};
    };
    // Read stage s's fragments (group and V offsets are immediates); the
    // fragments are tied to the wait so that no use moves above it.  Rows
    // past kv hold zeros (buffer ranges end at kv in both layouts), so the
    // zero weights of those masked keys never meet a NaN from an unused slot.
    auto read_stage = [&](int s) {
        const uint32_t kt = (uint32_t)(uintptr_t)(ring + (s % NST) * S::stage);
        if constexpr (FP8) {
            u32x4 kraw[4];
            u32x2 v8[8];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const uint32_t addr = kt + k_rd[q4];
                asm volatile("ds_read_b128 %0, %1" : "=v"(kraw[q4]) : "v"(addr) : "memory");
            }
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                const uint32_t addr = kt + v_rd[dt];
                asm volatile("ds_read_b64_tr_b8 %0, %1 offset:%2" : "=v"(v8[dt]) : "v"(addr), "i"(S::tile) : "memory");
            }
            asm volatile("s_waitcnt lgkmcnt(0)"
                         : "+v"(kraw[0]), "+v"(kraw[1]), "+v"(kraw[2]), "+v"(kraw[3])
                         :
                         : "memory");
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) asm volatile("" : "+v"(v8[dt]) : : "memory");
#pragma unroll
            for (int tau = 0; tau < 2; ++tau)
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const u32x4 r = kraw[2 * tau + (kk >> 1)];
                    kop[tau][kk] = (kk & 1) ? e4m3x8_to_bf16(r.z, r.w) : e4m3x8_to_bf16(r.x, r.y);
                }
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) vop[dt] = e4m3x8_to_bf16(v8[dt].x, v8[dt].y);
        } else {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const uint32_t addr = kt + k_rd[kk];
                asm volatile("ds_read_b128 %0, %1" : "=v"(kop[0][kk]) : "v"(addr) : "memory");
                asm volatile("ds_read_b128 %0, %1 offset:%2"
                             : "=v"(kop[1][kk]) : "v"(addr), "i"(kGroupBytes) : "memory");
            }
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                const uint32_t addr = kt + v_rd[dt];
                asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2"
                             : "=v"(vraw[0][dt]) : "v"(addr), "i"(S::tile) : "memory");
                asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2"
                             : "=v"(vraw[1][dt]) : "v"(addr), "i"(S::tile + kGroupBytes) : "memory");
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                asm volatile("s_waitcnt lgkmcnt(0)"
                             : "+v"(kop[u][0]), "+v"(kop[u][1]), "+v"(kop[u][2]), "+v"(kop[u][3])
                             :
                             : "memory");
#pragma unroll
                for (int dt = 0; dt < 8; ++dt) asm volatile("" : "+v"(vraw[u][dt]) : : "memory");
            }
        }
    };

    // Raw scores q.k of the stage for every query block (S^T tiles: lane
    // (n, g4) holds keys 16u + 4g4 + r for query n) and per block the lane's
    // largest and smallest visible score.  MASK: some key of the stage is
    // invisible to some row -- key 16u + 4g4 + r is visible to row n of block
    // qb iff 16u + r <= pos[qb] - t0 - 4g4 -- and invisible scores become -inf.
    f32x4 sacc[QB][2];
    float smax[QB], smin[QB];
    auto score_stage = [&](int s, auto mask_tag) {
        constexpr bool MASK = decltype(mask_tag)::value;
        const int t0 = BLK * s;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) acc = mfma_bf16(kop[u][kk], qf[qb][kk], acc);
                sacc[qb][u] = acc;
            }
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const int dpos = pos[qb] - t0 - 4 * g4;
            float mx = -INFINITY, mn = INFINITY;
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float x = sacc[qb][u][r];
                    if constexpr (MASK) {
                        const bool valid = 16 * u + r <= dpos;
                        mx = fmaxf(mx, valid ? x : -INFINITY);
                        mn = fminf(mn, valid ? x : INFINITY);
                        sacc[qb][u][r] = valid ? x : -INFINITY;
                    } else {
                        mx = fmaxf(mx, x);
                        mn = fminf(mn, x);
                    }
                }
            smax[qb] = mx;
            smin[qb] = mn;
        }
    };

    // Band test of the stage (closed band, raw score units); true if any row
    // of the wavefront saw a score outside it.
    auto band_stage = [&]() {
        bool any = false;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const bool out = smax[qb] > hi_raw || smin[qb] < lo_raw;
            bad[qb] |= out;
            any |= out;
        }
        return __builtin_amdgcn_ballot_w64(any) != 0;
    };

    // Weights of block qb: the fp32 weights add into the lane's weight sum;
    // P^T goes to the matrix cores as a bf16 high part and a bf16 remainder
    // (k = 8*g4 + j <-> group j/4, key row 4*g4 + j%4), O^T += V^T . P^T over
    // 32 keys for both parts.  The two parts carry every weight to a relative
    // 2^-18; a single bf16 weight (2^-9) misses a 2e-3 * max|out| bar on long
    // rows.  nm is the exponent offset: -phi*log2e (unified) or
    // -m*scale*log2e.
    auto accumulate = [&](int qb, float nm) {
        float w[2][4];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                w[u][r] = exp2_hw(fmaf(sacc[qb][u][r], c1, nm));  // -inf -> 0
                lacc[qb] += w[u][r];
            }
        uint32_t h0, h1, h2, h3, l0, l1, l2, l3;
        split_pair(w[0][0], w[0][1], h0, l0);
        split_pair(w[0][2], w[0][3], h1, l1);
        split_pair(w[1][0], w[1][1], h2, l2);
        split_pair(w[1][2], w[1][3], h3, l3);
        const u32x4 ph = {h0, h1, h2, h3}, pl = {l0, l1, l2, l3};
        // raised issue priority while this wavefront feeds the matrix cores:
        // the other wavefront of the SIMD fills the gaps with its vector work
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            const u32x4 va = vfrag(dt);
            o[qb][dt] = mfma_bf16(va, ph, o[qb][dt]);
            o[qb][dt] = mfma_bf16(va, pl, o[qb][dt]);
        }
        __builtin_amdgcn_s_setprio(0);
    };

    // Stages this wavefront computes: [0, nact); of those, [0, nfull) are
    // visible to every row (no mask).  Stages [nact, nblk) are only synchronised.
    const int nact = min(nblk, (kend_w + BLK - 1) / BLK);
    const int nfull = max(0, min(nact, (pos_min + 1) / BLK));

    // One unified-max stage: weights exp(s - phi), no maximum, no rescaling.
    // Returns true if some row of the wavefront sees a score outside the
    // band; such a stage adds exactly nothing here (exponent offset -inf, so
    // every weight is 0) and the online loop redoes it.  Accumulating
    // unconditionally keeps the loop body free of branches around the
    // products, so the accumulators are updated in place.
    auto unified_stage = [&](int s, auto mask_tag) {
        sync_stage(s);
        read_stage(s);
        score_stage(s, mask_tag);
        const bool leave = band_stage();
        const float nm = leave ? -INFINITY : p.c0;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) accumulate(qb, nm);
        return leave;
    };

    // ---- unified-max loops (each body straight-line but for the exit)
    int s = 0;
    bool switched = false;
#pragma unroll 1
    for (; s < nfull; ++s)
        if (unified_stage(s, std::false_type{})) {
            switched = true;
            break;
        }
    if (!switched) {
#pragma unroll 1
        for (; s < nact; ++s)
            if (unified_stage(s, std::true_type{})) {
                switched = true;
                break;
            }
    }

    // ---- online softmax from the stage that left the band on.  The sums so
    // far are relative to phi and built from in-band scores only: a row that
    // saw a key continues from reference phi, a row that saw none from -inf.
    if (switched) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            float l = lacc[qb];
            l += __shfl_xor(l, 16);
            l += __shfl_xor(l, 32);
            mrun[qb] = l > 0.f ? phi_raw : -INFINITY;
        }
#pragma unroll 1
        for (bool first = true; s < nact; ++s, first = false) {
            if (!first) {
                sync_stage(s);
                read_stage(s);
                if (s < nfull)
                    score_stage(s, std::false_type{});
                else
                    score_stage(s, std::true_type{});
                band_stage();
            }
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                float mx = smax[qb];
                mx = fmaxf(mx, __shfl_xor(mx, 16));
                mx = fmaxf(mx, __shfl_xor(mx, 32));
                const float mnew = fmaxf(mrun[qb], mx);
                const float f = (mrun[qb] == mnew) ? 1.f : exp2_hw((mrun[qb] - mnew) * c1);
#pragma unroll
                for (int dt = 0; dt < 8; ++dt) o[qb][dt] *= f;
                lacc[qb] *= f;
                mrun[qb] = mnew;
                accumulate(qb, mnew == -INFINITY ? 0.f : -mnew * c1);
            }
        }
    }

    // ---- stages only the other wavefronts compute
#pragma unroll 1
    for (; s < nblk; ++s) sync_stage(s);

    // ---- epilogue: flags over the 4 lane groups, normalise, store
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        int f = bad[qb] ? 1 : 0;
        f |= __shfl_xor(f, 16);
        f |= __shfl_xor(f, 32);
        const int j = jw0 + 16 * qb + n;
        if (j >= p.q_len) continue;
        float l = lacc[qb];
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        const float inv = l > 0.f ? vsc / l : 0.f;
        const size_t row = ((size_t)b * p.hq + h) * p.q_len + j;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            const f32x4 x = o[qb][dt] * inv;
            const size_t e = row * kHeadDim + 16 * dt + 4 * g4;
            if constexpr (OUT_BF16) {
                *reinterpret_cast<u32x2 *>(static_cast<uint16_t *>(p.out) + e) =
                    u32x2{pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3])};
            } else {
                *reinterpret_cast<f32x4 *>(static_cast<float *>(p.out) + e) = x;
            }
        }
        if (g4 == 0) p.flags[row] = (uint8_t)f;
    }
}

}  // namespace prefill
}  // namespace fd
