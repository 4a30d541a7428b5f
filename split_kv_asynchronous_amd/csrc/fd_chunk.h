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
// Per wave, per 16-token block (blocks of a unit are dealt round-robin to the
// 4 waves):
//   * 8 DMA instructions (4 for K, 4 for V), each moving 4 whole cache rows
//     (1 KiB, fully coalesced) into a 4 KiB K tile and a 4 KiB V tile;
//   * the 16-byte pieces of each row are rotated by rot(t) inside LDS so that
//     the fragment reads below are free of bank conflicts;
//   * S^T[16 tok x 16 heads] = K . Q^T from 4 ds_read_b128 K fragments and
//     4 v_mfma_f32_16x16x32_bf16;
//   * band test, p = exp(s - phi), weight sums in registers; p split into a
//     bf16 high part and a bf16 remainder;
//   * O^T[128 x 16 heads] += V^T . P^T with 8 x 2 v_mfma_f32_16x16x16_bf16,
//     each V^T fragment one ds_read_b64_tr_b16 (a transposing LDS read).
// The ring has two stages: the DMA for the next block is in flight while the
// current block is computed.
#pragma once

#include "fd_common.h"
#include "fd_mfma.h"

namespace fd {

namespace chunk {

constexpr int kWaves = 4;
constexpr int kBlk = 16;                           // tokens per block
constexpr int kRow = kHeadDim * 2;                 // bytes per bf16 cache row
constexpr int kTile = kBlk * kRow;                 // 4 KiB
constexpr int kStage = 2 * kTile;                  // K tile + V tile
constexpr int kStages = 2;
constexpr int kWaveLds = kStages * kStage;         // 16 KiB
constexpr int kLds = kWaves * kWaveLds;            // 64 KiB
constexpr int kRedStride = 16 * kHeadDim + 32;     // one wave's O^T + l + flags (floats)
static_assert(kWaves * kRedStride * 4 <= kLds, "epilogue reduction must fit in the ring");

typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8])
template <int N>
FD_DEV void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

FD_DEV void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }

// rotation of the 16-byte pieces of block-relative token t (0..15)
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

template <bool PAGED>
__global__ __launch_bounds__(256, 2) void chunk_bf16_kernel(Params p)
{
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kLds];
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
    wait_vmcnt<0>();   // queries resident before the DMA stream starts

    // ---- DMA addressing: instruction i of a tile moves tokens 4i .. 4i+3; lane
    // (n, g4) fetches piece (n - rot) & 15 of token 4i + g4 so that LDS slot n
    // of that row holds it.
    const uint32_t dma_voff_even = g4 * kRow + 16 * ((n - rot_of(g4)) & 15);
    const uint32_t dma_voff_odd = g4 * kRow + 16 * ((n - rot_of(4 + g4)) & 15);
    uint8_t *ring = lds + wave * kWaveLds;

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

    const int nblk = (t_end - t_begin + kBlk - 1) / kBlk;

    auto issue = [&](int j, int stage) {
        const int t0 = t_begin + kBlk * j;
        uint8_t *kt = ring + stage * kStage;
        uint8_t *vt = kt + kTile;
        size_t page_off = 0;
        if constexpr (PAGED) {
            int idx = t0 >> p.page_shift;
            idx = idx < last_page ? idx : last_page;
            page_off = (((size_t)btab[idx] * p.hkv + kvh) * (size_t)(pmask + 1) + (t0 & pmask)) * kRow;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t vo = (i & 1) ? dma_voff_odd : dma_voff_even;
            if constexpr (PAGED) {
                __builtin_amdgcn_global_load_lds(kpool + page_off + i * 4 * kRow + vo,
                                                 (lds_void *)(kt + i * 1024), 16, 0, 0);
                __builtin_amdgcn_global_load_lds(vpool + page_off + i * 4 * kRow + vo,
                                                 (lds_void *)(vt + i * 1024), 16, 0, 0);
            } else {
                const int so = (int)((uint32_t)(t0 + 4 * i) * kRow);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void *)(kt + i * 1024), 16, vo, so, 0, 0);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void *)(vt + i * 1024), 16, vo, so, 0, 0);
            }
        }
    };

    // fragment read addresses inside a tile (bytes)
    // K: lane (n, g4), k-step kk: token n, piece g4 + 4kk
    uint32_t k_rd[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) k_rd[kk] = n * kRow + 16 * ((g4 + 4 * kk + rot_of(n)) & 15);
    // V (transposing read): lane i of group g4 addresses token 4g4 + i/4,
    // components 16dt + 4(i%4) .. +3, i.e. half (i & 1) of piece 2dt + (i%4)/2
    const int vt_tok = 4 * g4 + (n >> 2);
    const uint32_t v_rd_row = vt_tok * kRow + 8 * (n & 1);
    const int v_rd_piece = (n & 3) >> 1;
    const int v_rd_rot = rot_of(vt_tok);

    f32x4 o[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float lsum = 0.f;
    int bad = 0;

    int j = wave;
    if (j < nblk) issue(j, 0);
    if (j + kWaves < nblk) issue(j + kWaves, 1);
    int stage = 0;
#pragma unroll 1
    for (; j < nblk; j += kWaves) {
        // wait for this block's 8 DMAs; the next block's 8 may stay in flight
        if (j + kWaves < nblk) wait_vmcnt<8>();
        else wait_vmcnt<0>();
        const uint8_t *kt = ring + stage * kStage;
        const uint8_t *vt = kt + kTile;

        // S^T: rows = tokens 4*g4 + r of the block, column = head n
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const u32x4 kf = *reinterpret_cast<const u32x4 *>(kt + k_rd[kk]);
            s = mfma_bf16(kf, qf[kk], s);
        }
        const int t0 = t_begin + kBlk * j;
        float w[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const bool valid = t0 + 4 * g4 + r < t_end;
            const float sv = s[r] * sc;
            bad |= (int)valid & (int)outside_band(sv, p.lo, p.hi);
            const float e = exp2_hw(fmaf(sv, kLog2e, nphi));
            w[r] = valid ? e : 0.f;
            lsum += w[r];
        }
        uint32_t h01, h23, l01, l23;
        split_pair(w[0], w[1], h01, l01);
        split_pair(w[2], w[3], h23, l23);
        const u32x2 ph = {h01, h23}, pl = {l01, l23};

        // V^T fragments.  Issued as inline assembly: the compiler does not
        // order its own waits for this read against the DMA ring (it would
        // drain every DMA in flight); the explicit waits above and below do.
        u32x2 va[8];
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            const uint32_t addr = (uint32_t)(uintptr_t)(vt + v_rd_row +
                                                        16 * ((2 * dt + v_rd_piece + v_rd_rot) & 15));
            asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(va[dt]) : "v"(addr) : "memory");
        }
        // the fragments are usable only after this wait; tying them to it keeps
        // the products below it
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(va[0]), "+v"(va[1]), "+v"(va[2]), "+v"(va[3]), "+v"(va[4]),
                       "+v"(va[5]), "+v"(va[6]), "+v"(va[7])
                     :
                     : "memory");
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            o[dt] = mfma16(va[dt], ph, o[dt]);
            o[dt] = mfma16(va[dt], pl, o[dt]);
        }
        // every LDS read of this stage has returned before the stage is refilled
        wait_lgkmcnt0();
        if (j + 2 * kWaves < nblk) issue(j + 2 * kWaves, stage);
        stage ^= 1;
    }

    // per-head weight sums and flags over the 4 lane groups
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    int badi = head_ok ? bad : 0;
    badi |= __shfl_xor(badi, 16);
    badi |= __shfl_xor(badi, 32);

    // combine the 4 waves in LDS (the ring is free now)
    __syncthreads();
    float *red = reinterpret_cast<float *>(lds);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wave * kRedStride + (16 * dt + 4 * g4 + r) * 16 + n] = o[dt][r];
    if (g4 == 0) {
        red[wave * kRedStride + 2048 + n] = lsum;
        red[wave * kRedStride + 2064 + n] = (float)badi;
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < GB * kHeadDim; idx += 256) {
        const int hh = idx >> 7, d = idx & 127;
        float acc = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < kWaves; ++w2) acc += red[w2 * kRedStride + d * 16 + hh];
        const size_t slot = ((size_t)b * p.hq + h0 + hh) * p.maxch + c;
        p.o_part[slot * kHeadDim + d] = acc;
    }
    if (threadIdx.x < GB) {
        const int hh = threadIdx.x;
        float l = 0.f, f = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < kWaves; ++w2) {
            l += red[w2 * kRedStride + 2048 + hh];
            f += red[w2 * kRedStride + 2064 + hh];
        }
        const size_t slot = ((size_t)b * p.hq + h0 + hh) * p.maxch + c;
        p.l_part[slot] = l;
        p.m_part[slot] = p.phi;
        p.cflag[slot] = f != 0.f ? 1 : 0;
    }
}

}  // namespace chunk
}  // namespace fd
