// Grouped-query chunk reduction on the matrix cores (bf16 / E4M3FN caches).
//
// When several query heads share one KV head, scoring a chunk is a small dense
// product: S^T[tokens x heads] = K_chunk[tokens x 128] . Q_g^T[128 x heads],
// and the value reduction is O^T[128 x heads] = V^T[128 x tokens] . P^T.
// Both run on v_mfma_f32_16x16x32_bf16 with the head group padded to 16
// columns.  Everything around them -- the band test, exp(s - phi), the weight
// sums -- stays in registers.
//
// Per wavefront, per 32-token block:
//   * K rows are loaded straight into the A-operand layout (16 tokens x 32
//     components per instruction);
//   * the S^T accumulator of two 16-token tiles already has, in each lane, the
//     8 weights that lane must supply as the B operand of the P.V product, so
//     P never leaves the registers.  The tokens are taken in the order
//     (4g..4g+3, 16+4g..16+4g+3) for lane group g, and V is read in that order;
//   * V rows are loaded coalesced (4 whole tokens per instruction) and staged
//     through a wavefront-private LDS buffer to be read back transposed;
//   * P is split into a bf16 high part and a bf16 remainder, so the product
//     keeps ~16 bits of each weight instead of bf16's 8.
#pragma once

#include "fd_common.h"

namespace fd {

constexpr int kMfmaWaves = 4;
constexpr int kVGroupBytes = 4 * 256 + 32;           // 4 tokens of bf16 + pad (bank spread)
constexpr int kVBufBytes = 8 * kVGroupBytes;         // one 32-token block
constexpr int kMfmaLdsBytes = kMfmaWaves * kVBufBytes;

FD_DEV f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// 8 E4M3FN codes -> 8 bf16 (exact: every finite code is a bf16 value).
FD_DEV u32x4 fp8x8_to_bf16x8(u32x2 w)
{
    f32x2 c0 = fp8x2_to_f32(w.x, false), c1 = fp8x2_to_f32(w.x, true);
    f32x2 c2 = fp8x2_to_f32(w.y, false), c3 = fp8x2_to_f32(w.y, true);
    u32x4 r;
    r.x = __builtin_amdgcn_perm(__float_as_uint(c0.y), __float_as_uint(c0.x), 0x07060302u);
    r.y = __builtin_amdgcn_perm(__float_as_uint(c1.y), __float_as_uint(c1.x), 0x07060302u);
    r.z = __builtin_amdgcn_perm(__float_as_uint(c2.y), __float_as_uint(c2.x), 0x07060302u);
    r.w = __builtin_amdgcn_perm(__float_as_uint(c3.y), __float_as_uint(c3.x), 0x07060302u);
    return r;
}

// Raw storage of 8 consecutive cache elements (converted to bf16 only when used,
// so a prefetched block stays in flight until its compute step).
template <int KV> struct Raw8 { typedef u32x4 type; };
template <> struct Raw8<FD_FP8_E4M3FN> { typedef u32x2 type; };

template <int KV>
FD_DEV typename Raw8<KV>::type load_raw8(const void *base, size_t off)
{
    if constexpr (KV == FD_BF16)
        return *reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(base) + off);
    else
        return *reinterpret_cast<const u32x2 *>(static_cast<const uint8_t *>(base) + off);
}

template <int KV>
FD_DEV u32x4 as_bf16x8(typename Raw8<KV>::type r)
{
    if constexpr (KV == FD_BF16) return r;
    else return fp8x8_to_bf16x8(r);
}

// Two floats -> packed bf16 pair, truncated (high) and the rounded remainder (low).
FD_DEV void split_pair(float a, float b, uint32_t &hi, uint32_t &lo)
{
    const uint32_t ua = __float_as_uint(a) & 0xffff0000u;
    const uint32_t ub = __float_as_uint(b) & 0xffff0000u;
    hi = (ua >> 16) | ub;
    const float ra = a - __uint_as_float(ua);
    const float rb = b - __uint_as_float(ub);
    // round-to-nearest-even of the remainders to bf16
    uint32_t xa = __float_as_uint(ra), xb = __float_as_uint(rb);
    xa = (xa + 0x7fffu + ((xa >> 16) & 1u)) >> 16;
    xb = (xb + 0x7fffu + ((xb >> 16) & 1u)) & 0xffff0000u;
    lo = xa | xb;
}

// Grid (maxch, Hq / heads_per_block, B), 256 threads.
template <int KV, bool PAGED>
__global__ __launch_bounds__(256, 2) void partial_mfma_kernel(Params p)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[kMfmaLdsBytes];
    const int c = blockIdx.x, hb = blockIdx.y, b = blockIdx.z;
    if ((blockIdx.x | blockIdx.y | blockIdx.z | threadIdx.x) == 0) *p.counter = 0;
    const int L = seq_len_of(p, b);
    const int t_begin = c * p.chunk;
    if (t_begin >= L) return;
    const int t_end = min(t_begin + p.chunk, L);

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int n = lane & 15;        // head column (B/C operands), token row (A operand)
    const int g4 = lane >> 4;       // lane group: k-slice 8*g4 .. 8*g4+7
    const int GB = p.heads_per_block;
    const int h0 = hb * GB;
    const int kvh = h0 / p.group;
    const bool head_ok = n < GB;

    // Q^T as B operand: lane (n, g4) holds q[h0+n][8*g4 + 32*kk + 0..7]
    u32x4 qf[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        qf[kk] = u32x4{0u, 0u, 0u, 0u};
        if (head_ok)
            qf[kk] = *reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(p.q) +
                                                      ((size_t)b * p.hq + h0 + n) * kHeadDim +
                                                      8 * g4 + 32 * kk);
    }
    float sc = p.scale;
    if constexpr (KV == FD_FP8_E4M3FN) sc *= as_const(p.k_scale)[kvh];
    const float nphi = -p.phi * kLog2e;

    f32x4 o[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float lsum = 0.f;
    int bad = 0;

    uint8_t *vbuf = lds + wave * kVBufBytes;
    const int nblk = (t_end - t_begin + 31) >> 5;

    // Addressing.  A cache row (one token of one KV head) is ROW bytes; every
    // load below is a wave-uniform base plus a per-lane 32-bit offset that is
    // the same for every block.
    constexpr int ELT = Elem<KV>::bytes;
    constexpr int ROW = kHeadDim * ELT;
    const uint32_t koff = n * ROW + 8 * g4 * ELT;      // K: token row n, k-slice g4
    const uint32_t voff = g4 * ROW + 8 * n * ELT;      // V: token g4 of 4, components 8n..
    // contiguous: raw buffer resources over this (b, kvh) stream, L rows long,
    // so rows past the sequence read as zero and nothing is clamped
    __amdgpu_buffer_rsrc_t krs, vrs;
    const uint8_t *kpool = static_cast<const uint8_t *>(p.k);
    const uint8_t *vpool = static_cast<const uint8_t *>(p.v);
    const __attribute__((address_space(4))) int32_t *btab = as_const(p.block_table);
    if constexpr (!PAGED) {
        const size_t slice = ((size_t)b * p.hkv + kvh) * (size_t)p.max_seq_len * ROW;
        krs = __builtin_amdgcn_make_buffer_rsrc((void *)(kpool + slice), (short)0, (int)((uint32_t)L * ROW), 0x00020000);
        vrs = __builtin_amdgcn_make_buffer_rsrc((void *)(vpool + slice), (short)0, (int)((uint32_t)L * ROW), 0x00020000);
    } else {
        btab += (size_t)b * p.max_blocks;
    }
    const int last_page = (L - 1) >> p.page_shift;
    const int pmask = (1 << p.page_shift) - 1;
    // byte offset of (page holding token t, slot of t) in the paged pool; the
    // page index is clamped to the last valid page, whose every slot is mapped
    auto page_row = [&](int t) -> size_t {
        int idx = t >> p.page_shift;
        idx = idx < last_page ? idx : last_page;
        const size_t page = (size_t)btab[idx];
        return ((page * p.hkv + kvh) * (size_t)(pmask + 1) + (t & pmask)) * ROW;
    };

    // One 32-token block of K (A-operand layout) and V (natural rows).
    struct Block {
        typename Raw8<KV>::type k[2][4];
        typename Raw8<KV>::type v[8];
    };
    auto load_block = [&](Block &blk, int j) {
        const int t0 = t_begin + 32 * j;
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) {
            const int tb = t0 + 16 * tau;
            if constexpr (PAGED) {
                const uint8_t *base = kpool + page_row(tb);
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
                    blk.k[tau][kk] = *reinterpret_cast<const typename Raw8<KV>::type *>(
                        base + koff + 32 * kk * ELT);
            } else {
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    if constexpr (KV == FD_BF16)
                        blk.k[tau][kk] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                            krs, koff + 32 * kk * ELT, (int)((uint32_t)tb * ROW), 0));
                    else
                        blk.k[tau][kk] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                            krs, koff + 32 * kk * ELT, (int)((uint32_t)tb * ROW), 0));
                }
            }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int tb = t0 + 4 * i;
            if constexpr (PAGED) {
                blk.v[i] = *reinterpret_cast<const typename Raw8<KV>::type *>(
                    vpool + page_row(tb) + voff);
            } else {
                if constexpr (KV == FD_BF16)
                    blk.v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                        vrs, voff, (int)((uint32_t)tb * ROW), 0));
                else
                    blk.v[i] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                        vrs, voff, (int)((uint32_t)tb * ROW), 0));
            }
        }
    };
    auto compute_block = [&](const Block &blk, int j) {
        const int t0 = t_begin + 32 * j;
        // S^T tiles: lane (n, g4) gets tokens 16*tau + 4*g4 + r, head n
        f32x4 s[2];
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) {
            s[tau] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                s[tau] = mfma_bf16(as_bf16x8<KV>(blk.k[tau][kk]), qf[kk], s[tau]);
        }
        // band test and unified-max weights
        float w[2][4];
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = t0 + 16 * tau + 4 * g4 + r;
                const bool valid = t < t_end;
                const float sv = s[tau][r] * sc;
                bad |= (int)valid & (int)outside_band(sv, p.lo, p.hi);
                const float e = exp2_hw(fmaf(sv, kLog2e, nphi));
                w[tau][r] = valid ? e : 0.f;
                lsum += w[tau][r];
            }
        }
        uint32_t h0w, h1w, h2w, h3w, l0w, l1w, l2w, l3w;
        split_pair(w[0][0], w[0][1], h0w, l0w);
        split_pair(w[0][2], w[0][3], h1w, l1w);
        split_pair(w[1][0], w[1][1], h2w, l2w);
        split_pair(w[1][2], w[1][3], h3w, l3w);
        const u32x4 ph = {h0w, h1w, h2w, h3w};
        const u32x4 pl = {l0w, l1w, l2w, l3w};

        // stage V in natural layout: token t at (t/4)*kVGroupBytes + (t%4)*256
#pragma unroll
        for (int i = 0; i < 8; ++i)
            *reinterpret_cast<u32x4 *>(vbuf + i * kVGroupBytes + g4 * 256 + 16 * n) =
                as_bf16x8<KV>(blk.v[i]);
        __builtin_amdgcn_wave_barrier();
        // V^T fragments: lane (n, g4), dim 16*dt + n, tokens 4*g4 + r (r<4) and 16 + 4*g4 + r
        const uint16_t *vb16 = reinterpret_cast<const uint16_t *>(vbuf);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            const int col = 16 * dt + n;
            const uint16_t *a0 = vb16 + (g4 * kVGroupBytes) / 2 + col;
            const uint16_t *a1 = vb16 + ((4 + g4) * kVGroupBytes) / 2 + col;
            u32x4 va;
            va.x = (uint32_t)a0[0] | ((uint32_t)a0[128] << 16);
            va.y = (uint32_t)a0[256] | ((uint32_t)a0[384] << 16);
            va.z = (uint32_t)a1[0] | ((uint32_t)a1[128] << 16);
            va.w = (uint32_t)a1[256] | ((uint32_t)a1[384] << 16);
            o[dt] = mfma_bf16(va, ph, o[dt]);
            o[dt] = mfma_bf16(va, pl, o[dt]);
        }
        __builtin_amdgcn_wave_barrier();
    };

    // Software pipeline, two register buffers: the next block's loads are in
    // flight while the current block is computed.  Past the last block the
    // prefetch re-reads the current block (a cache hit) so that every
    // iteration issues the same loads and the wait counts stay static.
    Block A, B;
    int j = wave;
    if (j < nblk) load_block(A, j);
    while (j < nblk) {
        load_block(B, j + kMfmaWaves < nblk ? j + kMfmaWaves : j);
        compute_block(A, j);
        j += kMfmaWaves;
        if (j >= nblk) break;
        load_block(A, j + kMfmaWaves < nblk ? j + kMfmaWaves : j);
        compute_block(B, j);
        j += kMfmaWaves;
    }

    // per-head weight sums and band flags: reduce over the 4 lane groups
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    int badi = head_ok ? bad : 0;
    badi |= __shfl_xor(badi, 16);
    badi |= __shfl_xor(badi, 32);

    // combine the wavefronts: red[w][dim*16 + head], then [2048 + head] = l, [2064 + head] = bad
    __syncthreads();
    float *red = reinterpret_cast<float *>(lds);
    constexpr int RS = 2048 + 32;
    static_assert(kMfmaWaves * RS * 4 <= kMfmaLdsBytes, "reduction does not fit");
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wave * RS + (16 * dt + 4 * g4 + r) * 16 + n] = o[dt][r];
    if (g4 == 0) {
        red[wave * RS + 2048 + n] = lsum;
        red[wave * RS + 2064 + n] = (float)badi;
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < 16 * kHeadDim; idx += 256) {
        const int hh = idx >> 7, d = idx & 127;
        if (hh < GB) {
            float acc = 0.f;
#pragma unroll
            for (int w = 0; w < kMfmaWaves; ++w) acc += red[w * RS + d * 16 + hh];
            const size_t slot = ((size_t)b * p.hq + h0 + hh) * p.maxch + c;
            p.o_part[slot * kHeadDim + d] = acc;
        }
    }
    if (threadIdx.x < GB) {
        const int hh = threadIdx.x;
        float l = 0.f, f = 0.f;
#pragma unroll
        for (int w = 0; w < kMfmaWaves; ++w) {
            l += red[w * RS + 2048 + hh];
            f += red[w * RS + 2064 + hh];
        }
        const size_t slot = ((size_t)b * p.hq + h0 + hh) * p.maxch + c;
        p.l_part[slot] = l;
        p.m_part[slot] = p.phi;
        p.cflag[slot] = f != 0.f ? 1 : 0;
    }
}

}  // namespace fd
