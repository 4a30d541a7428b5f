// Shared device-side definitions of the decode-attention kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fd_attn.h"

#define FD_DEV __device__ __forceinline__
#define FD_HOST_DEV __host__ __device__

namespace fd {

constexpr int kHeadDim = 128;
constexpr float kLog2e = 1.44269504088896340736f;

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;

// Everything a kernel of one call needs, passed by value.
struct Params {
    const void *q, *k, *v;
    const int32_t *seq_lens, *block_table;
    const float *k_scale, *v_scale;
    void *out;
    uint8_t *flags;
    // workspace carve-up
    float *o_part;        // [B][Hq][maxch][128]
    float *l_part;        // [B][Hq][maxch]
    float *m_part;        // [B][Hq][maxch]
    uint8_t *cflag;       // [B][Hq][maxch]
    unsigned long long *count_word;   // {recomputed (row, chunk) pairs, epoch} of the call
    unsigned long long *fused_word;   // fused merge: {epoch | merged row groups}
    unsigned long long *fused_count;  // fused merge: {epoch | recomputed (row, chunk) pairs}
    unsigned long long *claim_word;   // balanced shares: {epoch | pool grains claimed}
    unsigned long long *rg_count;     // [B][Hq] epoch-tagged unit counts per row group (first head)
    uint32_t epoch;                   // this call's epoch (never 0)
    int fused;                        // the last workgroup of a row group merges it (else a merge launch)
    int share_chunks;                 // balanced shares of whole chunks (else pieces cut at share edges)
    int ngroups;                      // row groups of the call (sequences x head blocks)
    int batch, hq, hkv, group;   // group = hq / hkv
    int heads_per_block;         // query heads one chunk workgroup serves (MFMA path)
    int max_seq_len, chunk, maxch;
    int page_shift;              // log2(page_size); unused when contiguous
    int max_blocks;
    float scale;                 // softmax scale (k_scale folded in per head by the kernels)
    float phi, lo, hi;
    int out_bf16;
};

// Read-only tables (lengths, block table, scales) are read through the
// constant address space: a wave-uniform index then becomes a scalar load.
template <typename T>
FD_DEV const __attribute__((address_space(4))) T *as_const(const T *ptr)
{
    return (const __attribute__((address_space(4))) T *)(ptr);
}

// Workspace slot of the partial of (sequence b, query head h, chunk c): the
// partials of one chunk of a sequence are contiguous over the heads.
FD_DEV size_t part_slot(const Params &p, int b, int h, int c)
{
    return ((size_t)b * p.maxch + c) * p.hq + h;
}

FD_DEV int seq_len_of(const Params &p, int b)
{
    int L = as_const(p.seq_lens)[b];
    return L < 0 ? 0 : (L > p.max_seq_len ? p.max_seq_len : L);
}

// Element offset of (sequence b, kv head kvh, token t, component 0).
template <bool PAGED>
FD_DEV size_t kv_offset(const Params &p, int b, int kvh, int t)
{
    if constexpr (PAGED) {
        const int P = 1 << p.page_shift;
        const int page = p.block_table[(size_t)b * p.max_blocks + (t >> p.page_shift)];
        return (((size_t)page * p.hkv + kvh) * P + (t & (P - 1))) * kHeadDim;
    } else {
        return (((size_t)b * p.hkv + kvh) * p.max_seq_len + t) * kHeadDim;
    }
}

template <int DT> struct Elem;
template <> struct Elem<FD_F32> { static constexpr int bytes = 4; };
template <> struct Elem<FD_BF16> { static constexpr int bytes = 2; };
template <> struct Elem<FD_FP8_E4M3FN> { static constexpr int bytes = 1; };

FD_DEV float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
FD_DEV float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two OCP E4M3FN codes (low or high 16-bit half of w) -> two floats, exact.
FD_DEV f32x2 fp8x2_to_f32(uint32_t w, bool high)
{
    return high ? __builtin_amdgcn_cvt_pk_f32_fp8(w, true) : __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
}

// Eight consecutive elements starting at element offset `off` -> float[8].
// STREAM marks the loads non-temporal, for data read once per call (the K/V
// stream) by instructions that cover whole cache lines: the caches then keep
// what is re-read instead of the stream.  (Loads whose lanes cover only half
// of each line, the other half following in the next instruction, lose the
// line between the two when marked so: measured slower.)
template <int DT, bool STREAM = false>
FD_DEV void load8(const void *base, size_t off, float (&x)[8])
{
    auto ld = [](const auto *p) { return STREAM ? __builtin_nontemporal_load(p) : *p; };
    if constexpr (DT == FD_F32) {
        const u32x4 *p = reinterpret_cast<const u32x4 *>(static_cast<const float *>(base) + off);
        u32x4 a = ld(p), b = ld(p + 1);
        x[0] = __uint_as_float(a.x); x[1] = __uint_as_float(a.y);
        x[2] = __uint_as_float(a.z); x[3] = __uint_as_float(a.w);
        x[4] = __uint_as_float(b.x); x[5] = __uint_as_float(b.y);
        x[6] = __uint_as_float(b.z); x[7] = __uint_as_float(b.w);
    } else if constexpr (DT == FD_BF16) {
        u32x4 a = ld(reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(base) + off));
        x[0] = bf16_lo(a.x); x[1] = bf16_hi(a.x); x[2] = bf16_lo(a.y); x[3] = bf16_hi(a.y);
        x[4] = bf16_lo(a.z); x[5] = bf16_hi(a.z); x[6] = bf16_lo(a.w); x[7] = bf16_hi(a.w);
    } else {
        u32x2 a = ld(reinterpret_cast<const u32x2 *>(static_cast<const uint8_t *>(base) + off));
        f32x2 c0 = fp8x2_to_f32(a.x, false), c1 = fp8x2_to_f32(a.x, true);
        f32x2 c2 = fp8x2_to_f32(a.y, false), c3 = fp8x2_to_f32(a.y, true);
        x[0] = c0.x; x[1] = c0.y; x[2] = c1.x; x[3] = c1.y;
        x[4] = c2.x; x[5] = c2.y; x[6] = c3.x; x[7] = c3.y;
    }
}

// Sum over the 16 lanes of a DPP row; every lane of the row gets the same,
// bit-identical result (each step adds a value to its mirror image).
FD_DEV float row16_sum(float x)
{
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));   // quad_perm 1,0,3,2
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));   // quad_perm 2,3,0,1
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, true));  // row_half_mirror
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xF, 0xF, true));  // row_mirror
    return x;
}

FD_DEV float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

FD_DEV bool outside_band(float s, float lo, float hi) { return !(s >= lo && s <= hi); }

}  // namespace fd
