// Pieces shared by the grouped-query chunk kernels: cache formats and their
// LDS piece rotation, vector-memory waits for the DMA rings, matrix-core and
// E4M3FN conversion helpers, and the unit list.
#pragma once

#include "fd_common.h"
#include "fd_merge.h"
#include "fd_mfma.h"

namespace fd {

namespace ring {

constexpr int kGroupBytes = 4096;   // one compute group of K (or V): 16 bf16 or 32 E4M3FN tokens

// Cache policy of the K/V stream's DMA loads: non-temporal.  The stream is
// read once and every DMA instruction covers whole cache lines, so the caches
// are better left to the partial sums.  Measured on the 32K GQA decode
// workload: 5.65 -> 6.22 TB/s for the chunk kernel, together with
// non-temporal partial stores.
constexpr int kStreamPolicy = 2;

// Cache policy of a device-coherent (agent-scope) buffer access: sc1, the
// bit an agent-scope atomic load or store carries.
constexpr int kCoherentPolicy = 16;

// Per storage format: row bytes, tokens per compute group, piece rotation.
// A cache row is moved into LDS as 16-byte pieces; piece j of group row t
// lands in slot (j + rot(t)) mod slots, which keeps the K fragment reads
// (ds_read_b128) and the transposing V reads free of bank conflicts.
// bf16: the LDS serves 256 bytes (64 banks) per cycle.  A K fragment read
// takes one piece from each of 16 rows at once, and the rotations of rows
// 0..15 are all distinct; a transposing V read takes two adjacent slots
// from each of 8 rows at once (0..7 or 8..15), which start on distinct even,
// or distinct odd, slots, so their slot pairs are disjoint.
template <int KV> struct Fmt;
template <> struct Fmt<FD_BF16> {
    static constexpr int row = 256, group = 16, slots = 16;
    static FD_DEV int rot(int t) { return 2 * (t & 7) + (t >> 3); }   // t = 0..15
};
template <> struct Fmt<FD_FP8_E4M3FN> {
    static constexpr int row = 128, group = 32, slots = 8;
    static FD_DEV int rot(int t) { return (t + 4 * ((t >> 4) & 1)) & 7; }   // t = 0..31
};

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

// Wait until at most min(k, KMAX) * D vector-memory operations are in flight.
// Loads complete in order, so with k = the ring blocks issued after block X
// (D operations each) this waits exactly for block X and everything older.
template <int D, int KMAX>
FD_DEV void wait_ring(int k)
{
    if constexpr (KMAX <= 0) {
        wait_vmcnt<0>();
    } else {
        if (k >= KMAX) wait_vmcnt<KMAX * D>();
        else wait_ring<D, KMAX - 1>(k);
    }
}

// Eight (or four) LDS fragment reads and their wait in one assembly statement
// (early-clobber outputs): no register a read still in flight will write is
// ever held by the compiler.
FD_DEV void lds_read8(const uint32_t (&a)[8], u32x4 (&o)[8])
{
    asm volatile("ds_read_b128 %0, %8\n\tds_read_b128 %1, %9\n\t"
                 "ds_read_b128 %2, %10\n\tds_read_b128 %3, %11\n\t"
                 "ds_read_b128 %4, %12\n\tds_read_b128 %5, %13\n\t"
                 "ds_read_b128 %6, %14\n\tds_read_b128 %7, %15\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]),
                   "=&v"(o[6]), "=&v"(o[7])
                 : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
                 : "memory");
}

FD_DEV void lds_read4(const uint32_t (&a)[4], u32x4 (&o)[4])
{
    asm volatile("ds_read_b128 %0, %4\n\tds_read_b128 %1, %5\n\t"
                 "ds_read_b128 %2, %6\n\tds_read_b128 %3, %7\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3])
                 : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
                 : "memory");
}

FD_DEV f32x4 mfma16(u32x2 a, u32x2 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                     __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

// 4 E4M3FN codes -> 4 bf16 (exact), packed as two dwords
FD_DEV u32x2 e4m3x4_to_bf16(uint32_t w)
{
    return u32x2{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true))};
}

FD_DEV u32x4 e4m3x8_to_bf16(uint32_t lo, uint32_t hi)
{
    const u32x2 a = e4m3x4_to_bf16(lo), b = e4m3x4_to_bf16(hi);
    return u32x4{a.x, a.y, b.x, b.y};
}

// AND-mask for the V^T fragments of the compute group that starts at token
// tg: the entries of tokens at or past t_end become +0.  Cache slots past the
// sequence (a page's tail, spare capacity) may hold anything, and the zero
// weight such a token gets would still turn a NaN or an infinity there into a
// NaN in the weight-value product.  Lane group g4 holds, per component,
// bf16: rows 4g4 .. 4g4+3 (16-bit halves in order, two per dword);
// E4M3FN: rows 4g4 + j (byte j of .x) and 16 + 4g4 + j (byte j of .y).
template <bool FP8>
FD_DEV u32x2 v_tail_mask(int tg, int g4, int t_end)
{
    const int n = t_end - tg - 4 * g4;     // valid rows from 4g4 on
    if constexpr (FP8) {
        auto bytes = [](int k) -> uint32_t { return k >= 4 ? ~0u : (k <= 0 ? 0u : (1u << (8 * k)) - 1u); };
        return u32x2{bytes(n), bytes(n - 16)};
    } else {
        auto halves = [](int k) -> uint32_t { return k >= 2 ? ~0u : (k == 1 ? 0xffffu : 0u); };
        return u32x2{halves(n), halves(n - 2)};
    }
}

// Wave-wide inclusive prefix sum on DPP lane moves (no LDS round trip):
// Hillis-Steele inside each row of 16 lanes (row_shr 1, 2, 4, 8; lanes
// shifted in from outside the row add 0), then the total of row 0 is added to
// row 1 and that of row 2 to row 3 (row_bcast:15 on rows 1 and 3), then the
// total of rows 0-1 to rows 2 and 3 (row_bcast:31).  Disabled rows add 0.
FD_DEV int wave_scan(int x)
{
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15, rows 1 and 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31, rows 2 and 3
    return x;
}

struct Unit {
    int b, hb, c, L;   // sequence, head block, chunk; L = the sequence's (clamped) length
    bool ok;
};

// floor(L / chunk) for 0 <= L <= 2^23 through a float reciprocal, corrected
// to the exact quotient (cheaper than an integer division per length).
FD_DEV int div_chunk(int L, int chunk, float rcp)
{
    int q = (int)((float)L * rcp);
    q -= q * chunk > L;
    q += (q + 1) * chunk <= L;
    return q;
}

// The u-th unit of "full chunks of every sequence, then the partial last
// chunks", sequence-major inside each part, chunks outer, head blocks inner:
// consecutive workgroups write the partials of one chunk of a sequence, which
// are contiguous over the heads.
// An empty sequence has one empty unit in the second part, so that its rows
// still get merged (to zeros).
// Every workgroup searches before it can issue a load of its own, so the
// search is kept to one memory round trip for up to 64 * kFindBlocks
// sequences: the lengths of that many are loaded at once (coalesced, indices
// clamped into the array so that no load is conditional), kept in registers
// for both parts, and scanned 64 at a time on DPP lane moves.
constexpr int kFindBlocks = 16;

FD_DEV Unit find_unit(const Params &p, int u, int nhb, int lane)
{
    constexpr int KB = kFindBlocks;
    Unit r = {0, 0, 0, 0, false};
    const int last = p.batch - 1;
    const float rcp = 1.0f / (float)p.chunk;
    int raw[KB];
    auto load = [&](int sb) {
#pragma unroll
        for (int k = 0; k < KB; ++k) {
            const int b = sb + 64 * k + lane;
            raw[k] = as_const(p.seq_lens)[b < last ? b : last];
        }
    };
    const bool resident = p.batch <= 64 * KB;     // one load serves both parts
    if (resident) load(0);
    int base = 0;
#pragma unroll 1
    for (int part = 0; part < 2; ++part) {
#pragma unroll 1
        for (int sb = 0; sb < p.batch; sb += 64 * KB) {
            if (!resident) load(sb);
#pragma unroll
            for (int k = 0; k < KB; ++k) {
                const int b0 = sb + 64 * k;
                if (b0 >= p.batch) break;
                const int b = b0 + lane;
                const int L = b < p.batch ? min(max(raw[k], 0), p.max_seq_len) : -1;   // -1: no sequence
                const int q = div_chunk(L < 0 ? 0 : L, p.chunk, rcp);
                const int cnt = L < 0 ? 0 : part == 0 ? q * nhb : ((L != q * p.chunk || L == 0) ? nhb : 0);
                const int incl = wave_scan(cnt);
                const int total = __builtin_amdgcn_readlane(incl, 63);
                if (u < base + total) {
                    const uint64_t m = __ballot(base + incl > u);
                    const int hit = __builtin_ctzll(m);
                    if (hit > 63) return r;                  // not found (never with a valid scan)
                    const int rem = u - base - __builtin_amdgcn_readlane(incl - cnt, hit);
                    r.b = b0 + hit;
                    r.L = __builtin_amdgcn_readlane(L, hit);
                    if (r.b >= p.batch || r.L < 0) return r;
                    if (part == 0) {
                        r.hb = rem % nhb;
                        r.c = rem / nhb;
                    } else {
                        r.hb = rem;
                        r.c = div_chunk(r.L, p.chunk, rcp);
                    }
                    r.ok = true;
                    return r;
                }
                base += total;
            }
        }
    }
    return r;
}

// ---- Balanced shares (share_kernel).  The call's work is counted in quanta
// of kQuantum tokens: a row group (sequence b, head block hb) has
// quanta_of(L_b) of them, row groups in (b, hb) order; N in all.  The axis of
// quanta is cut into segments, in order: W static shares (workgroup w takes
// share w), then pool grains of kGrainQuanta quanta each, which workgroups
// claim in turn from a counter as they run out of work, so that the
// workgroups that stream faster (the chip serves them unevenly) take more.
// The cut depends only on the lengths, never on who computes what, so the
// result is the same bits on every call.  A quantum is a multiple of the 16
// tokens a page-table entry covers, so a piece never starts inside a DMA
// instruction's rows.
constexpr int kQuantum = 64;
constexpr int kPoolNum = 1, kPoolDen = 4;    // pooled fraction of a call's quanta
constexpr int kGrainQuanta = 16;             // quanta of a pool grain (1024 tokens)

// Quanta of a row group of length L (an empty one counts one, so that some
// workgroup writes its rows).
FD_DEV int quanta_of(int L)
{
    return L > 0 ? (L + kQuantum - 1) / kQuantum : 1;
}

// The cut of a call of N quanta over a grid of `grid` workgroups.  Calls of
// at least 4 quanta per workgroup pool kPoolNum / kPoolDen of their quanta,
// in grains of kGrainQuanta, and keep the rest in the static shares; smaller
// ones are all static, in min(grid, N) shares (every share nonempty).  The
// host sizes the workspace for the grains of the largest N its descriptor
// allows (pool_grains() grows with N).
struct Cut {
    uint64_t N, S;       // quanta in all, in the static shares
    int W;               // static shares
    uint32_t ngrains;    // pool grains
    int G;               // quanta per grain
};

FD_HOST_DEV inline uint64_t pooled(uint64_t N, int grid)
{
    return N < 4 * (uint64_t)grid ? 0 : N * kPoolNum / kPoolDen;
}

FD_HOST_DEV inline uint32_t pool_grains(uint64_t N, int grid, int G = kGrainQuanta)
{
    return (uint32_t)((pooled(N, grid) + G - 1) / G);
}

FD_DEV Cut cut_of(uint64_t N, int grid, int G = kGrainQuanta)
{
    Cut c;
    c.N = N;
    c.G = G;
    c.ngrains = pool_grains(N, grid, G);
    if (c.ngrains) {
        c.S = N - pooled(N, grid);
        c.W = grid;
    } else {
        c.S = N;
        c.W = N < (uint64_t)grid ? (int)N : grid;
    }
    return c;
}

// Segment holding quantum x (static share w: floor(w S / W) <= x, the last
// such w; pool grain k: segment W + k).
FD_DEV uint32_t seg_of(const Cut &c, uint64_t x)
{
    if (x < c.S) return (uint32_t)(((x + 1) * (uint64_t)c.W - 1) / c.S);
    return (uint32_t)c.W + (uint32_t)((x - c.S) / (uint64_t)c.G);
}

// Quanta [lo, hi) of segment s.
FD_DEV void seg_range(const Cut &c, uint32_t s, uint64_t &lo, uint64_t &hi)
{
    if (s < (uint32_t)c.W) {
        lo = (uint64_t)s * c.S / (uint64_t)c.W;
        hi = (uint64_t)(s + 1) * c.S / (uint64_t)c.W;
    } else {
        lo = c.S + (uint64_t)(s - c.W) * (uint64_t)c.G;
        hi = lo + (uint64_t)c.G < c.N ? lo + (uint64_t)c.G : c.N;
    }
}

// Lengths and quanta of sequences sb + 64 k + lane, k < kFindBlocks (quanta 0
// past the batch): all loads issued at once (indices clamped into the array,
// so no load is conditional), one memory round trip per 64 kFindBlocks
// sequences.  Callers use every value (no path leaves a load's register to
// be reused while the load is in flight).
FD_DEV void load_quanta(const Params &p, int sb, int lane, int (&L)[kFindBlocks], int (&q)[kFindBlocks])
{
    const int last = p.batch - 1;
#pragma unroll
    for (int k = 0; k < kFindBlocks; ++k) {
        const int b = sb + 64 * k + lane;
        L[k] = seq_len_of(p, b < last ? b : last);
    }
#pragma unroll
    for (int k = 0; k < kFindBlocks; ++k) q[k] = sb + 64 * k + lane < p.batch ? quanta_of(L[k]) : 0;
}

// Quanta of the call (the same in every wavefront).  A lane's quanta over
// kFindBlocks sequences fit 32 bits, and so does their sum over 64 lanes;
// the running total is carried in 64 bits.
FD_DEV uint64_t call_quanta(const Params &p, int nhb, int lane)
{
    uint64_t seqq = 0;
#pragma unroll 1
    for (int sb = 0; sb < p.batch; sb += 64 * kFindBlocks) {
        int L[kFindBlocks], q[kFindBlocks];
        load_quanta(p, sb, lane, L, q);
        int mine = 0;
#pragma unroll
        for (int k = 0; k < kFindBlocks; ++k) mine += q[k];
        seqq += (uint32_t)__builtin_amdgcn_readlane(wave_scan(mine), 63);
    }
    return seqq * (uint64_t)nhb;
}

// The row group holding quantum x (x < N).  Row group (b, hb) starts at
// nhb P_b + hb quanta_of(L_b), with P_b the quanta of the sequences before b,
// so x lies in sequence b iff P_b <= floor(x / nhb) < P_b + quanta_of(L_b).
// The lengths are scanned 64 at a time on DPP prefix sums.
struct RowGroup {
    uint64_t A;          // its first quantum
    int b, hb, L, nq;    // sequence, head block, clamped length, quanta
};

FD_DEV RowGroup seek(const Params &p, int nhb, int lane, uint64_t x)
{
    RowGroup g = {0, 0, 0, 0, 1};
    const uint64_t xq = x / (uint64_t)nhb;
    uint64_t base = 0;
#pragma unroll 1
    for (int sb = 0; sb < p.batch; sb += 64 * kFindBlocks) {
        int L[kFindBlocks], q[kFindBlocks];
        load_quanta(p, sb, lane, L, q);
        // every block of the group is scanned (blocks past the batch add 0),
        // the hit kept, so that each loaded value is used
        bool found = false;
#pragma unroll
        for (int k = 0; k < kFindBlocks; ++k) {
            const int incl = wave_scan(q[k]);
            const uint32_t total = (uint32_t)__builtin_amdgcn_readlane(incl, 63);
            if (!found && xq < base + total) {
                const uint64_t m = __ballot(base + (uint32_t)incl > xq);
                const int hit = __builtin_ctzll(m);      // < 64: the last lane's sum exceeds xq
                const uint64_t P = base + (uint32_t)__builtin_amdgcn_readlane(incl - q[k], hit);
                g.b = sb + 64 * k + hit;
                g.L = __builtin_amdgcn_readlane(L[k], hit);
                g.nq = __builtin_amdgcn_readlane(q[k], hit);
                g.hb = (int)((x - P * (uint64_t)nhb) / (uint64_t)g.nq);
                g.A = P * (uint64_t)nhb + (uint64_t)g.hb * (uint64_t)g.nq;
                found = true;
            }
            base += total;
        }
        if (found) return g;
    }
    return g;
}

}  // namespace ring
}  // namespace fd
