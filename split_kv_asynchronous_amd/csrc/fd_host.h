// Host-side checks shared by the C-ABI entry points.
#pragma once

#include <hip/hip_ext.h>
#include <stdint.h>

#include <tuple>
#include <utility>

#include "fd_attn.h"
#include "fd_common.h"

namespace fd {
namespace host {

inline bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Launches k(args...) on stream s (optionally stamping events e0/e1 from the
// dispatch itself) and returns FD_OK or FD_ERR_LAUNCH from this launch's own
// status.  The thread's last-error state is neither read nor cleared, so an
// error that the caller's own earlier work left there stays for the caller.
template <typename... KArgs, typename... Args>
inline int launch(void (*k)(KArgs...), dim3 grid, dim3 block, size_t lds, hipStream_t s, hipEvent_t e0,
                  hipEvent_t e1, Args &&...args)
{
    static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
    std::tuple<KArgs...> held(std::forward<Args>(args)...);
    const hipError_t e = std::apply(
        [&](auto &...x) {
            void *argv[] = {static_cast<void *>(&x)...};
            return hipExtLaunchKernel(reinterpret_cast<const void *>(k), grid, block, argv, lds, s, e0, e1, 0);
        },
        held);
    return e == hipSuccess ? FD_OK : FD_ERR_LAUNCH;
}

// ---- The plan of a decode call: kernel family, chunk size, kernel shape
// and merge placement.  The table below was measured on MI355X (whole-call
// time, calls replayed back to back; see kTable); a descriptor can force a
// shape and a placement (desc->plan) for tuning and tests.

enum { kFamGroupedBf16 = 0, kFamGroupedFp8 = 1, kFamVector = 2 };

// Kernel family: grouped bf16 queries over a bf16 cache run the per-wavefront
// ring kernel (fd_chunk.h), over an E4M3FN cache the cooperative kernel
// (fd_coop.h); single queries per KV head and fp32 operands the vector kernel
// (fd_valu.h).
inline int family_of(const fd_attn_desc_t *d)
{
    const int group = d->num_q_heads / d->num_kv_heads;
    if (group > 1 && d->q_dtype == FD_BF16 && d->kv_dtype != FD_F32)
        return d->kv_dtype == FD_BF16 ? kFamGroupedBf16 : kFamGroupedFp8;
    return kFamVector;
}

// Largest divisor of g that is <= 16: the query heads one MFMA workgroup serves.
inline int heads_per_block(int g)
{
    for (int k = g < 16 ? g : 16; k > 1; --k)
        if (g % k == 0) return k;
    return 1;
}

// Kernel shapes per family (the shape index of a plan):
//   grouped bf16: 0 = 4 wavefronts x 2 ring stages, 1 = 4 x 3, 2 = 2 x 3
//   grouped E4M3FN: 0 = 2 wavefronts x 3 shared stages, 1 = 4 x 3, 2 = 2 x 4
//   vector: 0 = 4 wavefronts
constexpr int kShapes[3] = {3, 3, 1};

// One row of the plan table: for calls of `family`, paged or not, whose
// max_seq_len is at most max_len (rows in ascending max_len; the last row of
// a family takes every longer call): the chunk size for chunk_size == 0, the
// kernel shape at that chunk size (other chunk sizes run shape 0), and the
// largest chunk size whose calls merge inside the chunk launch (0: none).
// Whatever the row says, a call merges inside the launch if its grid has at
// most kSmallGrid units (sequence x head block x chunk), one round of
// workgroups, or if its chunk covers max_seq_len: then every row is one
// chunk, which the chunk kernel writes out itself, with no partials and no
// merge.
struct TableRow {
    int family, paged, max_len, chunk, shape, fused_chunk;
    int shares;   // chunk_size == 0: 0 = fixed chunks, k + 1 = balanced shares in shape k
};

constexpr int64_t kSmallGrid = 512;

// Calls of at least this many row groups (sequences x query-head blocks) run
// balanced shares in shape 2 unless a plan is forced: pieces for chunk_size
// 0, whole chunks of the given size otherwise (merged in a second launch
// unless a chunk covers max_seq_len).  The fixed-chunk kernels locate every
// unit by scanning all the lengths, and at serving batches that scan
// dominates.  Measured on MI355X, lengths U[128, 2048], paged, whole call,
// shares against fixed chunks: grouped bf16, 64/8 heads, chunk_size 0 (the
// table's plan), batch 512 / 1024 / 2048 / 4096: 0.98-1.02 / 0.91-0.94 /
// 0.80-0.82 / 0.68; chunk 512 at batch 1024 / 4096: 0.87 / 0.53, chunk 2048:
// 0.90 / 0.64; grouped E4M3FN, 32/8 heads, chunk_size 0: 1.03 / 1.01 / 0.94
// / 0.84, chunk 512 at batch 1024 / 4096: 0.97 / 0.67.
constexpr int64_t kServeGroups[2] = {8192, 16384};
// The same threshold for pieces under chunk_size 0.  For bf16 it is higher:
// against the best fixed plan (shape 0, below) rather than the table's first
// one, pieces at 1024 sequences of up to 1K / 2K tokens lost 9% / 5% (465.6
// against 424.2 µs, 845.9 against 804.7).
constexpr int64_t kServeGroupsAuto[2] = {16384, 16384};
// At those batches rows of up to kServeWholeMax tokens run whole-chunk
// shares with one chunk covering every row rather than pieces: µs, pieces
// against one-chunk rows, bf16 paged 2048 / 4096 x U[128, 1K] 920 / 1805
// against 899 / 1745; E4M3FN paged 2048 / 4096 x U[256, 2K] 892 / 1795
// against 855 / 1678; bf16 contiguous 2048 x U[256, 2K] 1660 against 1631.
constexpr int kServeWholeMax = 2048;

// Measured on MI355X: calls replayed back to back (best of 3 x 10), every
// chunk size 256 .. 4096 x every shape x both merge placements, on ragged
// synthetic batches of each family, paging and length range (whole-call
// TB/s of K/V; best against the runner-up):
//   grouped bf16, 64/8 heads: 256 x U[256,2K] 5.83 (chunk 2048, 4 waves x 3
//     stages, rows written by the chunk kernel; with a merge launch 5.72) ; 64 x
//     U[1K,8K] 6.12 (4096, 4 waves x 3 stages; 1024: 6.04) ; 32 x U[1K,32K]
//     6.32 (2048; 1024: 6.17, merged in the launch 6.22) ; 4 x U[32K,128K]
//     6.09 (1024; 2048: 5.91) ; paged: 5.69 (as contiguous), 5.98, 6.28 (in
//     the launch), 5.92
//   grouped E4M3FN, 32/8 heads: 512 x U[256,2K] 5.30 (1024, either way) ; 64 x
//     U[512,16K] 5.75 (1024, in the launch; 512 in the launch 5.64) ;
//     16 x U[16K,64K] 5.75 (2048) ; paged: 5.16, 5.59 (in the launch), 5.69
//   one query per KV head, 32 heads: 64 x 2K 6.77 (2048) ; 8 x 8K 6.66
//     (2048; 1024: 6.37) ; 1 x 128K 6.66 (4096; 1024: 6.60) ; paged: 6.49,
//     6.35, 6.50
// Merging inside the chunk launch against a second launch, by chunk size:
// ahead by 1-9% at chunks of 256-512 (up to 1024 for E4M3FN up to 16K and
// bf16 up to 32K, 2048 paged), level at 2048, behind by 2-6% at 4096, on
// the longest rows (64K-128K: more chunks per row to merge at the end of
// the launch) and on short E4M3FN rows at chunks of 1024 and more; the
// one-query-per-KV-head kernel was 3-60% behind at every chunk size.
// Balanced shares against the plan above (whole call, shares in shape 0,
// best of 3 x 10): grouped E4M3FN 64 x U[512,16K] 0.96 (paged 0.96), 16 x
// U[16K,64K] 0.98 (0.97); grouped bf16 32 x U[1K,32K] 0.98-0.99 (paged
// 1.00); shorter and longer bf16 rows and 2K E4M3FN rows 1.04-1.10.
// Rows of one query per KV head longer than 8K take chunks of 1024 too: a
// flagged chunk is recomputed in place at the end of the launch, so the
// chunk size sets the fallback's tail (1 x 32 heads x 128K with 1% of its
// chunks flagged: 343 µs at 1024, 369 at 2048, 422 at 4096); without
// fallback 1024 was within 1% of 4096 on that workload.
// Rows of one query per KV head up to 2K tokens take chunks of 1024 (32
// heads, µs, 1024 against 2048): ragged U[256, 2K] at 64 / 256 sequences
// 185.6 / 737.7 against 215.6 / 835.6 (paged 200.4 / 779.6 against 218.8 /
// 814.7); all rows of 2K 322.9 / 1261.5 against 314.7 / 1315.3.
// Rows of grouped bf16 up to 2K tokens run shape 0 (4 waves x 2 stages):
// measured later over batch sizes, 64 / 256 / 1024 sequences of up to 1K
// tokens 32.1 / 107.8 / 424.2 µs against 35.2 / 132.0 / 576.1 with 4 x 3,
// and of 256-2K tokens 57.6 / 225.2 / 804.7 against 57.9 / 219.2 / 887.0.
inline constexpr TableRow kTable[] = {
    {kFamGroupedBf16, 0, 2048, 2048, 0, 0, 0},
    {kFamGroupedBf16, 0, 8192, 4096, 1, 512, 0},
    {kFamGroupedBf16, 0, 32768, 2048, 0, 1024, 1},
    {kFamGroupedBf16, 0, 1 << 23, 1024, 0, 0, 0},
    {kFamGroupedBf16, 1, 2048, 2048, 0, 0, 0},
    {kFamGroupedBf16, 1, 8192, 4096, 1, 1024, 0},
    {kFamGroupedBf16, 1, 32768, 2048, 0, 2048, 0},
    {kFamGroupedBf16, 1, 1 << 23, 2048, 0, 0, 0},
    {kFamGroupedFp8, 0, 2048, 1024, 0, 1024, 0},
    {kFamGroupedFp8, 0, 16384, 1024, 0, 1024, 1},
    {kFamGroupedFp8, 0, 1 << 23, 2048, 0, 0, 1},
    {kFamGroupedFp8, 1, 2048, 1024, 0, 1024, 0},
    {kFamGroupedFp8, 1, 16384, 1024, 0, 1024, 1},
    {kFamGroupedFp8, 1, 1 << 23, 2048, 0, 0, 1},
    {kFamVector, 0, 2048, 1024, 0, 0, 0},
    {kFamVector, 0, 8192, 2048, 0, 0, 0},
    {kFamVector, 0, 1 << 23, 1024, 0, 0, 0},
    {kFamVector, 1, 2048, 1024, 0, 0, 0},
    {kFamVector, 1, 8192, 2048, 0, 0, 0},
    {kFamVector, 1, 1 << 23, 1024, 0, 0, 0},
};

inline const TableRow &table_row(const fd_attn_desc_t *d)
{
    const int fam = family_of(d), paged = d->page_size != 0;
    const TableRow *last = nullptr;
    for (const TableRow &r : kTable) {
        if (r.family != fam || r.paged != paged) continue;
        last = &r;
        if (d->max_seq_len <= r.max_len) return r;
    }
    return *last;
}

// The chunk size of a call: the descriptor's, or for 0 the table's (at least
// a page).
// Units of a call at chunk size c, counted as if every sequence were
// max_seq_len long (the host does not see the lengths).
inline int64_t units_at(const fd_attn_desc_t *d, int c)
{
    const int g = d->num_q_heads / d->num_kv_heads;
    const int blocks = family_of(d) == kFamVector ? d->num_q_heads : d->num_q_heads / heads_per_block(g);
    return ((int64_t)d->max_seq_len + c - 1) / c * blocks * d->batch;
}

// The table's chunk sizes were measured on full batches.  A call with few
// rows gets the table's chunk halved, down to kMinAutoChunk tokens, until it
// has kMinAutoUnits units of its family, so that it still spreads over the
// chip: 256 for the grouped bf16 kernel (per-wavefront rings), 2048 for the
// E4M3FN kernel (six workgroups per compute unit), 1024 for one query per KV
// head (below).
// Measured on MI355X, µs per call, table's chunk -> halved: 1 row x 4K fp32
// 20.9 -> 8.4 (chunk 256); 1 row x 128K bf16 137 -> 44 (512); 1 x 32/8
// heads x 8K bf16 41.8 -> 14.6 (256); 8 rows x 4K bf16 26.9 -> 11.0 (256);
// E4M3FN 32/8 heads, 16 / 64 sequences of 256-2K tokens 32.0 / 44.1 -> 19.2
// / 37.9 (256 / 512), 64 of 128-1K 36.6 -> 24.7 (256), 2 x 16K 31.8 -> 28.8
// (256).
// The one-query-per-KV-head kernel aims at 1024 units (32 heads: 8 x
// U[256, 2K] 68.3 -> 33.4 µs at chunk 512, 1 x U[4K, 32K] 97.7 -> 79.2 at
// 1024; its table rows were measured on rows of one length, 8 x 8K stays at
// 2048), and no family runs more than kMaxAutoChunksPerRow chunks per row
// (the table's chunk is doubled for rows that long, and halving stops
// there): one 128K row merges its chunks at the end of the launch, 61.2 µs
// at chunk 256 against 43.9 at 512.
// The grouped families also stop halving at 32 chunks per row: their merge
// of a row's chunks runs in the launch, and past 32 it costs more than the
// extra units give (E4M3FN, 8 x U[512, 16K] / U[4K, 16K]: 46.4 / 50.6 µs at
// chunk 256 against 41.9 / 44.1 at 512; bf16, 1 x 64/8 heads x 32K: 36.7 at
// 512 against 31.1 at 1024).
constexpr int kMinAutoUnits[3] = {256, 2048, 1024};
constexpr int kMinAutoChunk = 256;
constexpr int kMaxAutoChunksPerRow = 256;
constexpr int kMaxHalvedChunksPerRow[3] = {32, 32, 256};

inline int chunk_of(const fd_attn_desc_t *d)
{
    if (d->chunk_size != 0) return d->chunk_size;
    const int fam = family_of(d);
    int c = table_row(d).chunk;
    while ((int64_t)c * kMaxAutoChunksPerRow < d->max_seq_len) c *= 2;
    while (c > kMinAutoChunk && (int64_t)(c / 2) * kMaxHalvedChunksPerRow[fam] >= d->max_seq_len &&
           units_at(d, c) < kMinAutoUnits[fam])
        c /= 2;
    return d->page_size > c ? d->page_size : c;
}

// Workgroups of a balanced-share call, by kernel shape: the persistent grid
// of share_kernel, as many per compute unit (256 on an MI355X) as the
// shape's LDS ring lets be resident -- 64, 96 and 48 KiB -- so that every
// share streams from the start.
constexpr int kCUs = 256;
constexpr int kSharesPerCU[3] = {2, 1, 3};

// The library picks balanced shares (chunk_size 0) only for calls with at
// least kMinShareQuanta quanta of kQuantaTokens tokens per share (counted at
// max_seq_len): on smaller calls every share holds a sliver and the pieces'
// merges dominate.  Measured, µs, shares against the fixed plan taken
// instead: 1 x 64/8 heads x 32K bf16 (8 quanta per share) 54.3 against 31.1;
// 8 x U[2K, 32K] bf16 (64) 114.8 against 103.3; 8 x U[512, 16K] E4M3FN (32)
// 54.7 against 41.8; at 128 (32 x U[512, 16K] E4M3FN) shares tie the best
// fixed plan, and the 32K GQA and paged 16K E4M3FN workloads (256) gain.
constexpr int kQuantaTokens = 64;
constexpr int kMinShareQuanta = 128;

struct Plan {
    int family, chunk, shape, fused;
    int shares;         // balanced shares: the workgroups that split the call (0: fixed chunks)
    int share_chunks;   // balanced shares of whole chunks (chunk_size given), else pieces
};

// The plan of a call whose shape has passed check_shape(); FD_ERR_SHAPE for
// a forced shape or placement the family does not have.
inline int plan_of(const fd_attn_desc_t *d, Plan *pl)
{
    const TableRow &r = table_row(d);
    pl->family = family_of(d);
    pl->chunk = chunk_of(d);
    const int forced_shape = (d->plan & FD_PLAN_SHAPE_MASK) - 1;
    if (forced_shape >= kShapes[pl->family]) return FD_ERR_SHAPE;
    pl->shape = forced_shape >= 0 ? forced_shape : (pl->chunk == r.chunk ? r.shape : 0);
    const int place = d->plan & (FD_PLAN_FUSED | FD_PLAN_SPLIT);
    if (place == (FD_PLAN_FUSED | FD_PLAN_SPLIT) ||
        (d->plan & ~(FD_PLAN_SHAPE_MASK | FD_PLAN_FUSED | FD_PLAN_SPLIT | FD_PLAN_SHARES)))
        return FD_ERR_SHAPE;
    // balanced shares: grouped families only; forced, or the library's pick
    // for chunk_size == 0 when nothing is forced.  With chunk_size 0 the
    // units are pieces cut at the shares' edges (merged in the launch); with
    // a chunk size (a multiple of 64) they are whole chunks, merged as with
    // fixed chunks (in the launch unless a merge launch is forced).
    pl->shares = 0;
    pl->share_chunks = 0;
    if (d->plan & FD_PLAN_SHARES) {
        if (pl->family == kFamVector) return FD_ERR_SHAPE;
        pl->shares = kCUs * kSharesPerCU[pl->shape];
        if (d->chunk_size) {
            if (d->chunk_size % 64) return FD_ERR_SHAPE;
            pl->share_chunks = 1;
            pl->fused = place != FD_PLAN_SPLIT;
        } else {
            if (place == FD_PLAN_SPLIT) return FD_ERR_SHAPE;
            pl->chunk = 0;
            pl->fused = 1;
        }
        return FD_OK;
    }
    if (d->plan == 0 && pl->family != kFamVector) {
        const int64_t groups =
            (int64_t)d->batch * (d->num_q_heads / heads_per_block(d->num_q_heads / d->num_kv_heads));
        const bool serve = groups >= kServeGroups[pl->family];
        const int auto_shape = r.shares ? r.shares - 1 : 2;
        const int64_t quanta = groups * (((int64_t)d->max_seq_len + kQuantaTokens - 1) / kQuantaTokens);
        if (d->chunk_size == 0 && (r.shares || groups >= kServeGroupsAuto[pl->family]) &&
            quanta >= (int64_t)kMinShareQuanta * kCUs * kSharesPerCU[auto_shape]) {
            if (groups >= kServeGroupsAuto[pl->family] && d->max_seq_len <= kServeWholeMax) {
                // serving batches of short rows: whole-chunk shares, one
                // chunk covering every row (written directly, no merge)
                int c = 64;
                while (c < d->max_seq_len) c *= 2;
                pl->shape = 2;
                pl->shares = kCUs * kSharesPerCU[2];
                pl->share_chunks = 1;
                pl->chunk = c < d->page_size ? d->page_size : c;
                pl->fused = 1;
                return FD_OK;
            }
            pl->shape = auto_shape;
            pl->shares = kCUs * kSharesPerCU[pl->shape];
            pl->chunk = 0;
            pl->fused = 1;
            return FD_OK;
        }
        if (d->chunk_size != 0 && d->chunk_size % 64 == 0 && serve) {
            pl->shape = 2;
            pl->shares = kCUs * kSharesPerCU[2];
            pl->share_chunks = 1;
            pl->fused = pl->chunk >= d->max_seq_len;
            return FD_OK;
        }
    }
    const int64_t maxch = ((int64_t)d->max_seq_len + pl->chunk - 1) / pl->chunk;
    const int blocks = pl->family == kFamVector ? d->num_q_heads
                                                : d->num_q_heads / heads_per_block(d->num_q_heads / d->num_kv_heads);
    const int64_t units = maxch * blocks * d->batch;
    pl->fused = place == FD_PLAN_FUSED   ? 1
                : place == FD_PLAN_SPLIT ? 0
                                         : units <= kSmallGrid || pl->chunk <= r.fused_chunk ||
                                               pl->chunk >= d->max_seq_len;
    return FD_OK;
}

// Shape checks shared by the size query and the call.
inline int check_shape(const fd_attn_desc_t *d)
{
    if (d->batch < 1 || d->num_q_heads < 1 || d->num_kv_heads < 1) return FD_ERR_SHAPE;
    if (d->batch > 65535 || d->num_q_heads > 65535) return FD_ERR_SHAPE;   // grid limits
    if (d->num_q_heads % d->num_kv_heads) return FD_ERR_SHAPE;
    if (d->head_dim != fd::kHeadDim) return FD_ERR_SHAPE;
    if (d->max_seq_len < 1 || d->max_seq_len > (1 << 23)) return FD_ERR_SHAPE;
    const int chunk = chunk_of(d);
    if (chunk < 32 || chunk % 32) return FD_ERR_SHAPE;
    if (d->page_size) {
        if (!is_pow2(d->page_size) || d->page_size < 16 || d->page_size > 256) return FD_ERR_SHAPE;
        if (chunk % d->page_size) return FD_ERR_SHAPE;
        if (d->num_pages < 1) return FD_ERR_SHAPE;
        if ((int64_t)d->max_blocks_per_seq * d->page_size < d->max_seq_len) return FD_ERR_SHAPE;
    }
    const int64_t maxch = ((int64_t)d->max_seq_len + chunk - 1) / chunk;
    const int64_t slots = (int64_t)d->batch * d->num_q_heads * maxch;
    if (slots >= ((int64_t)1 << 31) || maxch >= ((int64_t)1 << 31)) return FD_ERR_SHAPE;
    if ((int64_t)d->batch * d->num_q_heads >= ((int64_t)1 << 31)) return FD_ERR_SHAPE;
    Plan pl;
    return plan_of(d, &pl);
}

}  // namespace host
}  // namespace fd
