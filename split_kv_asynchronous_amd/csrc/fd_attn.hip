// Host side of the C ABI declared in include/fd_attn.h: validation, workspace
// carve-up, kernel choice and launches.  No allocation, no synchronisation.
#include <hip/hip_ext.h>
#include <atomic>
#include <mutex>
#include <math.h>
#include <string.h>

#include "fd_chunk.h"
#include "fd_common.h"
#include "fd_coop.h"
#include "fd_host.h"
#include "fd_merge.h"
#include "fd_mfma.h"
#include "fd_valu.h"


namespace {

using fd::Params;
using fd::host::aligned16;
using fd::host::check_shape;

constexpr size_t kAlign = 256;
constexpr size_t kFusedWordOffset = 64;   // header word counting a fused call's merged row groups
constexpr size_t kFusedCountOffset = 128; // header word adding up a fused call's recomputed pairs
constexpr size_t kClaimOffset = 192;      // header word counting a balanced-share call's claimed grains

size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

struct Layout {
    size_t header, o_part, l_part, m_part, cflag, rg_count, total;
};

// `slots` partials of one row each, and one counter per row.
Layout layout_of(size_t rows, size_t slots)
{
    Layout L;
    L.header = 0;
    L.o_part = kAlign;
    L.l_part = align_up(L.o_part + slots * fd::kHeadDim * sizeof(float));
    L.m_part = align_up(L.l_part + slots * sizeof(float));
    L.cflag = align_up(L.m_part + slots * sizeof(float));
    L.rg_count = align_up(L.cflag + slots);
    L.total = align_up(L.rg_count + rows * sizeof(unsigned long long));
    return L;
}

// Partial slots of a plan: one per (row, chunk) with fixed chunks; with
// balanced shares GB per (segment, row group) piece, at (s + r) GB for
// segment s and row group r (s + r grows strictly along the cut): at most
// (segments + row groups) GB, segments being the shares plus the pool grains
// of the largest call the descriptor allows (every length max_seq_len).
size_t slots_of(const fd_attn_desc_t *d, const fd::host::Plan &pl)
{
    const size_t rows = (size_t)d->batch * d->num_q_heads;
    if (pl.shares && !pl.share_chunks) {
        const int gb = fd::host::heads_per_block(d->num_q_heads / d->num_kv_heads);
        const uint64_t qmax = ((uint64_t)d->max_seq_len + fd::ring::kQuantum - 1) / fd::ring::kQuantum;
        const uint64_t nmax = qmax * (uint64_t)d->batch * (uint64_t)(d->num_q_heads / gb);
        return ((size_t)pl.shares + fd::ring::pool_grains(nmax, pl.shares)) * gb + rows;
    }
    const size_t maxch = ((size_t)d->max_seq_len + pl.chunk - 1) / pl.chunk;
    return rows * maxch;
}

// A fresh nonzero epoch for every call (see fd_merge.h): the workspace's
// counters carry the epoch of the call that last wrote them.
uint32_t next_epoch()
{
    static std::atomic<uint32_t> epoch{0};
    uint32_t e = epoch.fetch_add(1, std::memory_order_relaxed) + 1;
    while (e == 0) e = epoch.fetch_add(1, std::memory_order_relaxed) + 1;
    return e;
}

using fd::host::heads_per_block;
using fd::host::Plan;

// Kernel shapes of the grouped families, by the plan's shape index (the
// lists in fd_host.h).
using ChunkShape0 = fd::chunk::Shape<4, 1, 2>;
using ChunkShape1 = fd::chunk::Shape<4, 1, 3>;
using ChunkShape2 = fd::chunk::Shape<2, 1, 3>;
using CoopShape0 = fd::coop::Shape<2, 1, 3>;
using CoopShape1 = fd::coop::Shape<4, 1, 3>;
using CoopShape2 = fd::coop::Shape<2, 1, 4>;

template <typename S, bool PAGED>
int launch_chunk(const Params &p, dim3 grid, hipStream_t s, hipEvent_t e0, hipEvent_t e1)
{
    return fd::host::launch(fd::chunk::chunk_kernel<FD_BF16, PAGED, S>, grid, dim3(S::waves * 64), 0, s, e0, e1, p);
}

template <typename S, bool PAGED>
int launch_coop(const Params &p, dim3 grid, hipStream_t s, hipEvent_t e0, hipEvent_t e1)
{
    return fd::host::launch(fd::coop::chunk_kernel<FD_FP8_E4M3FN, PAGED, S>, grid, dim3(S::waves * 64), 0, s, e0,
                            e1, p);
}

template <bool PAGED>
int dispatch_grouped(const Params &p, int family, int shape, dim3 grid, hipStream_t s, hipEvent_t e0, hipEvent_t e1)
{
    if (family == fd::host::kFamGroupedBf16) {
        if (shape == 1) return launch_chunk<ChunkShape1, PAGED>(p, grid, s, e0, e1);
        if (shape == 2) return launch_chunk<ChunkShape2, PAGED>(p, grid, s, e0, e1);
        return launch_chunk<ChunkShape0, PAGED>(p, grid, s, e0, e1);
    }
    if (shape == 1) return launch_coop<CoopShape1, PAGED>(p, grid, s, e0, e1);
    if (shape == 2) return launch_coop<CoopShape2, PAGED>(p, grid, s, e0, e1);
    return launch_coop<CoopShape0, PAGED>(p, grid, s, e0, e1);
}

template <typename S, int KV, bool PAGED>
int launch_shares(const Params &p, dim3 grid, hipStream_t s, hipEvent_t e0, hipEvent_t e1)
{
    return fd::host::launch(fd::chunk::share_kernel<KV, PAGED, S>, grid, dim3(S::waves * 64), 0, s, e0, e1, p);
}

// Balanced shares run the ring kernel of fd_chunk.h for both cache formats.
template <bool PAGED>
int dispatch_shares(const Params &p, int family, int shape, dim3 grid, hipStream_t s, hipEvent_t e0, hipEvent_t e1)
{
    if (family == fd::host::kFamGroupedBf16) {
        if (shape == 1) return launch_shares<ChunkShape1, FD_BF16, PAGED>(p, grid, s, e0, e1);
        if (shape == 2) return launch_shares<ChunkShape2, FD_BF16, PAGED>(p, grid, s, e0, e1);
        return launch_shares<ChunkShape0, FD_BF16, PAGED>(p, grid, s, e0, e1);
    }
    if (shape == 1) return launch_shares<ChunkShape1, FD_FP8_E4M3FN, PAGED>(p, grid, s, e0, e1);
    if (shape == 2) return launch_shares<ChunkShape2, FD_FP8_E4M3FN, PAGED>(p, grid, s, e0, e1);
    return launch_shares<ChunkShape0, FD_FP8_E4M3FN, PAGED>(p, grid, s, e0, e1);
}

template <int KV, int QT, bool PAGED>
int launch_valu(const Params &p, dim3 grid, hipStream_t s, hipEvent_t e0, hipEvent_t e1)
{
    return fd::host::launch(fd::partial_valu_kernel<KV, QT, PAGED>, grid, dim3(256), 0, s, e0, e1, p);
}

// Dispatch on (kv dtype, q dtype, paged) for the vector path.
int dispatch_valu(const Params &p, int kv, int qt, bool paged, dim3 grid, hipStream_t s, hipEvent_t e0,
                  hipEvent_t e1)
{
#define FD_CASE(KV, QT, PG)                                                   \
    if (kv == KV && qt == QT && paged == PG) return launch_valu<KV, QT, PG>(p, grid, s, e0, e1);
    FD_CASE(FD_F32, FD_F32, false) FD_CASE(FD_F32, FD_F32, true)
    FD_CASE(FD_F32, FD_BF16, false) FD_CASE(FD_F32, FD_BF16, true)
    FD_CASE(FD_BF16, FD_F32, false) FD_CASE(FD_BF16, FD_F32, true)
    FD_CASE(FD_BF16, FD_BF16, false) FD_CASE(FD_BF16, FD_BF16, true)
    FD_CASE(FD_FP8_E4M3FN, FD_F32, false) FD_CASE(FD_FP8_E4M3FN, FD_F32, true)
    FD_CASE(FD_FP8_E4M3FN, FD_BF16, false) FD_CASE(FD_FP8_E4M3FN, FD_BF16, true)
#undef FD_CASE
    return FD_ERR_DTYPE;
}

}  // namespace

extern "C" size_t fd_attn_workspace_size(const fd_attn_desc_t *desc)
{
    if (!desc || check_shape(desc) != FD_OK) return 0;
    fd::host::Plan pl;
    fd::host::plan_of(desc, &pl);
    return layout_of((size_t)desc->batch * desc->num_q_heads, slots_of(desc, pl)).total;
}

extern "C" int fd_attn_plan(const fd_attn_desc_t *desc, int32_t *chunk_size, int32_t *family, int32_t *shape,
                            int32_t *fused, int32_t *shares)
{
    if (!desc) return FD_ERR_NULL;
    const int rc = check_shape(desc);
    if (rc != FD_OK) return rc;
    Plan pl;
    fd::host::plan_of(desc, &pl);
    if (chunk_size) *chunk_size = pl.chunk;
    if (family) *family = pl.family;
    if (shape) *shape = pl.shape;
    if (fused) *fused = pl.fused;
    if (shares) *shares = pl.shares;
    return FD_OK;
}

extern "C" const char *fd_attn_status_string(int status)
{
    switch (status) {
    case FD_OK: return "ok";
    case FD_ERR_NULL: return "a required pointer is NULL";
    case FD_ERR_SHAPE: return "invalid or inconsistent sizes in the descriptor";
    case FD_ERR_DTYPE: return "unsupported storage format combination";
    case FD_ERR_ALIGN: return "q, caches and out must be 16-byte aligned";
    case FD_ERR_BAND: return "phi, a, b must be finite with 0 <= a, b <= 64";
    case FD_ERR_WORKSPACE: return "workspace missing, unaligned or too small";
    case FD_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
    }
}

namespace {

// Every check of a decode call but the workspace's.
int validate(const fd_attn_desc_t *d, const void *q, const void *k_cache, const void *v_cache,
             const int32_t *seq_lens, const int32_t *block_table, float phi, float a, float b, const void *out,
             const uint8_t *fallback_flags)
{
    if (!d || !q || !k_cache || !v_cache || !seq_lens || !out || !fallback_flags) return FD_ERR_NULL;
    int rc = check_shape(d);
    if (rc != FD_OK) return rc;
    if (d->page_size && !block_table) return FD_ERR_NULL;
    const int qt = d->q_dtype, kv = d->kv_dtype, ot = d->out_dtype;
    if (qt != FD_F32 && qt != FD_BF16) return FD_ERR_DTYPE;
    if (kv != FD_F32 && kv != FD_BF16 && kv != FD_FP8_E4M3FN) return FD_ERR_DTYPE;
    if (ot != FD_F32 && ot != FD_BF16) return FD_ERR_DTYPE;
    if (kv == FD_FP8_E4M3FN && (!d->k_scale || !d->v_scale)) return FD_ERR_NULL;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
        return FD_ERR_ALIGN;
    if (!isfinite(phi) || !isfinite(a) || !isfinite(b) || a < 0.f || b < 0.f || a > 64.f ||
        b > 64.f)
        return FD_ERR_BAND;
    if (!isfinite(d->scale)) return FD_ERR_SHAPE;
    return FD_OK;
}

// Enqueues a validated call with workspace `wsp` (256-byte aligned, at least
// fd_attn_workspace_size(d) bytes).
int enqueue(const fd_attn_desc_t *d, const void *q, const void *k_cache, const void *v_cache,
            const int32_t *seq_lens, const int32_t *block_table, float phi, float a, float b, void *out,
            uint8_t *fallback_flags, void *wsp, hipStream_t stream)
{
    const int qt = d->q_dtype, kv = d->kv_dtype, ot = d->out_dtype;
    Plan pl;
    int rc = fd::host::plan_of(d, &pl);
    if (rc != FD_OK) return rc;
    const int chunk = pl.chunk ? pl.chunk : fd::host::chunk_of(d);   // 0: pieces (p.chunk unused)
    const int maxch = (d->max_seq_len + chunk - 1) / chunk;
    const size_t rows = (size_t)d->batch * d->num_q_heads;
    const Layout L = layout_of(rows, slots_of(d, pl));
    uint8_t *ws = static_cast<uint8_t *>(wsp);

    Params p;
    memset(&p, 0, sizeof p);
    p.q = q;
    p.k = k_cache;
    p.v = v_cache;
    p.seq_lens = seq_lens;
    p.block_table = block_table;
    p.k_scale = kv == FD_FP8_E4M3FN ? d->k_scale : nullptr;
    p.v_scale = kv == FD_FP8_E4M3FN ? d->v_scale : nullptr;
    p.out = out;
    p.flags = fallback_flags;
    p.count_word = reinterpret_cast<unsigned long long *>(ws + L.header);
    p.fused_word = reinterpret_cast<unsigned long long *>(ws + L.header + kFusedWordOffset);
    p.fused_count = reinterpret_cast<unsigned long long *>(ws + L.header + kFusedCountOffset);
    p.claim_word = reinterpret_cast<unsigned long long *>(ws + L.header + kClaimOffset);
    p.rg_count = reinterpret_cast<unsigned long long *>(ws + L.rg_count);
    p.epoch = next_epoch();
    p.o_part = reinterpret_cast<float *>(ws + L.o_part);
    p.l_part = reinterpret_cast<float *>(ws + L.l_part);
    p.m_part = reinterpret_cast<float *>(ws + L.m_part);
    p.cflag = ws + L.cflag;
    p.batch = d->batch;
    p.hq = d->num_q_heads;
    p.hkv = d->num_kv_heads;
    p.group = d->num_q_heads / d->num_kv_heads;
    p.max_seq_len = d->max_seq_len;
    p.chunk = chunk;
    p.maxch = maxch;
    p.page_shift = 0;
    if (d->page_size)
        while ((1 << p.page_shift) < d->page_size) ++p.page_shift;
    p.max_blocks = d->max_blocks_per_seq;
    p.scale = d->scale > 0.f ? d->scale : 1.0f / sqrtf((float)fd::kHeadDim);
    p.phi = phi;
    p.lo = (float)((double)phi - (double)a);
    p.hi = (float)((double)phi + (double)b);
    p.out_bf16 = ot == FD_BF16;

    const bool paged = d->page_size != 0;
    const bool use_mfma = pl.family != fd::host::kFamVector;
    // Optional timing: the chunk kernel is launched with start/stop events
    // stamped by its own dispatch packet, so timing adds no marker packets.
    hipEvent_t *ev = d->stage_events;
    hipEvent_t ev0 = ev ? ev[0] : nullptr, ev1 = ev ? ev[1] : nullptr;

    // the merge runs inside the chunk launch (the last workgroup of each row
    // group merges it) or in a second launch, as the plan says
    p.fused = pl.fused;
    p.share_chunks = pl.share_chunks;

    if (use_mfma && pl.shares) {
        // a persistent grid: workgroup w takes share w of the call
        p.heads_per_block = heads_per_block(p.group);
        p.ngroups = p.batch * (p.hq / p.heads_per_block);
        rc = paged ? dispatch_shares<true>(p, pl.family, pl.shape, dim3((unsigned)pl.shares), stream, ev0, ev1)
                   : dispatch_shares<false>(p, pl.family, pl.shape, dim3((unsigned)pl.shares), stream, ev0, ev1);
    } else if (use_mfma) {
        p.heads_per_block = heads_per_block(p.group);
        // One workgroup per unit; workgroups past the real units exit at once.
        // The unit index is blockIdx.y * gridDim.x + blockIdx.x.
        const size_t units = (size_t)maxch * (p.hq / p.heads_per_block) * p.batch;
        const unsigned gx = (unsigned)(units < ((size_t)1 << 20) ? units : ((size_t)1 << 20));
        const dim3 flat(gx, (unsigned)((units + gx - 1) / gx));
        p.ngroups = p.batch * (p.hq / p.heads_per_block);
        rc = paged ? dispatch_grouped<true>(p, pl.family, pl.shape, flat, stream, ev0, ev1)
                   : dispatch_grouped<false>(p, pl.family, pl.shape, flat, stream, ev0, ev1);
    } else {
        p.heads_per_block = 1;
        p.ngroups = p.batch * p.hq;
        rc = dispatch_valu(p, kv, qt, paged, dim3(maxch, p.hq, p.batch), stream, ev0, ev1);
    }
    if (rc != FD_OK) return rc;

    // Every kernel recomputes an out-of-band chunk inside the workgroup that
    // found it.  Small grids merge inside the same launch (p.fused); larger
    // ones in a second launch, RW wavefronts per row for rows with many chunks.
    if (!p.fused) {
        if (maxch >= 64)
            rc = fd::host::launch(fd::merge_kernel<4>, dim3((unsigned)rows), dim3(256), 0, stream, nullptr, nullptr, p);
        else if (maxch >= 16)
            rc = fd::host::launch(fd::merge_kernel<2>, dim3((unsigned)((rows + 1) / 2)), dim3(256), 0, stream, nullptr,
                        nullptr, p);
        else
            rc = fd::host::launch(fd::merge_kernel<1>, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, nullptr,
                        nullptr, p);
    }
    return rc;
}

// ---- workspace in a static device array, for callers that cannot allocate
// (see fd_attn_decode_static).  Every GPU the library runs on holds its own
// copy from the library's load until the process ends.  In host code the
// array's name is only a host-side stand-in: kernels get the device address
// that hipGetSymbolAddress gives for the device, looked up once per device
// (with that device current) and kept.
static __device__ __align__(256) uint8_t scratch[FD_ATTN_STATIC_WORKSPACE_BYTES];

constexpr int kMaxDevices = 64;

int scratch_address(hipStream_t stream, void **ptr)
{
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    int dev = 0, cur = 0;
    if (hipStreamGetDevice(stream, &dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FD_ERR_LAUNCH;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        if (hipGetDevice(&cur) != hipSuccess) return FD_ERR_LAUNCH;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return FD_ERR_LAUNCH;
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) (void)hipSetDevice(cur);
        if (e != hipSuccess || !p || ((uintptr_t)p & (kAlign - 1))) return FD_ERR_LAUNCH;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return FD_OK;
}

}  // namespace

extern "C" int fd_attn_decode(const fd_attn_desc_t *d, const void *q, const void *k_cache,
                              const void *v_cache, const int32_t *seq_lens,
                              const int32_t *block_table, float phi, float a, float b, void *out,
                              uint8_t *fallback_flags, hipStream_t stream)
{
    const int rc = validate(d, q, k_cache, v_cache, seq_lens, block_table, phi, a, b, out, fallback_flags);
    if (rc != FD_OK) return rc;
    const size_t need = fd_attn_workspace_size(d);
    if (!d->workspace || ((uintptr_t)d->workspace & (kAlign - 1)) || d->workspace_bytes < need)
        return FD_ERR_WORKSPACE;
    return enqueue(d, q, k_cache, v_cache, seq_lens, block_table, phi, a, b, out, fallback_flags, d->workspace,
                   stream);
}

extern "C" int fd_attn_decode_static(const fd_attn_desc_t *d, const void *q, const void *k_cache,
                                     const void *v_cache, const int32_t *seq_lens,
                                     const int32_t *block_table, float phi, float a, float b, void *out,
                                     uint8_t *fallback_flags, hipStream_t stream)
{
    int rc = validate(d, q, k_cache, v_cache, seq_lens, block_table, phi, a, b, out, fallback_flags);
    if (rc != FD_OK) return rc;
    if (fd_attn_workspace_size(d) > FD_ATTN_STATIC_WORKSPACE_BYTES) return FD_ERR_WORKSPACE;
    void *ws = nullptr;
    rc = scratch_address(stream, &ws);
    if (rc != FD_OK) return rc;
    return enqueue(d, q, k_cache, v_cache, seq_lens, block_table, phi, a, b, out, fallback_flags, ws, stream);
}
