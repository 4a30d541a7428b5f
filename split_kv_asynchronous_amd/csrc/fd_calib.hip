// Host side of include/fd_calib.h: the score-statistics pass (validation and
// launches) and the band choice (plain host code).  No allocation on the
// device, no synchronisation.
#include <hip/hip_ext.h>
#include <math.h>
#include <string.h>

#include <algorithm>
#include <queue>
#include <utility>
#include <vector>

#include "fd_calib.h"
#include "fd_host.h"
#include "fd_stats.h"

namespace {

using fd::stats::StatsParams;

template <int KV, int QT, bool PAGED>
int launch_stats(const StatsParams &sp, unsigned grid, size_t lds, hipStream_t s)
{
    return fd::host::launch(fd::stats::score_stats_kernel<KV, QT, PAGED>, dim3(grid),
                            dim3(fd::stats::kStatsWaves * 64), lds, s, nullptr, nullptr, sp);
}

int dispatch_stats(const StatsParams &sp, int kv, int qt, bool paged, unsigned grid, size_t lds,
                   hipStream_t s)
{
#define FD_CASE(KV, QT, PG) \
    if (kv == KV && qt == QT && paged == PG) return launch_stats<KV, QT, PG>(sp, grid, lds, s);
    FD_CASE(FD_F32, FD_F32, false) FD_CASE(FD_F32, FD_F32, true)
    FD_CASE(FD_F32, FD_BF16, false) FD_CASE(FD_F32, FD_BF16, true)
    FD_CASE(FD_BF16, FD_F32, false) FD_CASE(FD_BF16, FD_F32, true)
    FD_CASE(FD_BF16, FD_BF16, false) FD_CASE(FD_BF16, FD_BF16, true)
    FD_CASE(FD_FP8_E4M3FN, FD_F32, false) FD_CASE(FD_FP8_E4M3FN, FD_F32, true)
    FD_CASE(FD_FP8_E4M3FN, FD_BF16, false) FD_CASE(FD_FP8_E4M3FN, FD_BF16, true)
#undef FD_CASE
    return FD_ERR_DTYPE;
}

struct Extremes {
    double mx, mn;
};

// The smallest W such that `need` rows have max(mx) - min(mn) <= W: for each
// row j as the set's smallest minimum L, the best set takes the `need`
// smallest maxima among the rows whose minimum is at least L.
double min_width(std::vector<Extremes> rows, size_t need)
{
    if (need == 0 || rows.size() < need) return 0.0;
    std::sort(rows.begin(), rows.end(), [](const Extremes &x, const Extremes &y) { return x.mn < y.mn; });
    std::priority_queue<double> kept;   // the `need` smallest maxima seen so far (largest on top)
    double best = INFINITY;
    for (size_t j = rows.size(); j-- > 0;) {
        kept.push(rows[j].mx);
        if (kept.size() > need) kept.pop();
        if (kept.size() == need) best = std::min(best, kept.top() - rows[j].mn);
    }
    return best;
}

// The phi that keeps the most rows in [phi - a0, phi + b0]: row r is kept
// for phi in [mx_r - b0, mn_r + a0].  Returns the centre of the widest range
// of phi with the largest count (the leftmost among equally wide ones).  At
// the minimal width the best range can be a single point, which rounding
// a0 and b0 separately may miss by an ulp: each range is widened by a
// relative 1e-12 (far below any useful pad).
double best_phi(const std::vector<Extremes> &rows, double a0, double b0)
{
    std::vector<std::pair<double, int>> ev;   // (position, +1 start / -1 end); starts first on ties
    for (const Extremes &r : rows) {
        const double tol = 1e-12 * (fabs(r.mx) + fabs(r.mn) + a0 + b0 + 1.0);
        const double lo = r.mx - b0 - tol, hi = r.mn + a0 + tol;
        if (lo <= hi) {
            ev.push_back({lo, +1});
            ev.push_back({hi, -1});
        }
    }
    if (ev.empty()) return rows.empty() ? 0.0 : 0.5 * (rows[0].mx + rows[0].mn);
    std::sort(ev.begin(), ev.end(), [](const std::pair<double, int> &x, const std::pair<double, int> &y) {
        return x.first < y.first || (x.first == y.first && x.second > y.second);
    });
    int count = 0, best = -1;
    double best_lo = 0.0, best_w = -1.0;
    for (size_t i = 0; i < ev.size(); ++i) {
        count += ev[i].second;
        if (ev[i].second > 0 && (i + 1 == ev.size() || ev[i + 1].second < 0 || ev[i + 1].first > ev[i].first)) {
            // [ev[i].first, next event] carries `count` rows
            const double lo = ev[i].first;
            const double hi = (i + 1 < ev.size()) ? ev[i + 1].first : lo;
            const double w = hi - lo;
            if (count > best || (count == best && w > best_w)) {
                best = count;
                best_lo = lo;
                best_w = w;
            }
        }
    }
    return best_lo + 0.5 * best_w;
}

}  // namespace

extern "C" int fd_attn_score_stats(const fd_attn_desc_t *d, const void *q, const void *k_cache,
                                   const int32_t *seq_lens, const int32_t *block_table,
                                   float hist_lo, float hist_hi, int32_t nbins, float *row_max,
                                   float *row_min, uint32_t *hist, hipStream_t stream)
{
    if (!d || !q || !k_cache || !seq_lens || !row_max || !row_min) return FD_ERR_NULL;
    int rc = fd::host::check_shape(d);
    if (rc != FD_OK) return rc;
    if (d->page_size && !block_table) return FD_ERR_NULL;
    const int qt = d->q_dtype, kv = d->kv_dtype;
    if (qt != FD_F32 && qt != FD_BF16) return FD_ERR_DTYPE;
    if (kv != FD_F32 && kv != FD_BF16 && kv != FD_FP8_E4M3FN) return FD_ERR_DTYPE;
    if (kv == FD_FP8_E4M3FN && !d->k_scale) return FD_ERR_NULL;
    if (!fd::host::aligned16(q) || !fd::host::aligned16(k_cache)) return FD_ERR_ALIGN;
    if (!isfinite(d->scale)) return FD_ERR_SHAPE;
    if (nbins < 0 || nbins > 8192) return FD_ERR_SHAPE;
    const bool take_hist = hist && nbins > 0;
    if (take_hist && (!isfinite(hist_lo) || !isfinite(hist_hi) || !(hist_lo < hist_hi))) return FD_ERR_SHAPE;

    StatsParams sp;
    memset(&sp, 0, sizeof sp);
    fd::Params &p = sp.base;
    p.q = q;
    p.k = k_cache;
    p.seq_lens = seq_lens;
    p.block_table = block_table;
    p.k_scale = kv == FD_FP8_E4M3FN ? d->k_scale : nullptr;
    p.batch = d->batch;
    p.hq = d->num_q_heads;
    p.hkv = d->num_kv_heads;
    p.group = d->num_q_heads / d->num_kv_heads;
    p.max_seq_len = d->max_seq_len;
    p.page_shift = 0;
    if (d->page_size)
        while ((1 << p.page_shift) < d->page_size) ++p.page_shift;
    p.max_blocks = d->max_blocks_per_seq;
    p.scale = d->scale > 0.f ? d->scale : 1.0f / sqrtf((float)fd::kHeadDim);
    sp.row_max = row_max;
    sp.row_min = row_min;
    sp.hist = take_hist ? hist : nullptr;
    sp.nbins = take_hist ? nbins : 0;
    sp.hist_lo = hist_lo;
    sp.hist_hi = hist_hi;
    sp.inv_w = take_hist ? (float)((double)nbins / ((double)hist_hi - (double)hist_lo)) : 0.f;
    // grouped bf16 queries over a bf16 or E4M3FN cache: matrix-core kernel
    const bool use_mfma = p.group > 1 && qt == FD_BF16 && kv != FD_F32;
    const int heads = use_mfma ? fd::stats::kStatsMfmaHeads : fd::stats::kStatsHeads;
    sp.chunk = !use_mfma ? fd::stats::kStatsChunk
               : kv == FD_FP8_E4M3FN ? fd::stats::stats_dma_chunk<FD_FP8_E4M3FN>()
                                     : fd::stats::stats_dma_chunk<FD_BF16>();
    sp.nchunk = (d->max_seq_len + sp.chunk - 1) / sp.chunk;
    sp.nhb = (p.group + heads - 1) / heads;
    const int64_t units = (int64_t)d->batch * d->num_kv_heads * sp.nhb * sp.nchunk;
    if (units >= ((int64_t)1 << 31)) return FD_ERR_SHAPE;

    const int64_t rows = (int64_t)d->batch * d->num_q_heads;
    const int64_t init_items = std::max<int64_t>(rows, take_hist ? nbins + 2 : 0);
    const unsigned init_grid = (unsigned)std::min<int64_t>((init_items + 255) / 256, 1024);
    int lrc = fd::host::launch(fd::stats::stats_init_kernel, dim3(init_grid), dim3(256), 0, stream, nullptr,
                               nullptr, sp);
    if (lrc != FD_OK) return lrc;
    const size_t lds = take_hist ? sizeof(uint32_t) * (size_t)(nbins + 2) : 0;
    const dim3 grid((unsigned)units), block(fd::stats::kStatsWaves * 64);
    if (use_mfma) {
        // K through DMA rings, 3 stages per wavefront, or 2 when the
        // histogram leaves too little of the 64 KiB of LDS
        const size_t fixed = sizeof(float) * fd::stats::kStatsWaves * 2 * fd::stats::kStatsMfmaHeads;
        const bool deep = (size_t)fd::stats::kStatsWaves * 3 * fd::ring::kGroupBytes + lds + fixed <= 64 * 1024;
        const size_t dl = (size_t)fd::stats::kStatsWaves * (deep ? 3 : 2) * fd::ring::kGroupBytes + lds;
        const bool pg = d->page_size != 0;
#define FD_DMA(KV, PG, NST) \
    lrc = fd::host::launch(fd::stats::score_stats_dma_kernel<KV, PG, NST>, grid, block, dl, stream, nullptr, nullptr, sp)
        if (kv == FD_BF16) {
            if (deep) { if (pg) FD_DMA(FD_BF16, true, 3); else FD_DMA(FD_BF16, false, 3); }
            else { if (pg) FD_DMA(FD_BF16, true, 2); else FD_DMA(FD_BF16, false, 2); }
        } else {
            if (deep) { if (pg) FD_DMA(FD_FP8_E4M3FN, true, 3); else FD_DMA(FD_FP8_E4M3FN, false, 3); }
            else { if (pg) FD_DMA(FD_FP8_E4M3FN, true, 2); else FD_DMA(FD_FP8_E4M3FN, false, 2); }
        }
#undef FD_DMA
    } else {
        lrc = dispatch_stats(sp, kv, qt, d->page_size != 0, (unsigned)units, lds, stream);
    }
    return lrc;
}

extern "C" int fd_attn_choose_band(const float *row_max, const float *row_min, int64_t nrows,
                                   double max_flag_fraction, double a_share, double max_width,
                                   double pad, float *phi, float *a, float *b, int64_t *flagged)
{
    if ((!row_max || !row_min) && nrows > 0) return FD_ERR_NULL;
    if (!phi || !a || !b || !flagged) return FD_ERR_NULL;
    if (nrows < 0) return FD_ERR_SHAPE;
    if (!(max_flag_fraction >= 0.0 && max_flag_fraction <= 1.0)) return FD_ERR_BAND;
    if (!(a_share >= 0.0 && a_share <= 1.0)) return FD_ERR_BAND;
    if (!(max_width > 0.0) || !isfinite(max_width)) return FD_ERR_BAND;
    if (!(pad >= 0.0) || !isfinite(pad)) return FD_ERR_BAND;

    std::vector<Extremes> rows;
    rows.reserve((size_t)nrows);
    for (int64_t r = 0; r < nrows; ++r)
        if ((double)row_max[r] >= (double)row_min[r]) rows.push_back({(double)row_max[r], (double)row_min[r]});
    const size_t m = rows.size();
    const size_t allowed = (size_t)floor(max_flag_fraction * (double)m);
    const size_t need = m - std::min(allowed, m);

    const double W = std::min(min_width(rows, need), max_width);
    const double a0 = a_share * W, b0 = (1.0 - a_share) * W;
    const double ph = best_phi(rows, a0, b0);
    *phi = (float)ph;
    *a = (float)(a0 + pad);
    *b = (float)(b0 + pad);
    // rows the returned (float) band keeps, on the given extremes
    const double lo = (double)*phi - (double)*a, hi = (double)*phi + (double)*b;
    int64_t kept = 0;
    for (const Extremes &r : rows)
        if (lo <= r.mn && r.mx <= hi) ++kept;
    *flagged = (int64_t)m - kept;
    return FD_OK;
}
