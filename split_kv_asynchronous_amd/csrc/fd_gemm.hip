// Host side of include/fd_gemm.h: validation, the configuration choice (a
// table measured offline, keyed by the layer's N and K and by M, and a rule
// for other shapes) and the launches.  No allocation, no synchronisation.
#include <hip/hip_ext.h>
#include <string.h>

#include <algorithm>

#include "fd_gemm.h"
#include "fd_gemm_kernel.h"
#include "fd_host.h"

namespace {

using fd::gemm::GemmParams;

// kind 0: A staged in LDS, weights loaded into registers by 4 wavefronts on
// different column blocks; kind 1: wk wavefronts split the workgroup's K
// slice of one column block and load A directly; kind 2: weights moved by
// DMA into per-wavefront LDS rings of nst stages of kst k-steps, A staged in
// LDS, 4 wavefronts on different column blocks.
struct Variant {
    int kind, wk, nb, gu, kst, nst;
};

constexpr Variant kVariants[FD_GEMM_VARIANTS] = {
    {0, 1, 1, 8, 0, 0},  {0, 1, 2, 4, 0, 0},  {0, 1, 1, 16, 0, 0}, {0, 1, 2, 8, 0, 0},
    {1, 4, 4, 4, 0, 0},  {1, 4, 2, 8, 0, 0},  {1, 4, 1, 8, 0, 0},  {1, 4, 1, 16, 0, 0},
    {1, 8, 1, 8, 0, 0},  {1, 8, 2, 4, 0, 0},  {1, 16, 1, 4, 0, 0}, {1, 16, 1, 8, 0, 0},
    {2, 1, 1, 0, 4, 3},  {2, 1, 1, 0, 4, 2},
};

constexpr size_t kLdsBudget = 64 * 1024;   // dynamic LDS without an attribute change

// Offline-measured picks (MI355X, bf16 weights rotated through more than the
// last-level cache, calls timed back to back in a graph): the layer's (N, K),
// an M range, and the variant and K slices that were fastest there.  Rows:
// the Q/K/V, O, gate/up and down projections of a 7B-class decoder block.
struct TableRow {
    int n, k, m_lo, m_hi, variant, ksplit;
};
constexpr TableRow kTable[] = {
    {12288, 4096, 1, 6, 7, 1},   {12288, 4096, 7, 24, 3, 4},  {12288, 4096, 25, 48, 2, 8},
    {12288, 4096, 49, 64, 5, 1},
    {4096, 4096, 1, 6, 7, 1},    {4096, 4096, 7, 24, 9, 1},   {4096, 4096, 25, 64, 5, 4},
    {22016, 4096, 1, 2, 14, 8},  {22016, 4096, 3, 6, 7, 2},   {22016, 4096, 7, 12, 6, 1},
    {22016, 4096, 13, 24, 1, 4}, {22016, 4096, 25, 48, 1, 8}, {22016, 4096, 49, 64, 5, 2},
    {4096, 11008, 1, 12, 8, 1},  {4096, 11008, 13, 24, 6, 4}, {4096, 11008, 25, 64, 5, 4},
};

// The same for packed weights (direct variants only).
constexpr TableRow kTablePacked[] = {
    {12288, 4096, 1, 12, 7, 1},   {12288, 4096, 13, 48, 6, 2},  {12288, 4096, 49, 64, 5, 1},
    {4096, 4096, 1, 2, 11, 1},    {4096, 4096, 3, 12, 7, 1},    {4096, 4096, 13, 24, 9, 1},
    {4096, 4096, 25, 48, 10, 2},  {4096, 4096, 49, 64, 5, 4},
    {22016, 4096, 1, 2, 7, 1},    {22016, 4096, 3, 6, 7, 4},    {22016, 4096, 7, 12, 7, 1},
    {22016, 4096, 13, 24, 6, 2},  {22016, 4096, 25, 48, 6, 1},  {22016, 4096, 49, 64, 5, 2},
    {4096, 11008, 1, 2, 11, 1},   {4096, 11008, 3, 12, 8, 1},   {4096, 11008, 13, 24, 6, 2},
    {4096, 11008, 25, 64, 5, 4},
};

// Packed weights, other shapes: the direct variant with 16-column blocks up
// to 12 rows, 32-column blocks up to 48, 64-column blocks beyond.
void rule_packed(int m, int *variant, int *target)
{
    if (m <= 12) {
        *variant = 7;
        *target = 256;
    } else if (m <= 48) {
        *variant = 6;
        *target = 512;
    } else {
        *variant = 5;
        *target = 256;
    }
}

// The rule for other shapes, read off the same measurements: up to 8 rows the
// direct variant with 16-column blocks; up to 24 rows A staged in LDS (shared
// by 4 column blocks); beyond, the direct variant with 64-column blocks.
// K is split until the grid has `target` workgroups (as far as one load batch
// per wavefront allows).
void rule(int m, int *variant, int *target)
{
    if (m <= 8) {
        *variant = 7;
        *target = 256;
    } else if (m <= 24) {
        *variant = 1;
        *target = 768;
    } else {
        *variant = 5;
        *target = 256;
    }
}

struct Plan {
    int variant, ksplit, per, mb, tiles, mgroups, ring, packed;
};

int check(const fd_gemm_desc_t *d)
{
    if (d->m < 1 || d->m > 4096) return FD_ERR_SHAPE;
    if (d->n < 1 || d->n > (1 << 20)) return FD_ERR_SHAPE;
    if (d->k < 32 || d->k > (1 << 20) || d->k % 32) return FD_ERR_SHAPE;
    if (d->a_dtype != FD_BF16 || d->w_dtype != FD_BF16) return FD_ERR_DTYPE;
    if (d->out_dtype != FD_F32 && d->out_dtype != FD_BF16) return FD_ERR_DTYPE;
    if (d->variant < 0 || d->variant > FD_GEMM_VARIANTS) return FD_ERR_SHAPE;
    if (d->w_layout != FD_GEMM_W_ROWS && d->w_layout != FD_GEMM_W_PACKED) return FD_ERR_DTYPE;
    if (d->w_layout == FD_GEMM_W_PACKED && d->variant && (d->variant < 5 || d->variant > 12)) return FD_ERR_SHAPE;
    if (d->ksplit < 0 || d->ksplit > d->k / 32) return FD_ERR_SHAPE;
    return FD_OK;
}

int make_plan(const fd_gemm_desc_t *d, Plan *pl)
{
    const int rc = check(d);
    if (rc != FD_OK) return rc;
    const int ksteps = d->k / 32;
    const int mb = (std::min(d->m, fd::gemm::kGemmMaxRows) + 15) / 16;
    const bool packed = d->w_layout == FD_GEMM_W_PACKED;
    int variant = d->variant, ksplit = d->ksplit;
    if (variant == 0 || ksplit == 0) {
        const TableRow *tab = packed ? kTablePacked : kTable;
        const size_t rows = packed ? sizeof(kTablePacked) / sizeof(TableRow) : sizeof(kTable) / sizeof(TableRow);
        for (size_t i = 0; i < rows; ++i) {
            const TableRow &r = tab[i];
            if (r.n == d->n && r.k == d->k && r.m_lo <= d->m && d->m <= r.m_hi) {
                if (variant == 0) variant = r.variant;
                if (ksplit == 0) ksplit = r.ksplit;
                break;
            }
        }
    }
    int target = 256;
    {
        int rv;
        if (packed) rule_packed(d->m, &rv, &target);
        else rule(d->m, &rv, &target);
        if (variant == 0) variant = rv;
    }
    const Variant &v = kVariants[variant - 1];
    const int cols = (v.kind == 1 ? 1 : 4) * v.nb * 16;
    const int tiles = (d->n + cols - 1) / cols;
    const int mgroups = (d->m + fd::gemm::kGemmMaxRows - 1) / fd::gemm::kGemmMaxRows;
    // the largest slice whose rows of A fit the LDS budget (beside the DMA
    // rings), in whole DMA stages
    const size_t ring = v.kind == 2 ? (size_t)4 * v.nst * 1024 * v.kst : 0;
    int max_per = v.kind == 1 ? ksteps : (int)(((kLdsBudget - ring) / (16 * mb) - 16) / 64);
    if (v.kind == 2) {
        if (ksteps % v.kst) return FD_ERR_SHAPE;          // slices of whole stages
        max_per -= max_per % v.kst;
        if (max_per < v.kst) return FD_ERR_SHAPE;
    }
    const int min_per = v.kind == 0 ? v.gu : v.kind == 1 ? v.wk * v.gu : v.nst * v.kst;
    if (ksplit == 0) {
        const int64_t base = (int64_t)tiles * mgroups;
        int want = (int)std::min<int64_t>((target + base - 1) / base, ksteps);
        want = std::min(want, std::max(1, ksteps / min_per));
        ksplit = std::max(want, 1);
    }
    int per = (ksteps + ksplit - 1) / ksplit;
    if (v.kind == 2) per = (per + v.kst - 1) / v.kst * v.kst;
    per = std::min(per, max_per);
    ksplit = (ksteps + per - 1) / per;   // no empty slice
    if ((int64_t)tiles * ksplit >= ((int64_t)1 << 31)) return FD_ERR_SHAPE;
    *pl = Plan{variant, ksplit, per, mb, tiles, mgroups, (int)ring, packed ? 1 : 0};
    return FD_OK;
}

template <int MB, int NB, int GU, int WAVES>
int launch_main(const GemmParams &gp, const Plan &pl, hipStream_t s, hipEvent_t e0, hipEvent_t e1)
{
    const size_t lds = fd::gemm::gemm_lds_bytes(16 * MB, pl.per);
    return fd::host::launch(fd::gemm::flat_gemm_kernel<MB, NB, GU, WAVES>,
                            dim3((unsigned)(pl.tiles * pl.ksplit), (unsigned)pl.mgroups), dim3(WAVES * 64), lds,
                            s, e0, e1, gp);
}

template <int MB, int NB, int GU, int WK, bool WP>
int launch_direct_wp(const GemmParams &gp, const Plan &pl, hipStream_t s, hipEvent_t e0, hipEvent_t e1)
{
    return fd::host::launch(fd::gemm::flat_gemm_direct_kernel<MB, NB, GU, WK, WP>,
                            dim3((unsigned)(pl.tiles * pl.ksplit), (unsigned)pl.mgroups), dim3(WK * 64), 0, s,
                            e0, e1, gp);
}

template <int MB, int KST, int NST>
int launch_dma(const GemmParams &gp, const Plan &pl, hipStream_t s, hipEvent_t e0, hipEvent_t e1)
{
    const size_t lds = (size_t)pl.ring + fd::gemm::gemm_lds_bytes(16 * MB, pl.per);
    return fd::host::launch(fd::gemm::flat_gemm_dma_kernel<MB, KST, NST>,
                            dim3((unsigned)(pl.tiles * pl.ksplit), (unsigned)pl.mgroups), dim3(256), lds, s, e0,
                            e1, gp);
}

template <int MB, int NB, int GU, int WK>
int launch_direct(const GemmParams &gp, const Plan &pl, hipStream_t s, hipEvent_t e0, hipEvent_t e1)
{
    if (pl.packed) return launch_direct_wp<MB, NB, GU, WK, true>(gp, pl, s, e0, e1);
    return launch_direct_wp<MB, NB, GU, WK, false>(gp, pl, s, e0, e1);
}

template <int MB>
int dispatch_variant(const GemmParams &gp, const Plan &pl, hipStream_t s, hipEvent_t e0, hipEvent_t e1)
{
    switch (pl.variant) {
    case 1: return launch_main<MB, 1, 8, 4>(gp, pl, s, e0, e1);
    case 2: return launch_main<MB, 2, 4, 4>(gp, pl, s, e0, e1);
    case 3: return launch_main<MB, 1, 16, 4>(gp, pl, s, e0, e1);
    case 4: return launch_main<MB, 2, 8, 4>(gp, pl, s, e0, e1);
    case 5: return launch_direct<MB, 4, 4, 4>(gp, pl, s, e0, e1);
    case 6: return launch_direct<MB, 2, 8, 4>(gp, pl, s, e0, e1);
    case 7: return launch_direct<MB, 1, 8, 4>(gp, pl, s, e0, e1);
    case 8: return launch_direct<MB, 1, 16, 4>(gp, pl, s, e0, e1);
    case 9: return launch_direct<MB, 1, 8, 8>(gp, pl, s, e0, e1);
    case 10: return launch_direct<MB, 2, 4, 8>(gp, pl, s, e0, e1);
    case 11: return launch_direct<MB, 1, 4, 16>(gp, pl, s, e0, e1);
    case 12: return launch_direct<MB, 1, 8, 16>(gp, pl, s, e0, e1);
    case 13: return launch_dma<MB, 4, 3>(gp, pl, s, e0, e1);
    default: return launch_dma<MB, 4, 2>(gp, pl, s, e0, e1);
    }
}

}  // namespace

extern "C" int fd_flat_gemm_plan(const fd_gemm_desc_t *d, int32_t *variant, int32_t *ksplit,
                                 int32_t *steps_per_slice, int32_t *workgroups)
{
    if (!d) return FD_ERR_NULL;
    Plan pl;
    const int rc = make_plan(d, &pl);
    if (rc != FD_OK) return rc;
    if (variant) *variant = pl.variant;
    if (ksplit) *ksplit = pl.ksplit;
    if (steps_per_slice) *steps_per_slice = pl.per;
    if (workgroups) *workgroups = (int32_t)std::min<int64_t>((int64_t)pl.tiles * pl.ksplit * pl.mgroups, INT32_MAX);
    return FD_OK;
}

extern "C" size_t fd_flat_gemm_workspace_size(const fd_gemm_desc_t *d)
{
    Plan pl;
    if (!d || make_plan(d, &pl) != FD_OK) return 0;
    return pl.ksplit > 1 ? (size_t)pl.ksplit * d->m * d->n * sizeof(float) : 0;
}

extern "C" int fd_flat_gemm(const fd_gemm_desc_t *d, const void *a, const void *w, void *c,
                            hipStream_t stream)
{
    if (!d || !a || !w || !c) return FD_ERR_NULL;
    Plan pl;
    const int rc = make_plan(d, &pl);
    if (rc != FD_OK) return rc;
    if (!fd::host::aligned16(a) || !fd::host::aligned16(w) || !fd::host::aligned16(c)) return FD_ERR_ALIGN;
    const size_t need = pl.ksplit > 1 ? (size_t)pl.ksplit * d->m * d->n * sizeof(float) : 0;
    if (need && (!d->workspace || ((uintptr_t)d->workspace & 255u) || d->workspace_bytes < need))
        return FD_ERR_WORKSPACE;

    GemmParams gp;
    memset(&gp, 0, sizeof gp);
    gp.a = static_cast<const uint16_t *>(a);
    gp.w = static_cast<const uint16_t *>(w);
    gp.c = c;
    gp.part = pl.ksplit > 1 ? static_cast<float *>(d->workspace) : nullptr;
    gp.m = d->m;
    gp.n = d->n;
    gp.k = d->k;
    gp.ksteps = d->k / 32;
    gp.ksplit = pl.ksplit;
    gp.per = pl.per;
    gp.out_bf16 = d->out_dtype == FD_BF16;
    gp.nblk = (d->n + 15) / 16;

    hipEvent_t *ev = d->stage_events;
    hipEvent_t e0 = ev ? ev[0] : nullptr, e1 = ev ? ev[1] : nullptr;
    int lrc;
    switch (pl.mb) {
    case 1: lrc = dispatch_variant<1>(gp, pl, stream, e0, e1); break;
    case 2: lrc = dispatch_variant<2>(gp, pl, stream, e0, e1); break;
    case 3: lrc = dispatch_variant<3>(gp, pl, stream, e0, e1); break;
    default: lrc = dispatch_variant<4>(gp, pl, stream, e0, e1); break;
    }
    if (lrc != FD_OK || pl.ksplit == 1) return lrc;
    const size_t plane = (size_t)d->m * d->n;
    const size_t items = plane % 4 ? plane : plane / 4;
    const unsigned grid = (unsigned)std::min<size_t>((items + 255) / 256, 4096);
    return fd::host::launch(fd::gemm::flat_gemm_reduce_kernel, dim3(grid), dim3(256), 0, stream, nullptr, nullptr,
                            gp);
}

extern "C" size_t fd_flat_gemm_packed_bytes(int32_t n, int32_t k)
{
    if (n < 1 || n > (1 << 20) || k < 32 || k > (1 << 20) || k % 32) return 0;
    return (size_t)((n + 15) / 16) * 16 * k * 2;
}

extern "C" int fd_flat_gemm_pack_weights(int32_t n, int32_t k, const void *w, void *w_packed, hipStream_t stream)
{
    if (!w || !w_packed) return FD_ERR_NULL;
    if (!fd_flat_gemm_packed_bytes(n, k)) return FD_ERR_SHAPE;
    if (!fd::host::aligned16(w) || !fd::host::aligned16(w_packed)) return FD_ERR_ALIGN;
    const size_t nfrag = fd_flat_gemm_packed_bytes(n, k) / 16;
    const unsigned grid = (unsigned)std::min<size_t>((nfrag + 255) / 256, 8192);
    return fd::host::launch(fd::gemm::pack_weights_kernel, dim3(grid), dim3(256), 0, stream, nullptr, nullptr,
                            static_cast<const uint16_t *>(w), static_cast<uint16_t *>(w_packed), (int)n, (int)k,
                            nfrag);
}
