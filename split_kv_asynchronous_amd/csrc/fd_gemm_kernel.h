// Flat GEMM of the decode linear layers: C[M][N] = A[M][K] . W[N][K]^T with M
// small (FlashDecoding++ theory page, section 2, the second bottleneck:
// libraries pad the flat M up to their tile and waste most of the work;
// section 4: minimal padding plus double buffering, the loads of the next
// tile overlapping the products of the current one).
//
// C^T = W . A^T on v_mfma_f32_16x16x32_bf16: the weights are the A operand
// (16 rows of W per block), the activations the B operand, so M is padded
// only to a multiple of 16 (MB blocks of 16 rows).  A workgroup of WAVES
// wavefronts owns WAVES * NB * 16 output columns over one slice of K; the
// slice of A is staged once in LDS (rows padded by 16 bytes, so that the 16
// rows one fragment read touches fall in distinct banks).  The weight
// fragments stream from memory straight into registers in batches of GU
// k-steps, two batches alternating: the loads of one batch are issued before
// the products of the other.  With K split over several workgroups each
// writes fp32 partials and a reduce kernel sums them in slice order.
#pragma once

#include "fd_common.h"
#include "fd_mfma.h"
#include "fd_ring.h"

namespace fd {
namespace gemm {

constexpr int kGemmMaxRows = 64;   // rows of A per m-group (grid dimension y)

struct GemmParams {
    const uint16_t *a;      // [M][K] bf16
    const uint16_t *w;      // [N][K] bf16
    void *c;                // [M][N] f32 or bf16
    float *part;            // [ksplit][M][N] fp32 partials when ksplit > 1
    int m, n, k;
    int ksteps;             // K / 32
    int ksplit;             // K slices
    int per;                // k-steps per slice (the last slice may be shorter)
    int out_bf16;
    int nblk;               // 16-row blocks of a packed W (ceil(N / 16))
};

FD_DEV uint32_t gemm_pack_bf16(float a, float b)
{
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

// Stores C[mg0 + mr][col .. col + 3] (or its slice partial), col = cb + c,
// dropping a row past the m-group and columns past N.  Rows of C are 16-byte
// aligned when N % 4 == 0 (vector stores); otherwise element by element.
FD_DEV void store_quad(const GemmParams &p, int slice, int mg0, int mrows, int mr, int cb, int c, f32x4 v)
{
    const int col = cb + c;
    if (mr >= mrows || col >= p.n) return;
    const size_t at = (size_t)(mg0 + mr) * p.n + col;
    const bool vec = (p.n & 3) == 0;
    if (p.ksplit > 1) {
        float *dst = p.part + (size_t)slice * p.m * p.n + at;
        if (vec) {
            *reinterpret_cast<f32x4 *>(dst) = v;
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (col + i < p.n) dst[i] = v[i];
        }
    } else if (p.out_bf16) {
        uint16_t *dst = static_cast<uint16_t *>(p.c) + at;
        const u32x2 h = u32x2{gemm_pack_bf16(v[0], v[1]), gemm_pack_bf16(v[2], v[3])};
        if (vec) {
            *reinterpret_cast<u32x2 *>(dst) = h;
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (col + i < p.n) dst[i] = (uint16_t)(h[i >> 1] >> (16 * (i & 1)));
        }
    } else {
        float *dst = static_cast<float *>(p.c) + at;
        if (vec) {
            *reinterpret_cast<f32x4 *>(dst) = v;
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (col + i < p.n) dst[i] = v[i];
        }
    }
}

// Bytes of LDS a workgroup needs for `rows` rows of A and `per` k-steps.
__host__ __device__ inline size_t gemm_lds_bytes(int rows, int per) { return (size_t)rows * (64 * per + 16); }

// Grid: x = tiles * ksplit (unit = tile * ksplit + slice), y = m-groups of 64
// rows.  Requires K % 32 == 0 and 16-byte aligned A, W and C.
template <int MB, int NB, int GU, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void flat_gemm_kernel(GemmParams p)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds_a[];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int n = lane & 15;
    const int g4 = lane >> 4;

    const int tile = blockIdx.x / p.ksplit;
    const int slice = blockIdx.x - tile * p.ksplit;
    const int mg0 = blockIdx.y * kGemmMaxRows;             // first row of A of this m-group
    const int mrows = min(kGemmMaxRows, p.m - mg0);        // 1 .. 64, at most 16 * MB
    const int s_begin = slice * p.per;
    const int nst = min(p.per, p.ksteps - s_begin);        // k-steps of this slice, >= 1
    const int kbase = 32 * s_begin;
    const int stride = 64 * nst + 16;                      // bytes per LDS row of A

    // this wavefront's NB blocks of 16 output columns; a row of W past N is
    // clamped onto the last one (loads stay in bounds, its sums are not stored)
    const int col0 = (tile * WAVES + wave) * NB * 16;
    const uint16_t *wrow[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
        wrow[nb] = p.w + (size_t)min(col0 + 16 * nb + n, p.n - 1) * p.k + kbase + 8 * g4;

    typedef u32x4 Batch[GU][NB];
    auto load = [&](Batch &buf, int j0) {
#pragma unroll
        for (int u = 0; u < GU; ++u)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                buf[u][nb] = *reinterpret_cast<const u32x4 *>(wrow[nb] + 32 * (j0 + u));
    };

    const int nbatch = nst / GU;
    Batch b0, b1;
    if (nbatch > 0) load(b0, 0);                           // in flight while A is staged

    // ---- A[mg0 .. mg0 + 16MB)[kbase .. kbase + 32 nst) into LDS; rows past M are zero
    {
        const int cpr = 4 * nst;                           // 16-byte chunks per row
        const uint16_t *abase = p.a + (size_t)mg0 * p.k + kbase;
        for (int i = threadIdx.x; i < 16 * MB * cpr; i += WAVES * 64) {
            const int r = i / cpr, c = i - r * cpr;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (r < mrows) v = *reinterpret_cast<const u32x4 *>(abase + (size_t)r * p.k + 8 * c);
            *reinterpret_cast<u32x4 *>(lds_a + r * stride + 16 * c) = v;
        }
    }
    __syncthreads();
    if (col0 >= p.n) return;                               // a wavefront wholly past N (no barrier follows)

    f32x4 acc[MB][NB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

    // k-step j: W fragment of block nb = row n, components 32j + 8g4 .. +7;
    // A^T fragment of block mb = LDS row 16mb + n, the same components
    const uint8_t *lrow = lds_a + n * stride + 16 * g4;
    auto step = [&](const u32x4 (&wf)[NB], int j) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const u32x4 af = *reinterpret_cast<const u32x4 *>(lrow + 16 * mb * stride + 64 * j);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = mfma_bf16(wf[nb], af, acc[mb][nb]);
        }
    };
    auto compute = [&](const Batch &buf, int j0) {
#pragma unroll
        for (int u = 0; u < GU; ++u) step(buf[u], j0 + u);
    };

    // Batch i is in flight in b0 at the top of each iteration.  The loads are
    // unconditional inside the loop (three or more batches left), so the
    // outstanding-load count is the same on every path into the products and
    // the waits before them cover only the batch they use; the scheduling
    // barriers keep each batch's loads ahead of the other batch's products.
    int i = 0;
#pragma unroll 1
    for (; i + 2 < nbatch; i += 2) {
        load(b1, (i + 1) * GU);
        __builtin_amdgcn_sched_barrier(0);
        compute(b0, i * GU);
        load(b0, (i + 2) * GU);
        __builtin_amdgcn_sched_barrier(0);
        compute(b1, (i + 1) * GU);
    }
    if (i + 1 < nbatch) {                                  // two batches left
        load(b1, (i + 1) * GU);
        __builtin_amdgcn_sched_barrier(0);
        compute(b0, i * GU);
        compute(b1, (i + 1) * GU);
    } else if (i < nbatch) {                               // one batch left
        compute(b0, i * GU);
    }
#pragma unroll 1
    for (int j = nbatch * GU; j < nst; ++j) {              // the k-steps short of a batch
        u32x4 wf[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) wf[nb] = *reinterpret_cast<const u32x4 *>(wrow[nb] + 32 * j);
        step(wf, j);
    }

    // ---- lane (n, g4) holds C[mg0 + 16mb + n][col0 + 16nb + 4g4 + i], i = 0..3
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) store_quad(p, slice, mg0, mrows, 16 * mb + n, col0 + 16 * nb, 4 * g4, acc[mb][nb]);
}

// Variant without LDS staging: the WK wavefronts of a workgroup share one
// block of NB * 16 output columns and take consecutive parts of the
// workgroup's K slice; each loads both operands straight into registers (the
// activation fragments are small and stay in L2), in double-buffered batches
// as above, and the WK partial sums are added through LDS at the end, in
// wavefront order.  With many wavefronts per workgroup a small layer has all
// of its weights in flight at once.  Grid as above with tiles of NB * 16
// columns.
//
// WP: W in the packed (fragment-major) layout of pack_weights_kernel, so one
// load instruction reads 1 KiB of consecutive bytes -- whole cache lines --
// instead of 64 bytes of each of 16 rows, and is marked non-temporal.
template <int MB, int NB, int GU0, int WK, bool WP>
__global__ __launch_bounds__(WK * 64) void flat_gemm_direct_kernel(GemmParams p)
{
    // load batches sized to the register file: 4 wavefronts per SIMD leave
    // 128 registers, fewer leave more
    constexpr int kFrag = WK >= 16 ? (MB >= 3 ? 10 : 12) : 24;
    constexpr int GU = GU0 * (NB + MB) <= kFrag ? GU0 : (kFrag / (NB + MB) > 0 ? kFrag / (NB + MB) : 1);
    __shared__ f32x4 red[WK - 1][MB][NB][64];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int n = lane & 15;
    const int g4 = lane >> 4;

    const int tile = blockIdx.x / p.ksplit;
    const int slice = blockIdx.x - tile * p.ksplit;
    const int mg0 = blockIdx.y * kGemmMaxRows;
    const int mrows = min(kGemmMaxRows, p.m - mg0);
    const int s_begin = slice * p.per;
    const int nst_wg = min(p.per, p.ksteps - s_begin);
    const int q = (nst_wg + WK - 1) / WK;                  // k-steps per wavefront
    const int w_begin = min(wave * q, nst_wg);
    const int nst = min(q, nst_wg - w_begin);              // this wavefront's k-steps, may be 0
    const int kbase = 32 * (s_begin + w_begin);

    const int col0 = tile * NB * 16;
    // elements between a lane's weight fragments of consecutive k-steps
    constexpr int WSTEP = WP ? 512 : 32;
    const uint16_t *wrow[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        if constexpr (WP)
            wrow[nb] = p.w + ((size_t)min(col0 / 16 + nb, p.nblk - 1) * p.ksteps + s_begin + w_begin) * 512 + 8 * lane;
        else
            wrow[nb] = p.w + (size_t)min(col0 + 16 * nb + n, p.n - 1) * p.k + kbase + 8 * g4;
    }
    auto wload = [](const uint16_t *ptr) {
        if constexpr (WP)
            return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(ptr));
        else
            return *reinterpret_cast<const u32x4 *>(ptr);
    };
    // rows past the m-group read its last row (their sums are not stored)
    const uint16_t *arow[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
        arow[mb] = p.a + (size_t)(mg0 + min(16 * mb + n, mrows - 1)) * p.k + kbase + 8 * g4;

    struct Batch {
        u32x4 w[GU][NB];
        u32x4 a[GU][MB];
    };
    auto load = [&](Batch &buf, int j0) {
#pragma unroll
        for (int u = 0; u < GU; ++u) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                buf.w[u][nb] = wload(wrow[nb] + WSTEP * (j0 + u));
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                buf.a[u][mb] = *reinterpret_cast<const u32x4 *>(arow[mb] + 32 * (j0 + u));
        }
    };

    f32x4 acc[MB][NB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto step = [&](const u32x4 (&wf)[NB], const u32x4 (&af)[MB]) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = mfma_bf16(wf[nb], af[mb], acc[mb][nb]);
    };
    auto compute = [&](const Batch &buf) {
#pragma unroll
        for (int u = 0; u < GU; ++u) step(buf.w[u], buf.a[u]);
    };

    const int nbatch = nst / GU;
    Batch b0, b1;
    if (nbatch > 0) load(b0, 0);
    int i = 0;
#pragma unroll 1
    for (; i + 2 < nbatch; i += 2) {
        load(b1, (i + 1) * GU);
        __builtin_amdgcn_sched_barrier(0);
        compute(b0);
        load(b0, (i + 2) * GU);
        __builtin_amdgcn_sched_barrier(0);
        compute(b1);
    }
    if (i + 1 < nbatch) {
        load(b1, (i + 1) * GU);
        __builtin_amdgcn_sched_barrier(0);
        compute(b0);
        compute(b1);
    } else if (i < nbatch) {
        compute(b0);
    }
#pragma unroll 1
    for (int j = nbatch * GU; j < nst; ++j) {
        u32x4 wf[NB], af[MB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) wf[nb] = wload(wrow[nb] + WSTEP * j);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) af[mb] = *reinterpret_cast<const u32x4 *>(arow[mb] + 32 * j);
        step(wf, af);
    }

    // ---- wavefronts 1..WK-1 hand their sums to wavefront 0, which adds them in order and stores
    if (wave > 0) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) red[wave - 1][mb][nb][lane] = acc[mb][nb];
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            f32x4 v = acc[mb][nb];
#pragma unroll
            for (int w = 0; w < WK - 1; ++w) v += red[w][mb][nb][lane];
            store_quad(p, slice, mg0, mrows, 16 * mb + n, col0 + 16 * nb, 4 * g4, v);
        }
}

// Variant with the weights moved by DMA into LDS.  Each weight-load
// instruction of the register variants touches 16 rows x 64 bytes (16 cache
// lines, half of each); here one buffer->LDS instruction moves 1 KiB of
// 16 / KST whole rows' pieces (KST k-steps of a row are 64 * KST contiguous
// bytes), so the vector memory path handles half as many lines per byte.
// Each wavefront owns a ring of NST stages of 16 weight rows x KST k-steps;
// piece j of ring row r sits in slot (j + rot(r)) mod 4KST, so the fragment
// reads (one piece from each of 16 rows) are free of bank conflicts.  A is
// staged in LDS as in the first variant and shared by the 4 wavefronts (4
// column blocks of 16).  Requires K slices that are whole stages.
template <int MB, int KST, int NST>
__global__ __launch_bounds__(256, 2) void flat_gemm_dma_kernel(GemmParams p)
{
    constexpr int PPR = 4 * KST;                           // 16-byte pieces per ring row
    constexpr int RPI = 16 / KST;                          // ring rows per 1 KiB instruction
    constexpr int ROWB = 64 * KST;                         // bytes per ring row
    constexpr int STAGE = 16 * ROWB;                       // bytes per stage
    constexpr int NF = KST * (1 + MB);                     // fragments read per stage
    static_assert(NF % 4 == 0, "fragment reads come in fours");
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15;
    const int g4 = lane >> 4;

    const int tile = blockIdx.x / p.ksplit;
    const int slice = blockIdx.x - tile * p.ksplit;
    const int mg0 = blockIdx.y * kGemmMaxRows;
    const int mrows = min(kGemmMaxRows, p.m - mg0);
    const int s_begin = slice * p.per;
    const int nst = min(p.per, p.ksteps - s_begin);        // a multiple of KST
    const int nstage = nst / KST;
    const int kbase = 32 * s_begin;
    const int stride = 64 * nst + 16;

    uint8_t *ring = lds + wave * (NST * STAGE);
    uint8_t *alds = lds + 4 * NST * STAGE;
    const int col0 = (tile * 4 + wave) * 16;
    const bool live = col0 < p.n;

    // buffer resource over this wavefront's 16 weight rows (rows past N read
    // the last row); lane l of instruction i fetches, of ring row
    // RPI * i + l / PPR, the piece that belongs in slot l % PPR
    const size_t rowbytes = (size_t)p.k * 2;
    const int rowc0 = min(col0, p.n - 1);
    const int nrows = min(16, p.n - rowc0);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(p.w + (size_t)rowc0 * p.k), (short)0, (int)(nrows * rowbytes), 0x00020000);
    uint32_t voff[KST];
#pragma unroll
    for (int i = 0; i < KST; ++i) {
        const int r = RPI * i + lane / PPR;
        const int piece = (lane % PPR - ring::Fmt<FD_BF16>::rot(r)) & (PPR - 1);
        voff[i] = (uint32_t)((min(col0 + r, p.n - 1) - rowc0) * rowbytes + 16 * piece);
    }
    auto issue = [&](int st, int slot) {
        uint8_t *dst = ring + slot * STAGE;
        const int so = 2 * (kbase + 32 * KST * st);
#pragma unroll
        for (int i = 0; i < KST; ++i) {
            // (the LDS pointer as a named local: written inline as a cast in
            // the call, the host compilation pass drops the kernel's stub)
            const uint32_t vo = voff[i];
            ring::lds_void *d = (ring::lds_void *)(dst + 1024 * i);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, d, 16, vo, so, 0, ring::kStreamPolicy);
        }
    };
    if (live) {
#pragma unroll
        for (int k = 0; k < NST; ++k)
            if (k < nstage) issue(k, k);
    }

    // ---- A[mg0 .. mg0 + 16MB)[kbase .. kbase + 32 nst) into LDS; rows past M are zero
    {
        const int cpr = 4 * nst;
        const uint16_t *abase = p.a + (size_t)mg0 * p.k + kbase;
        for (int i = threadIdx.x; i < 16 * MB * cpr; i += 256) {
            const int r = i / cpr, c = i - r * cpr;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (r < mrows) v = *reinterpret_cast<const u32x4 *>(abase + (size_t)r * p.k + 8 * c);
            *reinterpret_cast<u32x4 *>(alds + r * stride + 16 * c) = v;
        }
    }
    __syncthreads();
    if (!live) return;                                     // no barrier follows

    // fragment addresses: W of k-step kk = ring row n, piece 4kk + g4;
    // A^T of block mb, k-step j = LDS row 16mb + n, bytes 64j + 16g4
    uint32_t wrd[KST];
#pragma unroll
    for (int kk = 0; kk < KST; ++kk)
        wrd[kk] = n * ROWB + 16 * ((4 * kk + g4 + ring::Fmt<FD_BF16>::rot(n)) & (PPR - 1));
    const uint32_t ard = (uint32_t)(uintptr_t)alds + n * stride + 16 * g4;

    f32x4 acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
    int slot = 0;
#pragma unroll 1
    for (int st = 0; st < nstage; ++st) {
        // this stage's DMAs done; up to NST - 1 later stages stay in flight
        const int ahead = min(NST - 1, nstage - 1 - st);
        ring::wait_ring<KST, NST - 1>(ahead);
        const uint32_t sb = (uint32_t)(uintptr_t)(ring + slot * STAGE);
        uint32_t addr[NF];
#pragma unroll
        for (int kk = 0; kk < KST; ++kk) {
            addr[kk] = sb + wrd[kk];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                addr[KST + kk * MB + mb] = ard + 16 * mb * stride + 64 * (KST * st + kk);
        }
        u32x4 f[NF];
#pragma unroll
        for (int c = 0; c + 8 <= NF; c += 8) {
            uint32_t a8[8];
            u32x4 o8[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) a8[u] = addr[c + u];
            ring::lds_read8(a8, o8);
#pragma unroll
            for (int u = 0; u < 8; ++u) f[c + u] = o8[u];
        }
        if constexpr (NF % 8) {
            uint32_t a4[4];
            u32x4 o4[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) a4[u] = addr[NF - 4 + u];
            ring::lds_read4(a4, o4);
#pragma unroll
            for (int u = 0; u < 4; ++u) f[NF - 4 + u] = o4[u];
        }
        // the stage is read out: hand it back to the DMA engine, then multiply
        if (st + NST < nstage) issue(st + NST, slot);
        slot = slot + 1 == NST ? 0 : slot + 1;
#pragma unroll
        for (int kk = 0; kk < KST; ++kk)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) acc[mb] = mfma_bf16(f[kk], f[KST + kk * MB + mb], acc[mb]);
    }

#pragma unroll
    for (int mb = 0; mb < MB; ++mb) store_quad(p, slice, mg0, mrows, 16 * mb + n, col0, 4 * g4, acc[mb]);
}

// The packed (fragment-major) weight layout: W[N][K] as ceil(N/16) blocks of
// 16 rows, each as K/32 k-steps of 1 KiB, each holding the 64 lanes'
// 16-byte operand fragments in lane order -- lane l gets row 16cb + l % 16,
// components 32j + 8(l / 16) .. +7, the A-operand layout of
// v_mfma_f32_16x16x32_bf16.  Rows past N are zero.  One thread per fragment.
__global__ __launch_bounds__(256) void pack_weights_kernel(const uint16_t *w, uint16_t *wp, int n, int k,
                                                           size_t nfrag)
{
    const int ksteps = k / 32;
    for (size_t f = (size_t)blockIdx.x * 256 + threadIdx.x; f < nfrag; f += (size_t)gridDim.x * 256) {
        const int l = (int)(f & 63);
        const size_t rest = f >> 6;
        const int j = (int)(rest % ksteps);
        const size_t cb = rest / ksteps;
        const size_t row = 16 * cb + (l & 15);
        u32x4 v = {0u, 0u, 0u, 0u};
        if (row < (size_t)n) v = *reinterpret_cast<const u32x4 *>(w + row * k + 32 * j + 8 * (l >> 4));
        *reinterpret_cast<u32x4 *>(wp + 8 * f) = v;
    }
}

// C = sum over slices of the partials, in slice order: 4 outputs per thread
// when M * N % 4 == 0 (every plane then 16-byte aligned), else one.  The
// loads of up to 8 slices are issued together before they are added.
__global__ __launch_bounds__(256) void flat_gemm_reduce_kernel(GemmParams p)
{
    const size_t plane = (size_t)p.m * p.n;
    const size_t stride = (size_t)gridDim.x * 256;
    if ((plane & 3) == 0) {
        for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < plane / 4; i += stride) {
            const float *src = p.part + 4 * i;
            f32x4 s = *reinterpret_cast<const f32x4 *>(src);
            int sl = 1;
            for (; sl + 8 <= p.ksplit; sl += 8) {
                f32x4 v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const f32x4 *>(src + (sl + u) * plane);
#pragma unroll
                for (int u = 0; u < 8; ++u) s += v[u];
            }
            if (p.ksplit - sl >= 4) {
                f32x4 v[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const f32x4 *>(src + (sl + u) * plane);
#pragma unroll
                for (int u = 0; u < 4; ++u) s += v[u];
                sl += 4;
            }
            for (; sl < p.ksplit; ++sl) s += *reinterpret_cast<const f32x4 *>(src + sl * plane);
            if (p.out_bf16)
                *reinterpret_cast<u32x2 *>(static_cast<uint16_t *>(p.c) + 4 * i) =
                    u32x2{gemm_pack_bf16(s[0], s[1]), gemm_pack_bf16(s[2], s[3])};
            else
                *reinterpret_cast<f32x4 *>(static_cast<float *>(p.c) + 4 * i) = s;
        }
    } else {
        for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < plane; i += stride) {
            float s = p.part[i];
            for (int sl = 1; sl < p.ksplit; ++sl) s += p.part[sl * plane + i];
            if (p.out_bf16)
                static_cast<uint16_t *>(p.c)[i] = (uint16_t)gemm_pack_bf16(s, 0.f);
            else
                static_cast<float *>(p.c)[i] = s;
        }
    }
}

}  // namespace gemm
}  // namespace fd
