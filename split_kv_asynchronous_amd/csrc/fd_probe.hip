// Read-ceiling probe (include/fd_probe.h): the decode kernels' K/V load
// patterns with nothing computed, to measure what those patterns can reach.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

#include "fd_host.h"
#include "fd_probe.h"
#include "fd_ring.h"

namespace fd {
namespace probe {

using ring::kStreamPolicy;
using ring::lds_void;

constexpr int kMaxPages = 64;   // pages read per unit (one per lane)

// Ring shapes: W wavefronts, each with NST stages of SB bytes (half K, half V).
template <int W, int NST, int SB>
struct Shape {
    static constexpr int waves = W, nst = NST, stage = SB, part = SB / 2;
    static constexpr int dma = SB / 1024;   // 1 KiB instructions per stage
    static constexpr int lds = W * NST * SB;
    static_assert(part % 1024 == 0, "whole 1 KiB instructions per part");
};
using Shape0 = Shape<4, 2, 8192>;   // grouped bf16 kernel, shape 0
using Shape1 = Shape<4, 3, 8192>;   // grouped bf16 kernel, shape 1
using Shape2 = Shape<2, 3, 4096>;   // the E4M3FN kernel's bytes in flight (2 wavefronts, 3 x 8 KiB shared)

template <typename S, bool PAGED>
__global__ __launch_bounds__(S::waves * 64) void read_kernel(const uint8_t *k, const uint8_t *v,
                                                               const fd_probe_unit_t *units, const uint64_t *pages,
                                                               int page_bytes, uint32_t *sink)
{
    __shared__ __attribute__((aligned(1024))) uint8_t lds[S::lds];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint64_t off = __builtin_amdgcn_readfirstlane((uint32_t)units[blockIdx.x].offset) |
                         (uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(units[blockIdx.x].offset >> 32)) << 32;
    const uint32_t bytes = __builtin_amdgcn_readfirstlane(units[blockIdx.x].bytes);
    uint8_t *ring = lds + wave * S::nst * S::stage;
    // contiguous: buffer ranges ending at the unit's last byte; paged: the
    // unit's pages (offsets of whole pages, lane i holding page i), whole
    // pages read as the paged kernels read them
    __amdgpu_buffer_rsrc_t kr, vr;
    uint32_t npages = 0;
    uint64_t my_page = 0;
    int groups;
    if constexpr (PAGED) {
        npages = min((bytes + page_bytes - 1) / (uint32_t)page_bytes, (uint32_t)kMaxPages);
        if ((uint32_t)lane < npages) my_page = pages[off + lane];
        groups = (int)((npages * (uint64_t)page_bytes + S::part - 1) / S::part);
    } else {
        kr = __builtin_amdgcn_make_buffer_rsrc((void *)(k + off), (short)0, bytes, 0x00020000);
        vr = __builtin_amdgcn_make_buffer_rsrc((void *)(v + off), (short)0, bytes, 0x00020000);
        groups = (int)((bytes + S::part - 1) / S::part);
    }
    const int mine = groups > wave ? (groups - wave + S::waves - 1) / S::waves : 0;   // groups wave, wave + W, ..
    auto issue = [&](int i) {   // this wavefront's i-th group into slot i mod NST
        const uint32_t pos0 = (uint32_t)(wave + S::waves * i) * S::part;
        uint8_t *st = ring + (i % S::nst) * S::stage;
#pragma unroll
        for (int j = 0; j < S::part / 1024; ++j) {
            lds_void *kd = (lds_void *)(st + j * 1024);
            lds_void *vd = (lds_void *)(st + S::part + j * 1024);
            const uint32_t pos = pos0 + j * 1024;
            if constexpr (PAGED) {
                const uint32_t pg = pos / (uint32_t)page_bytes;
                if (pg >= npages) break;   // past the unit's last page (uniform)
                const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)my_page, pg);
                const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(my_page >> 32), pg);
                const size_t a = ((size_t)hi << 32 | lo) + pos % (uint32_t)page_bytes + 16 * lane;
                __builtin_amdgcn_global_load_lds(k + a, kd, 16, 0, kStreamPolicy);
                __builtin_amdgcn_global_load_lds(v + a, vd, 16, 0, kStreamPolicy);
            } else {
                __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, kd, 16, 16 * lane, pos, 0, kStreamPolicy);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, vd, 16, 16 * lane, pos, 0, kStreamPolicy);
            }
        }
    };
    for (int i = 0; i < S::nst - 1 && i < mine; ++i) issue(i);
    for (int i = 0; i < mine; ++i) {
        if (i + S::nst - 1 < mine) issue(i + S::nst - 1);
        // group i has landed once at most the groups issued after it are in
        // flight (a paged group cut short by the unit's last page issues
        // fewer instructions, and the wait may then pass early: nothing reads
        // the stages, so that only shortens the ring at the unit's end)
        ring::wait_ring<S::dma, S::nst - 1>(min(S::nst - 1, mine - 1 - i));
    }
    ring::wait_vmcnt<0>();
    // one word of the ring, read with its wait in the same statement
    uint32_t x;
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(x) : "v"((uint32_t)(uintptr_t)(ring + 4 * lane)) : "memory");
    if (x == 0x9E3779B9u && bytes == 0x9E3779B9u) *sink = x;
}

template <typename S>
int launch(const uint8_t *k, const uint8_t *v, const fd_probe_unit_t *units, int n, const uint64_t *pages,
           int page_bytes, uint32_t *sink, hipStream_t s)
{
    const dim3 grid((unsigned)n), block(S::waves * 64);
    if (pages)
        return fd::host::launch(read_kernel<S, true>, grid, block, 0, s, nullptr, nullptr, k, v, units, pages,
                                page_bytes, sink);
    return fd::host::launch(read_kernel<S, false>, grid, block, 0, s, nullptr, nullptr, k, v, units, pages,
                            page_bytes, sink);
}

}  // namespace probe
}  // namespace fd

extern "C" int fd_probe_read(const void *k, const void *v, const fd_probe_unit_t *units, int32_t num_units,
                             const uint64_t *pages, int32_t page_bytes, int32_t shape, uint32_t *sink,
                             void *stream)
{
    if (!k || !v || !sink || (num_units > 0 && !units)) return FD_ERR_NULL;
    if (num_units < 0 || shape < 0 || shape > 2) return FD_ERR_SHAPE;
    if (pages && (page_bytes < 1024 || page_bytes % 1024 || page_bytes > (1 << 20))) return FD_ERR_SHAPE;
    if (((uintptr_t)k | (uintptr_t)v) & 15) return FD_ERR_ALIGN;
    if (num_units == 0) return FD_OK;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const auto *kb = static_cast<const uint8_t *>(k);
    const auto *vb = static_cast<const uint8_t *>(v);
    if (shape == 1) return fd::probe::launch<fd::probe::Shape1>(kb, vb, units, num_units, pages, page_bytes, sink, s);
    if (shape == 2) return fd::probe::launch<fd::probe::Shape2>(kb, vb, units, num_units, pages, page_bytes, sink, s);
    return fd::probe::launch<fd::probe::Shape0>(kb, vb, units, num_units, pages, page_bytes, sink, s);
}
