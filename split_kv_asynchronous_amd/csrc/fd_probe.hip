// Read-ceiling probe (include/fd_probe.h): the decode kernels' K/V load
// pattern with nothing computed, to measure what that pattern can reach.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

#include "fd_host.h"
#include "fd_probe.h"
#include "fd_ring.h"

namespace fd {
namespace probe {

using ring::kGroupBytes;
using ring::kStreamPolicy;
using ring::lds_void;

constexpr int kWaves = 4;
constexpr int kStage = 2 * kGroupBytes;        // one 4 KiB group of K and one of V
constexpr int kDmaPerStage = 2 * kGroupBytes / 1024;

template <int NST>
__global__ __launch_bounds__(kWaves * 64, NST == 2 ? 2 : 1) void read_kernel(const uint8_t *k, const uint8_t *v,
                                                                                const fd_probe_unit_t *units,
                                                                                uint32_t *sink)
{
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kWaves * NST * kStage];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint64_t off = __builtin_amdgcn_readfirstlane((uint32_t)units[blockIdx.x].offset) |
                         (uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(units[blockIdx.x].offset >> 32)) << 32;
    const uint32_t bytes = __builtin_amdgcn_readfirstlane(units[blockIdx.x].bytes);
    const auto kr = __builtin_amdgcn_make_buffer_rsrc((void *)(k + off), (short)0, bytes, 0x00020000);
    const auto vr = __builtin_amdgcn_make_buffer_rsrc((void *)(v + off), (short)0, bytes, 0x00020000);
    uint8_t *ring = lds + wave * NST * kStage;
    const int groups = (int)((bytes + kGroupBytes - 1) / kGroupBytes);
    const int mine = groups > wave ? (groups - wave + kWaves - 1) / kWaves : 0;   // groups wave, wave + 4, ..
    auto issue = [&](int i) {   // this wavefront's i-th group into slot i mod NST
        const int so = (wave + kWaves * i) * kGroupBytes;
        uint8_t *st = ring + (i % NST) * kStage;
#pragma unroll
        for (int j = 0; j < kGroupBytes / 1024; ++j) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void *)(st + j * 1024), 16, 16 * lane, so + j * 1024,
                                                     0, kStreamPolicy);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void *)(st + kGroupBytes + j * 1024), 16, 16 * lane,
                                                     so + j * 1024, 0, kStreamPolicy);
        }
    };
    for (int i = 0; i < NST - 1 && i < mine; ++i) issue(i);
    for (int i = 0; i < mine; ++i) {
        if (i + NST - 1 < mine) issue(i + NST - 1);
        // group i has landed once at most the groups issued after it are in flight
        ring::wait_ring<kDmaPerStage, NST - 1>(min(NST - 1, mine - 1 - i));
    }
    ring::wait_vmcnt<0>();
    // one word of the ring, read with its wait in the same statement
    uint32_t x;
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(x) : "v"((uint32_t)(uintptr_t)(ring + 4 * lane)) : "memory");
    if (x == 0x9E3779B9u && bytes == 0x9E3779B9u) *sink = x;
}

}  // namespace probe
}  // namespace fd

extern "C" int fd_probe_read(const void *k, const void *v, const fd_probe_unit_t *units, int32_t num_units,
                             int32_t stages, uint32_t *sink, void *stream)
{
    if (!k || !v || !sink || (num_units > 0 && !units)) return FD_ERR_NULL;
    if (num_units < 0 || (stages != 2 && stages != 3)) return FD_ERR_SHAPE;
    if (((uintptr_t)k | (uintptr_t)v) & 15) return FD_ERR_ALIGN;
    if (num_units == 0) return FD_OK;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const auto *kb = static_cast<const uint8_t *>(k);
    const auto *vb = static_cast<const uint8_t *>(v);
    const dim3 grid((unsigned)num_units), block(fd::probe::kWaves * 64);
    if (stages == 2)
        return fd::host::launch(fd::probe::read_kernel<2>, grid, block, 0, s, nullptr, nullptr, kb, vb, units, sink);
    return fd::host::launch(fd::probe::read_kernel<3>, grid, block, 0, s, nullptr, nullptr, kb, vb, units, sink);
}
