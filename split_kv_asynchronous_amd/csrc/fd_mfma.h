// Matrix-core helpers shared by the grouped-query chunk kernel.
#pragma once

#include "fd_common.h"

namespace fd {

// D = A . B + C on a 16x16x32 bf16 tile: lane l supplies A[l % 16][8(l / 16) + j]
// and B[8(l / 16) + j][l % 16] (j = 0..7) and receives C[4(l / 16) + i][l % 16].
FD_DEV f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
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

}  // namespace fd
