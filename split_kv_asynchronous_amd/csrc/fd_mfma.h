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

// Two floats -> packed bf16 pair rounded to nearest even (high part) and the
// packed bf16 of the remainders, also rounded to nearest even (low part):
// high + low carries each value to a relative 2^-18.  Two hardware
// conversions (v_cvt_pk_bf16_f32); the remainder a - high is exact in fp32.
FD_DEV void split_pair(float a, float b, uint32_t &hi, uint32_t &lo)
{
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
    hi = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
    const float ra = a - __uint_as_float(hi << 16);
    const float rb = b - __uint_as_float(hi & 0xffff0000u);
    lo = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){ra, rb}, bf16x2));
}

}  // namespace fd
