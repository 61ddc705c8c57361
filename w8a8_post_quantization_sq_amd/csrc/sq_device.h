// Device helpers shared by the kernel sources (not by the host layer).
#pragma once

#include "sq_internal.h"

namespace sq {

// ---- device helpers --------------------------------------------------------

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

// Exact binary16 -> binary32 (v_cvt_f32_f16).
__device__ __forceinline__ float h2f(uint32_t bits16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// binary32 -> binary16 bits, round to nearest even (v_cvt_f16_f32 in the
// default rounding mode; never the packed round-toward-zero form).
__device__ __forceinline__ uint16_t f2h_bits(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// Maximum over a 64-lane wavefront.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        uint32_t t = (uint32_t)__shfl_xor((int)v, o, 64);
        v = v > t ? v : t;
    }
    return v;
}

}  // namespace sq
