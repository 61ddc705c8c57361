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

// A row's quantization multiplier r = QMAX / a is finite (false only where
// the quotient overflowed: a maximum a below QMAX / FLT_MAX).
__device__ __forceinline__ bool finite_r(float r) { return r <= 3.40282347e38f; }

// Running maximum of |v| as float bits (magnitude bits order like
// magnitudes, NaN above +inf), kept as two maxima of the raw bits so each
// value costs one integer max and no sign masking: the unsigned maximum
// holds the largest negative magnitude (sign bit set) whenever a negative
// value was seen, else the largest positive one; the signed maximum holds
// the largest positive magnitude (negative values are negative integers).
struct AbsMax {
    uint32_t u = 0;
    int32_t i = 0;
    __device__ __forceinline__ void add(float v) {
        const uint32_t b = __float_as_uint(v);
        u = u > b ? u : b;
        i = i > (int32_t)b ? i : (int32_t)b;
    }
    __device__ __forceinline__ uint32_t bits() const {
        const uint32_t n = u & 0x7fffffffu;
        return n > (uint32_t)i ? n : (uint32_t)i;      // i >= 0
    }
};

// Maximum over a 64-lane wavefront (every lane active), returned to every
// lane.  DPP row shifts by 1, 2, 4 and 8 (a lane shifted in from outside its
// row of 16 reads 0, the identity) leave each row's maximum in the row's last
// lane; the four row maxima are read as scalars.  No LDS round trips, unlike
// lane shuffles through ds_bpermute.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    auto umax = [](uint32_t a, uint32_t b) { return a > b ? a : b; };
    // dpp_ctrl row_shr:n = 0x110 + n; all rows and banks; out-of-row lanes take old (0)
    v = umax(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false));
    v = umax(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false));
    v = umax(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false));
    v = umax(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false));
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 15);
    const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 31);
    const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 47);
    const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
    return umax(umax(r0, r1), umax(r2, r3));
}

// Lanes of one wave exchanging data through LDS: orders this lane's earlier
// LDS writes before its later reads of what other lanes wrote (and its reads
// before later writes to the same area).  The hardware keeps a wave's LDS
// operations in order; the wavefront-scope release/acquire pair around a wave
// barrier keeps the compiler from moving a lane's access across the exchange,
// which per-thread alias analysis alone would allow.  No workgroup barrier.
__device__ __forceinline__ void wave_lds_exchange() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace sq
