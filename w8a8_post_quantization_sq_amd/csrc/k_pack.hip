// Layout helpers: row-major int8 codes <-> the packed operand order of the
// int8 matrix instruction (16-row x 64-byte fragments, 1 KiB each, lane order
// l = 16 * quarter + row).  One lane per 16-byte chunk of the packed buffer.
#include "sq_device.h"

namespace sq {

__global__ void __launch_bounds__(256)
k_pack_i8(const int8_t *__restrict__ src, int64_t rows, int64_t K, int64_t ld,
          int8_t *__restrict__ dst, int64_t chunks) {
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (c >= chunks) return;
    const int64_t KW = (K + 63) >> 6;
    const int64_t f = c >> 6;
    const int l = (int)(c & 63);
    const int64_t r = (f / KW) * 16 + (l & 15);
    const int64_t k = (f % KW) * 64 + (l >> 4) * 16;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (r < rows && k < K) v = *reinterpret_cast<const uint4 *>(src + r * ld + k);
    *reinterpret_cast<uint4 *>(dst + c * 16) = v;
}

__global__ void __launch_bounds__(256)
k_unpack_i8(const int8_t *__restrict__ src, int64_t rows, int64_t K, int8_t *__restrict__ dst,
            int64_t ld, int64_t chunks) {
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (c >= chunks) return;
    const int64_t KW = (K + 63) >> 6;
    const int64_t f = c >> 6;
    const int l = (int)(c & 63);
    const int64_t r = (f / KW) * 16 + (l & 15);
    const int64_t k = (f % KW) * 64 + (l >> 4) * 16;
    if (r < rows && k < K)
        *reinterpret_cast<uint4 *>(dst + r * ld + k) = *reinterpret_cast<const uint4 *>(src + c * 16);
}

hipError_t launch_pack_i8(const int8_t *src, int64_t rows, int64_t K, int64_t ld, int8_t *dst,
                          hipStream_t st) {
    const int64_t chunks = ((rows + 15) / 16) * ((K + 63) / 64) * 64;
    if (chunks <= 0) return hipSuccess;
    k_pack_i8<<<dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, st>>>(src, rows, K, ld, dst,
                                                                           chunks);
    return hipGetLastError();
}

hipError_t launch_unpack_i8(const int8_t *src, int64_t rows, int64_t K, int8_t *dst, int64_t ld,
                            hipStream_t st) {
    const int64_t chunks = ((rows + 15) / 16) * ((K + 63) / 64) * 64;
    if (chunks <= 0) return hipSuccess;
    k_unpack_i8<<<dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, st>>>(src, rows, K, dst,
                                                                             ld, chunks);
    return hipGetLastError();
}

// Packed int8 codes in [-8, 7] -> the packed 4-bit layout: every lane chunk
// of 16 codes (16 bytes) becomes 8 bytes, byte j of each half holding code j
// of that half's 8 in its low nibble and code j + 4 in its high nibble (two's
// complement).  One thread per chunk; padding stays zero.
__global__ void __launch_bounds__(256)
k_pack4_from8(const int8_t *__restrict__ src, uint8_t *__restrict__ dst, int64_t chunks) {
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (c >= chunks) return;
    const uint4 v = *reinterpret_cast<const uint4 *>(src + c * 16);
    constexpr uint32_t LO = 0x0F0F0F0Fu;
    const uint2 o = make_uint2((v.x & LO) | ((v.y & LO) << 4), (v.z & LO) | ((v.w & LO) << 4));
    *reinterpret_cast<uint2 *>(dst + c * 8) = o;
}

hipError_t launch_pack4_from8(const int8_t *src, int64_t rows, int64_t K, uint8_t *dst,
                              hipStream_t st) {
    const int64_t chunks = (rows + 15) / 16 * ((K + 63) / 64) * 64;
    if (chunks <= 0) return hipSuccess;
    k_pack4_from8<<<dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, st>>>(src, dst, chunks);
    return hipGetLastError();
}

}  // namespace sq
