// Measured ceilings for the benchmark (libsq_probe.so; not part of the
// layer's API): what the matrix cores sustain with the product kernel's
// register pattern on given operand data, and what a plain streaming read of
// HBM reaches.  The benchmark reports them beside the published peaks.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sq_probe.h"

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

// Each wave repeats the product's k-step pattern: 8 weight operands times 2
// activation operands into 16 accumulators of 16 x 16 (v_mfma_i32_16x16x64_i8),
// `iters` times, on operands loaded once from a (weights) and b (activations).
// Workgroups of 8 waves, one per CU and two waves per SIMD as in the product.
__global__ void __launch_bounds__(512)
k_mfma_rate(const int8_t *__restrict__ a, const int8_t *__restrict__ b, int iters,
            int *__restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    v4i wa[8], xb[2];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        wa[j] = *reinterpret_cast<const v4i *>(a + ((wave * 8 + j) * 64 + lane) * 16);
#pragma unroll
    for (int i = 0; i < 2; ++i)
        xb[i] = *reinterpret_cast<const v4i *>(b + ((wave * 2 + i) * 64 + lane) * 16);
    v4i acc[2][8];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = v4i{0, 0, 0, 0};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int i = 0; i < 2; ++i)
                acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wa[j], xb[i], acc[i][j], 0, 0, 0);
    }
    int s = 0;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) s += acc[i][j][0] + acc[i][j][1] + acc[i][j][2] + acc[i][j][3];
    out[(size_t)blockIdx.x * 512 + threadIdx.x] = s;
}

// Grid-stride 16-byte non-temporal loads over the buffer; one xor per
// thread is written so that nothing is dead code.
__global__ void __launch_bounds__(256)
k_stream_read(const v4i *__restrict__ p, int64_t n, int *__restrict__ out) {
    v4i acc = {0, 0, 0, 0};
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        const v4i v = __builtin_nontemporal_load(p + i);
        acc ^= v;
    }
    out[(size_t)blockIdx.x * 256 + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

// The shader clock over a stretch of real time: one lane reads the shader
// cycle counter (s_memtime) and the constant-rate real-time counter
// (s_memrealtime) at its start, sleeps until `ticks` real-time ticks have
// passed (or `max_iter` sleeps, whichever comes first, so the wave always
// ends), and reads both again.  Launched on a second stream just before a run
// of product kernels, it shares a CU with them and sees the clock they run at.
__global__ void __launch_bounds__(64)
k_clock_watch(uint64_t ticks, uint64_t max_iter, uint64_t *__restrict__ out) {
    if (threadIdx.x != 0) return;
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    const uint64_t c0 = __builtin_amdgcn_s_memtime();
    uint64_t r = r0, it = 0;
    while (r - r0 < ticks && it < max_iter) {
        __builtin_amdgcn_s_sleep(8);
        r = __builtin_amdgcn_s_memrealtime();
        ++it;
    }
    const uint64_t c1 = __builtin_amdgcn_s_memtime();
    out[0] = r0;
    out[1] = r;
    out[2] = c0;
    out[3] = c1;
    out[4] = it;
}

}  // namespace

extern "C" {

__attribute__((visibility("default")))
int sqp_wall_clock_khz(int *khz) {
    int dev = 0;
    if (!khz) return 1;
    if (hipGetDevice(&dev) != hipSuccess) return 7;
    return hipDeviceGetAttribute(khz, hipDeviceAttributeWallClockRate, dev) == hipSuccess ? 0 : 7;
}

__attribute__((visibility("default")))
int sqp_clock_watch(uint64_t ticks, uint64_t max_iter, uint64_t *out, void *stream) {
    if (!out || ticks < 1 || max_iter < 1) return 1;
    k_clock_watch<<<dim3(1), dim3(64), 0, (hipStream_t)stream>>>(ticks, max_iter, out);
    return hipGetLastError() == hipSuccess ? 0 : 7;
}

__attribute__((visibility("default")))
int sqp_mfma_rate(const int8_t *a, const int8_t *b, int iters, int blocks, int *out,
                  void *stream) {
    if (!a || !b || !out || iters < 1 || blocks < 1) return 1;
    k_mfma_rate<<<dim3((unsigned)blocks), dim3(512), 0, (hipStream_t)stream>>>(a, b, iters, out);
    return hipGetLastError() == hipSuccess ? 0 : 7;
}

__attribute__((visibility("default")))
int sqp_stream_read(const void *buf, int64_t bytes, int blocks, int *out, void *stream) {
    if (!buf || !out || bytes < 16 || (bytes % 16) != 0 || blocks < 1) return 1;
    k_stream_read<<<dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream>>>(
        static_cast<const v4i *>(buf), bytes / 16, out);
    return hipGetLastError() == hipSuccess ? 0 : 7;
}

}  // extern "C"
