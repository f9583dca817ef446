// Streaming copy with 16-byte accesses: the bandwidth ceiling, cache flush
// and byte-counter calibration kernel used by the benchmark.
#include "rn_device.h"
#include "rn_internal.h"

namespace rn {

// UNITS 16-byte units per thread (a workgroup's units are contiguous, each
// step of its threads one coalesced block), THREADS-thread workgroups over
// the whole buffer, non-temporal loads and stores.
#ifndef RN_COPY_UNITS
#define RN_COPY_UNITS 1
#endif
#ifndef RN_COPY_THREADS
#define RN_COPY_THREADS 1024
#endif
template <int UNITS, int THREADS>
__global__ __launch_bounds__(THREADS) void copy16_kernel(const u32x4 *src, u32x4 *dst,
                                                         int64_t n) {
    const int64_t base = (int64_t)blockIdx.x * (THREADS * UNITS) + threadIdx.x;
    u32x4 v[UNITS];
#pragma unroll
    for (int k = 0; k < UNITS; ++k)
        if (base + k * THREADS < n) v[k] = __builtin_nontemporal_load(src + base + k * THREADS);
#pragma unroll
    for (int k = 0; k < UNITS; ++k)
        if (base + k * THREADS < n) __builtin_nontemporal_store(v[k], dst + base + k * THREADS);
}

__global__ __launch_bounds__(256) void copy1_kernel(const uint8_t *src,
                                                    uint8_t *dst, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += stride)
        dst[i] = src[i];
}

hipError_t launch_copy(const void *src, void *dst, size_t bytes,
                       hipStream_t s) {
    const bool vec = ((uintptr_t)src % 16 == 0) && ((uintptr_t)dst % 16 == 0);
    const int64_t n16 = vec ? (int64_t)(bytes / 16) : 0;
    const int64_t tail = (int64_t)bytes - n16 * 16;
    if (n16 > 0) {
        constexpr int per = RN_COPY_THREADS * RN_COPY_UNITS;
        const int64_t blocks = (n16 + per - 1) / per;
        if (blocks > 0x7fffffff) return hipErrorInvalidValue;
        hipLaunchKernelGGL((copy16_kernel<RN_COPY_UNITS, RN_COPY_THREADS>),
                           dim3((unsigned)blocks), dim3(RN_COPY_THREADS), 0, s,
                           (const u32x4 *)src, (u32x4 *)dst, n16);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (tail > 0) {
        int64_t blocks = (tail + 255) / 256;
        if (blocks > 65536) blocks = 65536;
        hipLaunchKernelGGL(copy1_kernel, dim3((unsigned)blocks), dim3(256), 0,
                           s, (const uint8_t *)src + n16 * 16,
                           (uint8_t *)dst + n16 * 16, tail);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace rn
