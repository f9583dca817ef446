// Streaming copy with 16-byte accesses: the bandwidth ceiling, cache flush
// and byte-counter calibration kernel used by the benchmark.
#include "rn_device.h"
#include "rn_internal.h"

namespace rn {

// One 16-byte unit per thread, 1024-thread workgroups over the whole buffer:
// the fastest plain streaming copy measured on MI355X (a persistent
// grid-stride loop reads lower).
__global__ __launch_bounds__(1024) void copy16_kernel(const u32x4 *src,
                                                      u32x4 *dst, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = __builtin_nontemporal_load(src + i);
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
        // up to 2^31 - 1 workgroups of 1024 units: 32 TiB per launch
        const int64_t blocks = (n16 + 1023) / 1024;
        if (blocks > 0x7fffffff) return hipErrorInvalidValue;
        hipLaunchKernelGGL(copy16_kernel, dim3((unsigned)blocks), dim3(1024), 0,
                           s, (const u32x4 *)src, (u32x4 *)dst, n16);
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
