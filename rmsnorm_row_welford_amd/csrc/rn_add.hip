// Element-wise h = a + b (float32 add, rounded to the storage type): the
// first launch of the unfused add-then-RMSNorm comparison that the
// benchmark times against the fused kernel.  16-byte chunks, grid-stride,
// non-temporal hints; a tail (or unaligned buffers) goes element by element.
#include "rn_device.h"
#include "rn_internal.h"

namespace rn {

template <int VEC>
__device__ __forceinline__ void store_sum(float *p, const float *v) {
    if constexpr (VEC == 4) {
        __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, (f32x4 *)p);
    } else {
        *p = v[0];
    }
}
template <int VEC>
__device__ __forceinline__ void store_sum(bf16_bits *p, const float *v) {
    if constexpr (VEC == 8) {
        u32x4 w;
#pragma unroll
        for (int k = 0; k < 4; ++k) w[k] = pack_bf16(v[2 * k], v[2 * k + 1]);
        __builtin_nontemporal_store(w, (u32x4 *)p);
    } else {
        *p = to_bf16(v[0]);
    }
}
template <int VEC>
__device__ __forceinline__ void store_sum(f16_t *p, const float *v) {
    if constexpr (VEC == 8) {
        u32x4 w;
#pragma unroll
        for (int k = 0; k < 4; ++k) w[k] = pack_f16(v[2 * k], v[2 * k + 1]);
        __builtin_nontemporal_store(w, (u32x4 *)p);
    } else {
        *p = (f16_t)v[0];
    }
}

template <class T, int VEC>
__global__ __launch_bounds__(256) void add_kernel(const T *a, const T *b, T *out,
                                                  int64_t nchunks) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nchunks;
         i += stride) {
        float va[VEC], vb[VEC];
        load_chunk<VEC, true>(a + i * VEC, va);
        load_chunk<VEC, true>(b + i * VEC, vb);
#pragma unroll
        for (int k = 0; k < VEC; ++k) va[k] += vb[k];
        store_sum<VEC>(out + i * VEC, va);
    }
}

template <class T>
hipError_t launch_add_t(const void *a, const void *b, void *out, int64_t n,
                        hipStream_t s) {
    constexpr int VEC = Vec16<T>::N;
    const bool vec = ((uintptr_t)a | (uintptr_t)b | (uintptr_t)out) % 16 == 0;
    const int64_t nch = vec ? n / VEC : 0;
    const int64_t done = nch * VEC;
    auto grid = [](int64_t units) {
        int64_t blocks = (units + 255) / 256;
        return (unsigned)(blocks > 65536 ? 65536 : blocks);
    };
    if (nch > 0) {
        hipLaunchKernelGGL((add_kernel<T, VEC>), dim3(grid(nch)), dim3(256), 0, s,
                           (const T *)a, (const T *)b, (T *)out, nch);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (n > done) {
        hipLaunchKernelGGL((add_kernel<T, 1>), dim3(grid(n - done)), dim3(256), 0, s,
                           (const T *)a + done, (const T *)b + done, (T *)out + done,
                           n - done);
        return hipGetLastError();
    }
    return hipSuccess;
}

hipError_t launch_add(int elem, const void *a, const void *b, void *out, int64_t n,
                      hipStream_t s) {
    switch (elem) {
    case 0: return launch_add_t<float>(a, b, out, n, s);
    case 1: return launch_add_t<bf16_bits>(a, b, out, n, s);
    default: return launch_add_t<f16_t>(a, b, out, n, s);
    }
}

}  // namespace rn
