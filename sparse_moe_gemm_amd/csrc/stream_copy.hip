// stream_copy.hip - the library's own streaming copy, for measurement only.
//
// It is not a step of the layer. It states the HBM rate this chip reaches on
// plain streaming traffic, next to the 8 TB/s nominal figure and the layer
// kernels' own rates. The kernel has one grid-stride loop of 16-byte loads and
// stores, with every lane's four loads issued before its stores, and a few
// workgroups per compute unit. A copy of known size also scales the
// rocprofv3 FETCH_SIZE / WRITE_SIZE counters to bytes.
#include "common.hpp"

namespace cmoe {

namespace {

__global__ __launch_bounds__(256) void stream_copy_kernel(const Vec16* __restrict__ src, Vec16* __restrict__ dst,
                                                          int64_t n)
{
    constexpr int U = 4;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + (U - 1) * stride < n; i += U * stride) {
        Vec16 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            v[u] = __builtin_nontemporal_load(&src[i + u * stride]);
#pragma unroll
        for (int u = 0; u < U; ++u)
            __builtin_nontemporal_store(v[u], &dst[i + u * stride]);
    }
    for (; i < n; i += stride)
        dst[i] = src[i];
}

}  // namespace

hipError_t launch_stream_copy(const void* src, void* dst, int64_t bytes, int cus, hipStream_t s)
{
    const int64_t n = bytes / 16;
    if (n <= 0)
        return hipSuccess;
    const int64_t want = (n + 255) / 256;
    const int blocks = (int)std::min<int64_t>(want, (int64_t)cus * 32);
    hipLaunchKernelGGL(stream_copy_kernel, dim3(blocks), dim3(256), 0, s, (const Vec16*)src, (Vec16*)dst, n);
    return hipGetLastError();
}

}  // namespace cmoe
