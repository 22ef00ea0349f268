// Plain streaming read of a device buffer: the machine's read rate that the
// decode (one pass over its packed K/V cache per call) is measured against.
// Each of the G workgroups of 256 threads reads one contiguous range with
// 16-byte loads, four in flight per thread; each wave writes the XOR of what
// it read to one word of the sink so that no load can be removed.
#include "qkv_internal.hpp"
#include "qkv_measure.h"

namespace qkv {

namespace {

constexpr int kReadThreads = 256;

__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const uint4* __restrict__ p, uint64_t n16,
                                                                    uint64_t per_wg, uint32_t* __restrict__ sink) {
    const uint64_t b = (uint64_t)blockIdx.x * per_wg;
    const uint64_t e = b + per_wg < n16 ? b + per_wg : n16;
    constexpr uint64_t T = kReadThreads;
    uint32_t acc = 0;
    uint64_t i = b + threadIdx.x;
    for (; i + 3 * T < e; i += 4 * T) {
        const uint4 x0 = p[i], x1 = p[i + T], x2 = p[i + 2 * T], x3 = p[i + 3 * T];
        acc ^= x0.x ^ x0.y ^ x0.z ^ x0.w ^ x1.x ^ x1.y ^ x1.z ^ x1.w ^ x2.x ^ x2.y ^ x2.z ^ x2.w ^ x3.x ^ x3.y ^
               x3.z ^ x3.w;
    }
    for (; i < e; i += T) {
        const uint4 x = p[i];
        acc ^= x.x ^ x.y ^ x.z ^ x.w;
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, 64);
    if ((threadIdx.x & 63) == 0) sink[blockIdx.x * (kReadThreads / 64) + (threadIdx.x >> 6)] = acc;
}

// The same read with a configurable shape: blockDim.x threads per workgroup,
// U loads in flight per thread, each W bytes wide (4, 8 or 16).
template <int W> struct Vec;
template <> struct Vec<4> { using T = uint32_t; };
template <> struct Vec<8> { using T = uint2; };
template <> struct Vec<16> { using T = uint4; };

__device__ __forceinline__ uint32_t fold(uint32_t x) { return x; }
__device__ __forceinline__ uint32_t fold(uint2 x) { return x.x ^ x.y; }
__device__ __forceinline__ uint32_t fold(uint4 x) { return x.x ^ x.y ^ x.z ^ x.w; }

template <int W, int U>
__global__ __launch_bounds__(1024) void stream_read_config_kernel(const void* __restrict__ buf, uint64_t n,
                                                                   uint64_t per_wg, uint32_t* __restrict__ sink) {
    using V = typename Vec<W>::T;
    const V* p = (const V*)buf;
    const uint64_t T = blockDim.x;
    const uint64_t b = (uint64_t)blockIdx.x * per_wg;
    const uint64_t e = b + per_wg < n ? b + per_wg : n;
    uint32_t acc = 0;
    uint64_t i = b + threadIdx.x;
    for (; i + (U - 1) * T < e; i += U * T) {
        V x[U];
#pragma unroll
        for (int u = 0; u < U; ++u) x[u] = p[i + u * T];
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= fold(x[u]);
    }
    for (; i < e; i += T) acc ^= fold(p[i]);
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, 64);
    if ((threadIdx.x & 63) == 0) sink[blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6)] = acc;
}

template <int W>
hipError_t launch_cfg(const void* buf, size_t bytes, int wgs, int threads, int u, uint32_t* sink,
                      hipStream_t stream) {
    const uint64_t n = bytes / W;
    const uint64_t per = (n + (uint64_t)wgs - 1) / (uint64_t)wgs;
    const dim3 g((unsigned)wgs), b((unsigned)threads);
    switch (u) {
        case 1: hipLaunchKernelGGL((stream_read_config_kernel<W, 1>), g, b, 0, stream, buf, n, per, sink); break;
        case 2: hipLaunchKernelGGL((stream_read_config_kernel<W, 2>), g, b, 0, stream, buf, n, per, sink); break;
        case 4: hipLaunchKernelGGL((stream_read_config_kernel<W, 4>), g, b, 0, stream, buf, n, per, sink); break;
        case 8: hipLaunchKernelGGL((stream_read_config_kernel<W, 8>), g, b, 0, stream, buf, n, per, sink); break;
        case 16: hipLaunchKernelGGL((stream_read_config_kernel<W, 16>), g, b, 0, stream, buf, n, per, sink); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_measure_read_config(const void* buf, size_t bytes, int workgroups, int threads, int in_flight,
                                      int width, uint32_t* sink, hipStream_t stream) {
    switch (width) {
        case 4: return launch_cfg<4>(buf, bytes, workgroups, threads, in_flight, sink, stream);
        case 8: return launch_cfg<8>(buf, bytes, workgroups, threads, in_flight, sink, stream);
        case 16: return launch_cfg<16>(buf, bytes, workgroups, threads, in_flight, sink, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_measure_read(const void* buf, size_t bytes, int workgroups, uint32_t* sink,
                               hipStream_t stream) {
    const uint64_t n16 = bytes / 16;
    const uint64_t per = (n16 + (uint64_t)workgroups - 1) / (uint64_t)workgroups;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)workgroups), dim3(kReadThreads), 0, stream,
                       (const uint4*)buf, n16, per, sink);
    return hipGetLastError();
}

}  // namespace qkv
